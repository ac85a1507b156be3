"""Convenience wrapper: moves synthetic inputs to the GPU and runs rounds
through the C ABI (allocation and marshalling only)."""
import numpy as np

from . import _lib


def to_device(inputs, device="cuda"):
    import torch
    out = {}
    for k, v in inputs["weights"].items():
        a = np.ascontiguousarray(v)
        t = torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a)
        out[k] = t.to(device)
    H = torch.from_numpy(np.ascontiguousarray(inputs["H"], dtype=np.float32)).to(device)
    root = torch.from_numpy(np.ascontiguousarray(inputs["root"], dtype=np.int32)).to(device)
    return out, H, root


class Round:
    """One context + output buffers for a fixed (batch, params)."""

    def __init__(self, dev_weights, wtype, caps, batch, D, M, K, W, B, beta, device=0,
                 scoring="conditional", builder="depthwise"):
        import torch
        self.p = _lib.params(D, M, K, W, B, beta)
        self.batch = batch
        self.ctx = _lib.dtree_create(dev_weights, wtype, caps, device)
        if scoring != "conditional":
            _lib.dtree_set_scoring(self.ctx, scoring)
        self.builder = builder
        if builder != "depthwise":
            _lib.dtree_set_builder(self.ctx, builder)
        self.weights = dev_weights   # keep the borrowed weights alive
        N = B + 1
        dev = f"cuda:{device}"
        self.tok = torch.empty((batch, N), dtype=torch.int32, device=dev)
        self.parent = torch.empty_like(self.tok)
        self.depth = torch.empty_like(self.tok)
        self.score = torch.empty((batch, N), dtype=torch.float32, device=dev)
        self.mask = torch.empty((batch, N, N), dtype=torch.uint8, device=dev)
        self.n_nodes = torch.empty((batch,), dtype=torch.int32, device=dev)

    def run(self, H, root, stream=None):
        _lib.dtree_build_round(self.ctx, self.p, self.batch, H, root, self.tok, self.parent,
                               self.depth, self.score, self.mask, self.n_nodes, stream)

    def outputs(self):
        return [dict(tok=self.tok[q].cpu().numpy(), parent=self.parent[q].cpu().numpy(),
                     depth=self.depth[q].cpu().numpy(), score=self.score[q].cpu().numpy(),
                     mask=self.mask[q].cpu().numpy(), n_nodes=int(self.n_nodes[q]))
                for q in range(self.batch)]

    def trace(self, req):
        n = (_lib.dtree_heap_nodes(self.p) if self.builder == "heap"
             else _lib.dtree_superarbol_nodes(self.p))
        return _lib.dtree_get_trace(self.ctx, req, self.p, n)

    def close(self):
        if self.ctx is not None:
            _lib.dtree_destroy(self.ctx)
            self.ctx = None


class TreeAttention:
    """Device buffers for tree-attention calls of one shape: Q, K, V (raw
    bf16 bits as numpy uint16 or device tensors), per-request lengths, the
    mask (numpy or a round's device mask), the output and the workspace."""

    def __init__(self, Q, K, V, prefix_len, n_nodes, mask, scale, splits=0, device="cuda"):
        import torch

        def dev(a, dtype=None):
            if isinstance(a, torch.Tensor):
                return a.to(device).contiguous()
            a = np.ascontiguousarray(a)
            if a.dtype == np.uint16:
                a = a.view(np.int16)
            t = torch.from_numpy(a if dtype is None else a.astype(dtype))
            return t.to(device)

        self.Q, self.K, self.V = dev(Q), dev(K), dev(V)
        self.prefix_len = dev(prefix_len, np.int32)
        self.n_nodes = dev(n_nodes, np.int32)
        self.mask = dev(mask, np.uint8)
        self.O = torch.empty(tuple(self.Q.shape), dtype=torch.float32, device=device)
        self.workspace = None
        a = _lib.attn_args(self.Q, self.K, self.V, self.prefix_len, self.n_nodes, self.mask,
                           scale, self.O, splits)
        need = _lib.dtree_tree_attention_workspace(a)
        if need:
            self.workspace = torch.empty(need, dtype=torch.uint8, device=device)
        self.args = _lib.attn_args(self.Q, self.K, self.V, self.prefix_len, self.n_nodes,
                                   self.mask, scale, self.O, splits, self.workspace)

    def run(self, stream=None):
        _lib.dtree_tree_attention(self.args, stream)

    def output(self):
        return self.O.cpu().numpy()
