"""Seeded generator for the inputs of tree-attention verification.

A verification call attends, for every request, the N = B + 1 tree tokens
of a draft tree to the request's prefix (the verified context, already in
the KV cache) and to their own ancestors in the tree.  Nothing here
computes any part of the method: it draws tensors and random trees.

Layouts (bf16 tensors are returned as raw uint16 bit patterns):
  * Q      [batch, n_max, Hq, dh]   query of tree token i, head h;
  * K, V   [batch, Hkv, L_cap, dh]  cache: positions [0, prefix_len[q]) the
                                    prefix, then tree token j at prefix_len[q] + j;
  * prefix_len [batch] int32, n_nodes [batch] int32 (1 <= n_nodes <= n_max);
  * parent [batch, n_max] int32: -1 for the root (node 0) and for slots past
    n_nodes, else a node index smaller than the child's (canonical order).

Distributions: Q ~ N(0, 1), K ~ N(0, 2^2), V ~ N(0, 1), each rounded to
bf16 nearest-even; with scale 1/sqrt(dh) the logits are about N(0, 2^2).
Cache slots past prefix_len + n_nodes hold the same draws (they must never
be read).  Trees are random recursive trees: parent[i] is uniform on the
nodes of the previous depth level when ``shape="levels"`` (a tree that grows
depth by depth, as the draft builders do), or uniform on [0, i) when
``shape="recursive"``; ``shape="chain"`` gives parent[i] = i - 1.
"""
from dataclasses import dataclass, replace

import numpy as np

from .inputs import _normal, _rng, _to_bf16_bits

T_Q, T_K, T_V, T_TREE, T_PREFIX = range(20, 25)


@dataclass(frozen=True)
class AttnConfig:
    name: str
    cfg_id: int
    Hq: int
    Hkv: int
    dh: int
    n_max: int                    # B + 1
    batch: int
    prefix: tuple = ()            # per-request prefix lengths (len == batch)
    L_cap: int = 0                # cache capacity; 0 = max(prefix) + n_max
    n_nodes: tuple = ()           # per-request tree sizes; () = all n_max
    shape: str = "levels"

    def cap(self):
        return self.L_cap or (max(self.prefix) + self.n_max)

    def nodes(self):
        return self.n_nodes or (self.n_max,) * self.batch

    def with_(self, **kw):
        return replace(self, **kw)


# Attention shapes of the two target models named on the DARTree page
# (Qwen3-4B and Qwen3-8B: 32 query heads, 8 KV heads, head dim 128), one
# layer's call, with a 4096-token verified prefix per request.
ATTN_CONFIGS = {
    "attn_tiny": AttnConfig("attn_tiny", 40, Hq=4, Hkv=2, dh=64, n_max=17, batch=2,
                            prefix=(5, 40), n_nodes=(17, 11)),
    "attn_qwen3_4b": AttnConfig("attn_qwen3_4b", 41, Hq=32, Hkv=8, dh=128, n_max=65,
                                batch=1, prefix=(4096,)),
    "attn_wide": AttnConfig("attn_wide", 42, Hq=32, Hkv=8, dh=128, n_max=257, batch=1,
                            prefix=(4096,)),
    "attn_qwen3_8b_x8": AttnConfig("attn_qwen3_8b_x8", 43, Hq=32, Hkv=8, dh=128, n_max=129,
                                   batch=8, prefix=(4096,) * 8),
}


def random_parents(n_max, n, rng, shape="levels"):
    par = np.full(n_max, -1, np.int32)
    if shape == "chain":
        par[1:n] = np.arange(n - 1)
        return par
    if shape == "recursive":
        for i in range(1, n):
            par[i] = rng.integers(0, i)
        return par
    # depth by depth: each level's size drawn in [1, 2 * previous], nodes of
    # a level take parents from the previous level
    lo, hi, i = 0, 1, 1
    while i < n:
        width = int(rng.integers(1, 2 * (hi - lo) + 1))
        width = min(width, n - i)
        ps = np.sort(rng.integers(lo, hi, size=width))
        par[i:i + width] = ps
        lo, hi, i = i, i + width, i + width
    return par


def make_attn_inputs(cfg: AttnConfig, seed: int = 0) -> dict:
    b, L = cfg.batch, cfg.cap()
    assert len(cfg.prefix) == b and all(p + n <= L for p, n in zip(cfg.prefix, cfg.nodes()))
    Q = _normal((b, cfg.n_max, cfg.Hq, cfg.dh), 1.0, seed, cfg.cfg_id, T_Q)
    K = _normal((b, cfg.Hkv, L, cfg.dh), 2.0, seed, cfg.cfg_id, T_K)
    V = _normal((b, cfg.Hkv, L, cfg.dh), 1.0, seed, cfg.cfg_id, T_V)
    parent = np.stack([random_parents(cfg.n_max, n, _rng(seed, cfg.cfg_id, T_TREE, q), cfg.shape)
                       for q, n in enumerate(cfg.nodes())])
    return {"Q": _to_bf16_bits(Q), "K": _to_bf16_bits(K), "V": _to_bf16_bits(V),
            "prefix_len": np.array(cfg.prefix, np.int32),
            "n_nodes": np.array(cfg.nodes(), np.int32), "parent": parent,
            "scale": float(1.0 / np.sqrt(cfg.dh)), "L_cap": L}

