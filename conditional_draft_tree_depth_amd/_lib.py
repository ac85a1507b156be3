"""ctypes binding of libdtree.so: the C ABI of include/dtree.h, same names.

Argument marshalling only.  Every step of a round runs in the library's HIP
kernels; torch tensors are used for device memory and the stream handle.
There is no fallback: if the library is missing or the device is not a
gfx950, the calls raise.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdtree.so")

DTREE_F32, DTREE_BF16 = 0, 1
STATUS = {0: "DTREE_OK", 1: "DTREE_E_ARG", 2: "DTREE_E_SHAPE", 3: "DTREE_E_DTYPE",
          4: "DTREE_E_DEVICE", 5: "DTREE_E_NOMEM", 6: "DTREE_E_HIP", 7: "DTREE_E_STATE"}
EXPORTS = ("dtree_create", "dtree_build_round", "dtree_build_round_static",
           "dtree_superarbol_nodes",
           "dtree_get_trace", "dtree_profile_enable", "dtree_profile_read",
           "dtree_set_persistent_launch", "dtree_set_scoring", "dtree_last_error",
           "dtree_destroy", "dtree_tree_attention_workspace", "dtree_tree_attention",
           "dtree_set_builder", "dtree_heap_nodes")
NSTAGES = 6
STAGES = ("round_start", "lmhead_topm", "topm_merge", "prologue", "depth_loop", "topb_emit")

c_i32, c_vp, c_f32 = ctypes.c_int32, ctypes.c_void_p, ctypes.c_float


class dtree_weights(ctypes.Structure):
    _fields_ = [("d", c_i32), ("V", c_i32), ("e", c_i32), ("s", c_i32), ("r", c_i32),
                ("wtype", c_i32), ("W_lm", c_vp), ("lm_bias", c_vp), ("Emb", c_vp),
                ("W_ih", c_vp), ("W_hh", c_vp), ("b_ih", c_vp), ("b_hh", c_vp),
                ("W1", c_vp), ("W2", c_vp)]


class dtree_caps(ctypes.Structure):
    _fields_ = [("max_batch", c_i32), ("max_D", c_i32), ("max_M", c_i32),
                ("max_K", c_i32), ("max_W", c_i32), ("max_B", c_i32)]


class dtree_params(ctypes.Structure):
    _fields_ = [("D", c_i32), ("M", c_i32), ("K", c_i32), ("W", c_i32), ("B", c_i32),
                ("beta", c_f32)]


class dtree_trace(ctypes.Structure):
    _fields_ = [("C", c_vp), ("Cl", c_vp), ("node_tok", c_vp), ("node_parent", c_vp),
                ("node_score", c_vp), ("surv", c_vp), ("sel", c_vp), ("n_sa", c_i32),
                ("status", c_i32)]


class dtree_attn_args(ctypes.Structure):
    _fields_ = [("batch", c_i32), ("n_max", c_i32), ("Hq", c_i32), ("Hkv", c_i32),
                ("dh", c_i32), ("L_cap", c_i32), ("Q", c_vp), ("K", c_vp), ("V", c_vp),
                ("prefix_len", c_vp), ("n_nodes", c_vp), ("mask", c_vp), ("scale", c_f32),
                ("O", c_vp), ("splits", c_i32), ("workspace", c_vp),
                ("workspace_bytes", ctypes.c_size_t)]


class DTreeError(RuntimeError):
    def __init__(self, fn, code, msg):
        super().__init__(f"{fn}: {STATUS.get(code, code)}: {msg}")
        self.code = code


_lib = None


def load(path=LIB_PATH):
    """Open libdtree.so and declare the C signatures (once)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run __graft_entry__.build() first")
    # torch brings its own HIP runtime; loading it first makes the library bind
    # to that same runtime instance, so torch's device pointers are valid here
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    lib.dtree_create.argtypes = [P(dtree_weights), P(dtree_caps), ctypes.c_int,
                                 P(ctypes.c_void_p)]
    lib.dtree_create.restype = c_i32
    lib.dtree_build_round.argtypes = [c_vp, P(dtree_params), c_i32, c_vp, c_vp, c_vp, c_vp,
                                      c_vp, c_vp, c_vp, c_vp, c_vp]
    lib.dtree_build_round.restype = c_i32
    lib.dtree_build_round_static.argtypes = [P(dtree_weights), P(dtree_params), c_i32, c_vp,
                                             c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]
    lib.dtree_build_round_static.restype = c_i32
    lib.dtree_superarbol_nodes.argtypes = [P(dtree_params)]
    lib.dtree_superarbol_nodes.restype = c_i32
    lib.dtree_get_trace.argtypes = [c_vp, c_i32, P(dtree_trace)]
    lib.dtree_get_trace.restype = c_i32
    lib.dtree_profile_enable.argtypes = [c_vp, ctypes.c_int]
    lib.dtree_profile_enable.restype = c_i32
    lib.dtree_profile_read.argtypes = [c_vp, P(c_f32), P(c_i32)]
    lib.dtree_profile_read.restype = c_i32
    lib.dtree_set_persistent_launch.argtypes = [c_vp, c_i32, c_i32]
    lib.dtree_set_persistent_launch.restype = c_i32
    lib.dtree_set_scoring.argtypes = [c_vp, c_i32]
    lib.dtree_set_scoring.restype = c_i32
    lib.dtree_last_error.argtypes = [c_vp]
    lib.dtree_last_error.restype = ctypes.c_char_p
    lib.dtree_destroy.argtypes = [c_vp]
    lib.dtree_destroy.restype = c_i32
    lib.dtree_set_builder.argtypes = [c_vp, c_i32]
    lib.dtree_set_builder.restype = c_i32
    lib.dtree_heap_nodes.argtypes = [P(dtree_params)]
    lib.dtree_heap_nodes.restype = c_i32
    lib.dtree_tree_attention_workspace.argtypes = [P(dtree_attn_args), P(ctypes.c_size_t)]
    lib.dtree_tree_attention_workspace.restype = c_i32
    lib.dtree_tree_attention.argtypes = [P(dtree_attn_args), c_vp]
    lib.dtree_tree_attention.restype = c_i32
    _lib = lib
    return lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(fn, code, ctx=None):
    if code != 0:
        msg = load().dtree_last_error(ctx).decode()
        raise DTreeError(fn, code, msg)


def params(D, M, K, W, B, beta):
    return dtree_params(D, M, K, W, B, beta)


def dtree_superarbol_nodes(p):
    return load().dtree_superarbol_nodes(ctypes.byref(p))


def weights_struct(weights, wtype):
    """dtree_weights of a dict of contiguous device tensors (W_lm, bias, Emb,
    W_ih, W_hh, b_ih, b_hh, W1, W2); bf16 matrices as torch.bfloat16 or int16
    views."""
    W_lm, W1 = weights["W_lm"], weights["W1"]
    V, d = W_lm.shape
    s = weights["W_hh"].shape[1]
    return dtree_weights(d, V, weights["Emb"].shape[1], s, W1.shape[0],
                         DTREE_BF16 if wtype == "bf16" else DTREE_F32,
                         _ptr(W_lm), _ptr(weights.get("bias")), _ptr(weights["Emb"]),
                         _ptr(weights["W_ih"]), _ptr(weights["W_hh"]), _ptr(weights.get("b_ih")),
                         _ptr(weights.get("b_hh")), _ptr(W1), _ptr(weights["W2"]))


def dtree_create(weights, wtype, caps, device=0):
    """weights: dict of contiguous device tensors (see weights_struct).
    Returns an opaque context handle (c_void_p)."""
    lib = load()
    w = weights_struct(weights, wtype)
    c = dtree_caps(*caps) if not isinstance(caps, dtree_caps) else caps
    ctx = ctypes.c_void_p()
    _check("dtree_create", lib.dtree_create(ctypes.byref(w), ctypes.byref(c), device,
                                            ctypes.byref(ctx)))
    return ctx


def dtree_build_round(ctx, p, batch, H, root, tok, parent, depth, score, mask, n_nodes,
                      stream=None):
    """Enqueue one round; all tensors are device tensors (see dtree.h)."""
    import torch
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    _check("dtree_build_round",
           load().dtree_build_round(ctx, ctypes.byref(p), batch, _ptr(H), _ptr(root),
                                    _ptr(tok), _ptr(parent), _ptr(depth), _ptr(score),
                                    _ptr(mask), _ptr(n_nodes), ctypes.c_void_p(stream)),
           ctx)


def dtree_build_round_static(weights, wtype, p, batch, H, root, tok, parent, depth, score,
                             mask, n_nodes, stream=None):
    """The allocation-free round (no context): weights as for dtree_create."""
    import torch
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    w = weights_struct(weights, wtype)
    _check("dtree_build_round_static",
           load().dtree_build_round_static(ctypes.byref(w), ctypes.byref(p), batch, _ptr(H),
                                           _ptr(root), _ptr(tok), _ptr(parent), _ptr(depth),
                                           _ptr(score), _ptr(mask), _ptr(n_nodes),
                                           ctypes.c_void_p(stream)))


def dtree_get_trace(ctx, req, p, batch_nodes):
    """Host numpy copies of request `req`'s intermediates of the last round."""
    import numpy as np
    C = np.empty(p.D * p.M, np.int32)
    Cl = np.empty(p.D * p.M, np.float32)
    nt = np.empty(batch_nodes, np.int32)
    npar = np.empty(batch_nodes, np.int32)
    nsc = np.empty(batch_nodes, np.float32)
    surv = np.empty((p.D + 1) * p.W, np.int32)
    sel = np.empty(p.B, np.int32)
    tr = dtree_trace(C.ctypes.data, Cl.ctypes.data, nt.ctypes.data, npar.ctypes.data,
                     nsc.ctypes.data, surv.ctypes.data, sel.ctypes.data, 0, 0)
    _check("dtree_get_trace", load().dtree_get_trace(ctx, req, ctypes.byref(tr)), ctx)
    return dict(C=C.reshape(p.D, p.M), Cl=Cl.reshape(p.D, p.M), node_tok=nt[:tr.n_sa],
                node_parent=npar[:tr.n_sa], node_score=nsc[:tr.n_sa],
                surv=surv.reshape(p.D + 1, p.W), sel=sel, n_sa=tr.n_sa, status=tr.status)


def dtree_profile_enable(ctx, enable=True):
    _check("dtree_profile_enable", load().dtree_profile_enable(ctx, 1 if enable else 0), ctx)


def dtree_profile_read(ctx):
    """{stage name: summed ms}, rounds -- over the rounds since enabling."""
    ms = (c_f32 * NSTAGES)()
    n = c_i32(0)
    _check("dtree_profile_read", load().dtree_profile_read(ctx, ms, ctypes.byref(n)), ctx)
    return dict(zip(STAGES, list(ms))), n.value


def dtree_last_error(ctx=None):
    return load().dtree_last_error(ctx).decode()


def dtree_destroy(ctx):
    _check("dtree_destroy", load().dtree_destroy(ctx))


def dtree_set_persistent_launch(ctx, cooperative, spin_limit=0):
    _check("dtree_set_persistent_launch",
           load().dtree_set_persistent_launch(ctx, int(cooperative), int(spin_limit)), ctx)


SCORE_CONDITIONAL, SCORE_MARGINAL, SCORE_MARKOV = 0, 1, 2
SCORINGS = {"conditional": SCORE_CONDITIONAL, "marginal": SCORE_MARGINAL,
            "markov": SCORE_MARKOV}


BUILD_DEPTHWISE, BUILD_HEAP = 0, 1
BUILDERS = {"depthwise": BUILD_DEPTHWISE, "heap": BUILD_HEAP}


def dtree_set_builder(ctx, builder):
    """builder: "depthwise" / "heap" (or the DTREE_BUILD_* value)."""
    code = BUILDERS[builder] if isinstance(builder, str) else int(builder)
    _check("dtree_set_builder", load().dtree_set_builder(ctx, code), ctx)


def dtree_heap_nodes(p):
    return load().dtree_heap_nodes(ctypes.byref(p))


def dtree_set_scoring(ctx, scoring):
    """scoring: "conditional" / "marginal" / "markov" (or the DTREE_SCORE_* value)."""
    code = SCORINGS[scoring] if isinstance(scoring, str) else int(scoring)
    _check("dtree_set_scoring", load().dtree_set_scoring(ctx, code), ctx)


def attn_args(Q, K, V, prefix_len, n_nodes, mask, scale, O, splits=0, workspace=None):
    """dtree_attn_args of device tensors: Q [b, n_max, Hq, dh] and K, V
    [b, Hkv, L_cap, dh] bf16 (torch.bfloat16 or int16 views), prefix_len and
    n_nodes [b] int32, mask [b, n_max, n_max] uint8, O [b, n_max, Hq, dh] fp32."""
    b, n_max, Hq, dh = Q.shape
    Hkv, L_cap = K.shape[1], K.shape[2]
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return dtree_attn_args(b, n_max, Hq, Hkv, dh, L_cap, _ptr(Q), _ptr(K), _ptr(V),
                           _ptr(prefix_len), _ptr(n_nodes), _ptr(mask), float(scale), _ptr(O),
                           int(splits), _ptr(workspace), nbytes)


def dtree_tree_attention_workspace(a):
    """Workspace bytes a dtree_attn_args needs (0: none)."""
    n = ctypes.c_size_t(0)
    _check("dtree_tree_attention_workspace",
           load().dtree_tree_attention_workspace(ctypes.byref(a), ctypes.byref(n)))
    return n.value


def dtree_tree_attention(a, stream=None):
    """Enqueue one tree-attention call (see dtree.h)."""
    import torch
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    _check("dtree_tree_attention",
           load().dtree_tree_attention(ctypes.byref(a), ctypes.c_void_p(stream)))
