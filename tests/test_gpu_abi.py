"""The C ABI on a live context (needs a gfx950 GPU): every argument error of
dtree_build_round returns its code before anything is enqueued (the output
buffers keep a sentinel fill, the stream stays empty), dtree_get_trace
before any round returns DTREE_E_STATE, and the persistent depth loop is
deterministic at the Qwen3-4B shape it serves."""
import ctypes
import math

import numpy as np
import pytest

import synth
from gpu_util import caps_for, gpu_round

pytestmark = pytest.mark.gpu

E_ARG, E_STATE = 1, 7


def _ctx(cfg, seed=0):
    from conditional_draft_tree_depth_amd import runner
    x = synth.make_inputs(cfg, seed)
    wd, H, root = runner.to_device(x)
    rnd = runner.Round(wd, cfg.wtype, caps_for(cfg), cfg.batch, cfg.D, cfg.M, cfg.K, cfg.W,
                       cfg.B, cfg.beta)
    return rnd, H, root


def _call(lib, rnd, p, batch, H, root, null=None):
    args = dict(H=H, root=root, tok=rnd.tok, parent=rnd.parent, depth=rnd.depth,
                score=rnd.score, mask=rnd.mask, n_nodes=rnd.n_nodes)
    ptr = {k: (None if k == null else ctypes.c_void_p(v.data_ptr())) for k, v in args.items()}
    return lib.dtree_build_round(rnd.ctx, ctypes.byref(p), batch, ptr["H"], ptr["root"],
                                 ptr["tok"], ptr["parent"], ptr["depth"], ptr["score"],
                                 ptr["mask"], ptr["n_nodes"], None)


def test_build_round_argument_errors_enqueue_nothing(gpu_lib):
    import torch
    from conditional_draft_tree_depth_amd import _lib
    cfg = synth.custom_config(cfg_id=9800, d=128, V=3000, e=128, s=128, r=32, D=5, M=32, K=4,
                              W=8, B=40, beta=-0.05, batch=2, wtype="bf16")
    rnd, H, root = _ctx(cfg)
    lib = _lib.load()
    try:
        # no round yet: the trace is out of order
        tr = _lib.dtree_trace()
        assert lib.dtree_get_trace(rnd.ctx, 0, ctypes.byref(tr)) == E_STATE
        assert b"no round" in lib.dtree_last_error(rnd.ctx)
        for t in (rnd.tok, rnd.parent, rnd.depth, rnd.n_nodes):
            t.fill_(-7)
        rnd.score.fill_(7.0)
        rnd.mask.fill_(7)
        torch.cuda.synchronize()
        good = dict(D=5, M=32, K=4, W=8, B=40, beta=-0.05)
        bad = [
            dict(beta=0.25), dict(beta=math.nan), dict(beta=-math.inf), dict(K=33),
            dict(K=0), dict(M=0), dict(M=40), dict(W=0), dict(W=9), dict(B=0), dict(B=41),
            dict(D=0), dict(D=6),
        ]
        for over in bad:
            p = _lib.params(**{**good, **over})
            assert _call(lib, rnd, p, 2, H, root) == E_ARG, over
            assert lib.dtree_last_error(rnd.ctx) != b""
        p = _lib.params(**good)
        for batch in (0, 3, -1):
            assert _call(lib, rnd, p, batch, H, root) == E_ARG, batch
        for null in ("H", "root", "tok", "parent", "depth", "score", "mask", "n_nodes"):
            assert _call(lib, rnd, p, 2, H, root, null=null) == E_ARG, null
        assert lib.dtree_build_round(rnd.ctx, None, 2, *([None] * 9)) == E_ARG
        torch.cuda.synchronize()
        # nothing was enqueued: every output still holds its sentinel, and
        # the trace is still out of order
        for t in (rnd.tok, rnd.parent, rnd.depth, rnd.n_nodes):
            assert bool((t == -7).all())
        assert bool((rnd.score == 7.0).all()) and bool((rnd.mask == 7).all())
        assert lib.dtree_get_trace(rnd.ctx, 0, ctypes.byref(tr)) == E_STATE
        # and the context still builds a valid round afterwards
        assert _call(lib, rnd, p, 2, H, root) == 0
        torch.cuda.synchronize()
        assert int(rnd.n_nodes.min()) >= 1
        with pytest.raises(_lib.DTreeError):
            rnd.trace(2)   # request index out of range
    finally:
        rnd.close()


def test_persistent_loop_deterministic_at_qwen3_4b_shape(gpu_lib):
    """Three rounds of the Qwen3-4B workload on one context (the persistent
    depth loop at s = 1024) are bit-identical."""
    cfg = synth.CONFIGS["qwen3_4b"]
    outs, _ = gpu_round(synth.make_inputs(cfg, 5), cfg, runs=3)
    for o in outs[1:]:
        for k in ("tok", "parent", "depth", "score", "mask", "n_nodes"):
            assert np.array_equal(o[0][k], outs[0][0][k]), k
