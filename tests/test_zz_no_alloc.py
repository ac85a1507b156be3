"""The allocation-free round (dtree_build_round_static) through the C ABI:
two calls in a row, the second with a smaller input, each compared with
dtree_build_round on a context with the same parameters and inputs
(structure identical, scores within 1e-4) and with the oracle's round."""
import numpy as np
import pytest

import synth
from gpu_util import gpu_round
from oracle import dtree_oracle as O

pytestmark = pytest.mark.gpu


def _static_round(x, cfg):
    import torch
    from conditional_draft_tree_depth_amd import _lib, runner
    wd, H, root = runner.to_device(x)
    N = cfg.B + 1
    dev = "cuda"
    o = dict(tok=torch.full((cfg.batch, N), 7, dtype=torch.int32, device=dev),
             parent=torch.full((cfg.batch, N), 7, dtype=torch.int32, device=dev),
             depth=torch.full((cfg.batch, N), 7, dtype=torch.int32, device=dev),
             score=torch.full((cfg.batch, N), 7.0, dtype=torch.float32, device=dev),
             mask=torch.full((cfg.batch, N, N), 7, dtype=torch.uint8, device=dev),
             n_nodes=torch.full((cfg.batch,), 7, dtype=torch.int32, device=dev))
    p = _lib.params(cfg.D, cfg.M, cfg.K, cfg.W, cfg.B, cfg.beta)
    _lib.dtree_build_round_static(wd, cfg.wtype, p, cfg.batch, H, root, o["tok"], o["parent"],
                                  o["depth"], o["score"], o["mask"], o["n_nodes"])
    torch.cuda.synchronize()
    return [{k: (int(v[q]) if k == "n_nodes" else v[q].cpu().numpy()) for k, v in o.items()}
            for q in range(cfg.batch)]


def _same_round(a, b, where):
    n = a["n_nodes"]
    assert n == b["n_nodes"], where
    for k in ("tok", "parent", "depth", "mask"):
        assert np.array_equal(a[k], b[k]), f"{where}: {k}"
    assert np.max(np.abs(a["score"][:n] - b["score"][:n])) <= 1e-4, where
    assert np.array_equal(np.isneginf(a["score"]), np.isneginf(b["score"])), where


def test_static_round_two_calls_second_smaller(gpu_lib):
    big = synth.CONFIGS["qwen3_4b"]
    small = synth.custom_config(cfg_id=9900, d=256, V=3000, e=64, s=64, r=32, D=4, M=16,
                                K=3, W=6, B=30, beta=-0.1, batch=1, wtype="bf16")
    for cfg, seed in ((big, 11), (small, 12)):
        print(f"[gpu] static round {cfg.name}: batch={cfg.batch} D={cfg.D} M={cfg.M} "
              f"W={cfg.W} B={cfg.B}", flush=True)
        x = synth.make_inputs(cfg, seed)
        got = _static_round(x, cfg)
        ref, _ = gpu_round(x, cfg)
        orc = O.build_round(x, cfg.D, cfg.M, cfg.K, cfg.W, cfg.B, cfg.beta)
        for q in range(cfg.batch):
            _same_round(got[q], ref[q], f"{cfg.name} req {q} vs dtree_build_round")
            _same_round(got[q], orc[q], f"{cfg.name} req {q} vs oracle")
