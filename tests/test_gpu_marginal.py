"""Marginal (uncorrected, DDTree-style) scoring on the GPU vs the oracle's
marginal scoring: every branch is scored by the base logits of its depth's
candidates, with the rest of the round unchanged."""
import numpy as np
import pytest

import synth
from gpu_util import check_config, caps_for

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("seed", range(20))
def test_marginal_tiny_exact(gpu_lib, seed):
    cfg = synth.CONFIGS["tiny"]
    check_config(synth.make_inputs(cfg, seed), cfg, f"marginal tiny {seed}", scoring="marginal",
                 seed=seed)


@pytest.mark.parametrize("seed,wtype,d,V,M,K,W,B,D,batch", [
    (0, "f32", 40, 900, 16, 3, 8, 60, 5, 2),
    (1, "bf16", 256, 3000, 32, 4, 8, 64, 8, 1),
    (2, "bf16", 128, 2500, 64, 8, 32, 200, 6, 3),
    (3, "bf16", 256, 4000, 128, 8, 64, 300, 4, 8),
])
def test_marginal_shapes(gpu_lib, seed, wtype, d, V, M, K, W, B, D, batch):
    cfg = synth.custom_config(cfg_id=9500 + seed, d=d, V=V, e=64, s=64, r=32, D=D, M=M, K=K, W=W,
                              B=B, beta=-0.05, batch=batch, wtype=wtype)
    check_config(synth.make_inputs(cfg, seed), cfg, f"marginal shape {seed}", max_ties_per_request=2,
                 scoring="marginal", seed=seed)


@pytest.mark.parametrize("name", ["qwen3_4b", "wide", "qwen3_8b_x8"])
def test_marginal_full_size(gpu_lib, name):
    cfg = synth.CONFIGS[name]
    check_config(synth.make_inputs(cfg, 0), cfg, f"marginal {name}", max_ties_per_request=2,
                 scoring="marginal", seed=0)


def test_scoring_switch_on_one_context(gpu_lib):
    """One context: a marginal round, then conditional rounds again (the
    persistent depth loop included), each matching the oracle."""
    from conditional_draft_tree_depth_amd import runner, _lib
    from oracle import dtree_oracle as O
    from checker import compare_request
    import torch
    cfg = synth.custom_config(cfg_id=9600, d=128, V=3000, e=128, s=128, r=32, D=5, M=32, K=4,
                              W=8, B=40, beta=-0.05, batch=1, wtype="bf16")
    x = synth.make_inputs(cfg, 0)
    wd, H, root = runner.to_device(x)
    rnd = runner.Round(wd, cfg.wtype, caps_for(cfg), cfg.batch, cfg.D, cfg.M, cfg.K, cfg.W,
                       cfg.B, cfg.beta, scoring="marginal")
    prm = dict(D=cfg.D, M=cfg.M, K=cfg.K, W=cfg.W, B=cfg.B, beta=cfg.beta)
    prep = O.prepare_round(x, cfg.D)
    try:
        for mode in ("marginal", "conditional", "marginal", "conditional"):
            _lib.dtree_set_scoring(rnd.ctx, mode)
            rnd.run(H, root)
            torch.cuda.synchronize()
            out = rnd.outputs()[0]
            res = compare_request(out, rnd.trace(0), prep, 0, prm, where=f"switch {mode}: ",
                                  scoring=mode)
            assert res["exact"], res
        with pytest.raises(_lib.DTreeError):
            _lib.dtree_set_scoring(rnd.ctx, 7)
    finally:
        rnd.close()
