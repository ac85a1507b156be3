"""Markov (parent-token-only) scoring on the GPU vs the oracle's Markov
scoring: every survivor's GRU step starts from a zero state, the rest of
the round is unchanged."""
import pytest

import synth
from gpu_util import check_config

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("seed", range(20))
def test_markov_tiny_exact(gpu_lib, seed):
    cfg = synth.CONFIGS["tiny"]
    check_config(synth.make_inputs(cfg, seed), cfg, f"markov tiny {seed}", scoring="markov",
                 seed=seed)


@pytest.mark.parametrize("seed,wtype,d,V,s,M,K,W,B,D,batch", [
    (0, "f32", 40, 900, 24, 16, 3, 8, 60, 5, 2),
    (1, "bf16", 256, 3000, 128, 32, 4, 8, 64, 8, 1),
    (2, "bf16", 128, 2500, 64, 64, 8, 32, 200, 6, 3),
    (3, "bf16", 256, 4000, 64, 128, 8, 64, 300, 4, 8),
])
def test_markov_shapes(gpu_lib, seed, wtype, d, V, s, M, K, W, B, D, batch):
    cfg = synth.custom_config(cfg_id=9650 + seed, d=d, V=V, e=64, s=s, r=32, D=D, M=M, K=K, W=W,
                              B=B, beta=-0.05, batch=batch, wtype=wtype)
    check_config(synth.make_inputs(cfg, seed), cfg, f"markov shape {seed}",
                 max_ties_per_request=2, scoring="markov", seed=seed)


@pytest.mark.parametrize("name", ["qwen3_4b", "wide", "qwen3_8b_x8"])
def test_markov_full_size(gpu_lib, name):
    cfg = synth.CONFIGS[name]
    check_config(synth.make_inputs(cfg, 0), cfg, f"markov {name}", max_ties_per_request=2,
                 scoring="markov", seed=0)


def test_three_scorings_on_one_context(gpu_lib):
    """One context switching between the three scorings round by round (the
    persistent depth loop included for conditional rounds)."""
    from conditional_draft_tree_depth_amd import runner, _lib
    from oracle import dtree_oracle as O
    from checker import compare_request
    from gpu_util import caps_for
    import torch
    cfg = synth.custom_config(cfg_id=9660, d=128, V=3000, e=128, s=128, r=32, D=5, M=32, K=4,
                              W=8, B=40, beta=-0.05, batch=1, wtype="bf16")
    x = synth.make_inputs(cfg, 0)
    wd, H, root = runner.to_device(x)
    rnd = runner.Round(wd, cfg.wtype, caps_for(cfg), cfg.batch, cfg.D, cfg.M, cfg.K, cfg.W,
                       cfg.B, cfg.beta)
    prm = dict(D=cfg.D, M=cfg.M, K=cfg.K, W=cfg.W, B=cfg.B, beta=cfg.beta)
    prep = O.prepare_round(x, cfg.D)
    try:
        for mode in ("markov", "conditional", "marginal", "markov", "conditional"):
            _lib.dtree_set_scoring(rnd.ctx, mode)
            rnd.run(H, root)
            torch.cuda.synchronize()
            res = compare_request(rnd.outputs()[0], rnd.trace(0), prep, 0, prm,
                                  where=f"switch {mode}: ", scoring=mode)
            assert res["exact"], res
    finally:
        rnd.close()
