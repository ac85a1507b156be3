"""The sequential best-first builder on the GPU vs the oracle's best-first
builder, every request compared to its last node: candidates, every
expansion's children, every pushed node's score, the pop set, and the
emitted tree."""
import numpy as np
import pytest

import synth
from gpu_util import check_config, caps_for

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("seed", range(20))
def test_heap_tiny_exact(gpu_lib, seed):
    cfg = synth.CONFIGS["tiny"]
    check_config(synth.make_inputs(cfg, seed), cfg, f"heap tiny {seed}", seed=seed,
                 builder="heap")


@pytest.mark.parametrize("seed", range(6))
def test_heap_tiny_markov(gpu_lib, seed):
    cfg = synth.CONFIGS["tiny"]
    check_config(synth.make_inputs(cfg, seed), cfg, f"heap markov tiny {seed}", seed=seed,
                 scoring="markov", builder="heap")


@pytest.mark.parametrize("seed,wtype,d,V,s,M,K,B,D,batch,beta", [
    (0, "f32", 40, 900, 24, 16, 3, 60, 5, 2, -0.05),
    (1, "bf16", 256, 3000, 128, 32, 4, 64, 8, 1, -0.05),
    (2, "bf16", 128, 2500, 64, 64, 8, 200, 6, 3, 0.0),
    (3, "bf16", 256, 4000, 64, 16, 2, 40, 3, 4, -0.2),
    (4, "f32", 64, 512, 32, 4, 2, 20, 2, 2, -0.1),      # the heap empties after 6 pops
])
def test_heap_shapes(gpu_lib, seed, wtype, d, V, s, M, K, B, D, batch, beta):
    cfg = synth.custom_config(cfg_id=9700 + seed, d=d, V=V, e=64, s=s, r=32, D=D, M=M, K=K, W=4,
                              B=B, beta=beta, batch=batch, wtype=wtype)
    check_config(synth.make_inputs(cfg, seed), cfg, f"heap shape {seed}", max_ties_per_request=2,
                 seed=seed, builder="heap")


@pytest.mark.parametrize("seed,wtype,s,r,M,K,B,D", [
    (10, "f32", 30, 30, 5, 2, 30, 3),       # rows not 16-byte multiples: scalar loads
    (11, "bf16", 40, 36, 12, 3, 40, 5),     # bf16 rows of 72 bytes: scalar loads
    (12, "bf16", 64, 32, 128, 8, 50, 4),    # the most candidates: two lanes each
    (13, "bf16", 64, 64, 100, 8, 50, 3),    # 100 candidates, 8 pieces per lane
])
def test_heap_load_paths(gpu_lib, seed, wtype, s, r, M, K, B, D):
    """Shapes on both sides of the 16-byte load path and of the lanes per
    candidate of the correction dot products."""
    cfg = synth.custom_config(cfg_id=9700 + seed, d=128, V=2000, e=48, s=s, r=r, D=D, M=M, K=K,
                              W=4, B=B, beta=-0.05, batch=2, wtype=wtype)
    check_config(synth.make_inputs(cfg, seed), cfg, f"heap load path {seed}",
                 max_ties_per_request=2, seed=seed, builder="heap")


@pytest.mark.parametrize("name", ["qwen3_4b", "qwen3_8b_x8"])
def test_heap_full_size(gpu_lib, name):
    cfg = synth.CONFIGS[name]
    check_config(synth.make_inputs(cfg, 0), cfg, f"heap {name}", max_ties_per_request=2,
                 seed=0, builder="heap")


def test_builders_and_scorings_on_one_context(gpu_lib):
    """One context switching builder and scoring round by round; the heap
    builder refuses marginal scoring before enqueueing anything."""
    from conditional_draft_tree_depth_amd import runner, _lib
    from oracle import dtree_oracle as O
    from checker import compare_request, compare_heap_request
    import torch
    cfg = synth.custom_config(cfg_id=9760, d=128, V=3000, e=128, s=128, r=32, D=5, M=32, K=4,
                              W=8, B=40, beta=-0.05, batch=1, wtype="bf16")
    x = synth.make_inputs(cfg, 0)
    wd, H, root = runner.to_device(x)
    rnd = runner.Round(wd, cfg.wtype, caps_for(cfg), cfg.batch, cfg.D, cfg.M, cfg.K, cfg.W,
                       cfg.B, cfg.beta)
    prm = dict(D=cfg.D, M=cfg.M, K=cfg.K, W=cfg.W, B=cfg.B, beta=cfg.beta)
    prep = O.prepare_round(x, cfg.D)
    try:
        for builder, scoring in (("heap", "conditional"), ("depthwise", "conditional"),
                                 ("heap", "markov"), ("depthwise", "marginal"),
                                 ("heap", "conditional")):
            _lib.dtree_set_builder(rnd.ctx, builder)
            _lib.dtree_set_scoring(rnd.ctx, scoring)
            rnd.builder = builder
            rnd.run(H, root)
            torch.cuda.synchronize()
            cmp = compare_heap_request if builder == "heap" else compare_request
            res = cmp(rnd.outputs()[0], rnd.trace(0), prep, 0, prm,
                      where=f"{builder}/{scoring}: ", scoring=scoring)
            assert res["exact"], res
        _lib.dtree_set_scoring(rnd.ctx, "marginal")
        with pytest.raises(_lib.DTreeError) as e:
            rnd.run(H, root)
        assert e.value.code == 1
    finally:
        rnd.close()
