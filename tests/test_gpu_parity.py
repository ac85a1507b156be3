"""GPU path vs the CPU oracle, through the C ABI (needs a gfx950 GPU).

Structure must be identical and scores within 1e-4; near-ties are
tolerated only as described in checker.py.
"""
import numpy as np
import pytest

import synth
import fixtures_io
from checker import check_invariants
from gpu_util import check_config, gpu_round, caps_for

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", fixtures_io.fixture_names())
def test_golden_fixture_on_gpu(gpu_lib, name):
    g, x, exp = fixtures_io.load(name)
    p = g["params"]
    cfg = synth.custom_config(d=4, V=4, e=1, s=1, r=1, batch=1, wtype="f32", **p)
    out, tr = gpu_round(x, cfg)
    out = out[0]
    n = exp["n_nodes"]
    assert out["n_nodes"] == n
    assert out["tok"][:n].tolist() == exp["tok"]
    assert out["parent"][:n].tolist() == exp["parent"]
    assert out["depth"][:n].tolist() == exp["depth"]
    assert np.max(np.abs(out["score"][:n] - np.array(exp["score"]))) < g["score_tol"]
    assert out["mask"][:n, :n].tolist() == exp["mask"]
    check_invariants(out, p["B"])


@pytest.mark.parametrize("seed", range(240))
def test_tiny_seeds_exact(gpu_lib, seed):
    cfg = synth.CONFIGS["tiny"]
    check_config(synth.make_inputs(cfg, seed), cfg, f"tiny seed {seed}", seed=seed)


def _small_cfg(seed):
    rng = np.random.default_rng(100 + seed)
    wtype = "bf16" if seed % 2 else "f32"
    M = int(rng.choice([4, 16, 33, 64, 128]))
    K = int(rng.integers(1, min(M, 8) + 1))
    W = int(rng.choice([1, 3, 8, 17, 64]))
    while W * K > 1024:
        W //= 2
    d = 128 * int(rng.integers(1, 3)) if wtype == "bf16" else int(rng.integers(8, 100))
    V = int(rng.integers(max(M, 40), 3000))
    return synth.custom_config(cfg_id=5000 + seed, d=d, V=V, e=int(rng.integers(4, 80)),
                               s=int(rng.integers(4, 70)), r=int(rng.integers(2, 64)),
                               D=int(rng.integers(1, 9)), M=M, K=K, W=W,
                               B=int(rng.integers(1, 300)),
                               beta=float(rng.choice([0.0, -0.01, -0.3])),
                               batch=int(rng.integers(1, 5)), wtype=wtype)


@pytest.mark.parametrize("seed", range(24))
def test_random_small_shapes(gpu_lib, seed):
    cfg = _small_cfg(seed)
    check_config(synth.make_inputs(cfg, seed), cfg, f"small {seed}", max_ties_per_request=2,
                 seed=seed)


@pytest.mark.parametrize("seed,d,e,s,r,D,M,K,W,B,batch", [
    (0, 128, 128, 128, 32, 5, 32, 4, 8, 40, 1),
    (1, 256, 384, 128, 64, 8, 64, 8, 8, 100, 2),
    (2, 512, 128, 256, 16, 6, 16, 3, 16, 60, 4),
    (3, 128, 256, 384, 48, 4, 128, 8, 8, 90, 8),
    (4, 384, 128, 128, 256, 7, 33, 5, 12, 77, 3),
    # 8 x 32 = 256 expanded branches and 40 hidden rows: tiled products over
    # the two-plane states, tiled LM head with lists from the logits
    (5, 256, 128, 128, 64, 5, 64, 8, 32, 200, 8),
    (6, 128, 192, 256, 32, 4, 128, 4, 64, 150, 6),
    # 32 hidden rows and M > 64: exact lists by bisection from the logits,
    # V odd (4-byte logit loads) and V % 4 == 0 (16-byte loads)
    (7, 128, 128, 128, 32, 4, 128, 4, 16, 120, 8),
    (8, 256, 128, 128, 32, 4, 96, 4, 16, 120, 8),
    # rank 40 (a 32-wide k step and an 8-wide tail) on the matrix-core
    # correction logits: in the selection kernel up to 2048 branch-candidate
    # pairs, then 64 x 64 = 4096 in the stand-alone kernel (last depth)
    (9, 128, 128, 128, 40, 4, 64, 4, 64, 120, 2),
    # rank 8 (one partial k step), 96 candidates
    (10, 128, 64, 64, 8, 4, 96, 4, 32, 100, 2),
    # batched selection: odd state size (u rows not 16-byte aligned: scalar
    # loads), rank 24 (one partial k step), 12 survivors from 5 branches
    # (the Top-W bound over the first 3 children of every branch), ragged M
    (11, 128, 64, 61, 24, 5, 33, 5, 12, 60, 3),
    # rank 512 (16 k steps), 128 candidates, 64 survivors of 512 children
    (12, 128, 128, 128, 512, 4, 128, 8, 64, 200, 2),
    # 2560 candidates, e = 2048: the distinct tokens' input projections on
    # 128 x 64 tiles with the row count read on the device
    (13, 128, 2048, 192, 32, 4, 64, 4, 8, 60, 10),
])
def test_mfma_product_paths(gpu_lib, seed, d, e, s, r, D, M, K, W, B, batch):
    """bf16 shapes whose products run on the MFMA kernels: the row-gathered
    product, and for many rows the tiled products and tiled LM head."""
    cfg = synth.custom_config(cfg_id=8000 + seed, d=d, V=4000 + 17 * seed, e=e, s=s, r=r,
                              D=D, M=M, K=K, W=W, B=B, beta=-0.05, batch=batch, wtype="bf16")
    check_config(synth.make_inputs(cfg, seed), cfg, f"mfma {seed}", max_ties_per_request=2,
                 seed=seed)


def test_caps_larger_than_round(gpu_lib):
    cfg = synth.CONFIGS["tiny"].with_(batch=2)
    check_config(synth.make_inputs(cfg, 7), cfg, "tiny caps>params",
                 caps=caps_for(cfg, max_batch=5, max_D=9, max_M=32, max_K=4, max_W=16, max_B=40))


def test_determinism(gpu_lib):
    cfg = synth.custom_config(cfg_id=6000, d=256, V=5000, e=64, s=64, r=32, D=6, M=32, K=4,
                              W=8, B=40, beta=-0.05, batch=3, wtype="bf16")
    outs, _ = gpu_round(synth.make_inputs(cfg, 1), cfg, runs=3)
    for o in outs[1:]:
        for q in range(cfg.batch):
            for k in ("tok", "parent", "depth", "score", "mask"):
                assert np.array_equal(o[q][k], outs[0][q][k])


@pytest.mark.parametrize("seed,d,e,s,r,D,M,K,W,B,batch,beta", [
    (0, 128, 128, 128, 32, 5, 32, 4, 8, 40, 1, -0.05),
    (1, 256, 256, 256, 64, 9, 16, 3, 5, 60, 2, 0.0),
    (2, 128, 384, 128, 16, 1, 8, 2, 4, 3, 1, -0.1),
    (3, 256, 128, 384, 48, 7, 64, 1, 1, 7, 1, -0.2),
    (4, 128, 128, 128, 256, 12, 32, 8, 16, 120, 1, -0.01),
    (5, 384, 256, 128, 128, 6, 20, 4, 8, 50, 2, -0.05),
    (6, 128, 128, 1024, 256, 16, 32, 4, 8, 64, 1, -0.05),
])
def test_persistent_depth_loop(gpu_lib, seed, d, e, s, r, D, M, K, W, B, batch, beta):
    """Shapes that run the depth loop as one cooperative persistent kernel
    (bf16, GRU sizes multiple of 128, few branches per depth)."""
    cfg = synth.custom_config(cfg_id=9000 + seed, d=d, V=3000 + 31 * seed, e=e, s=s, r=r,
                              D=D, M=M, K=K, W=W, B=B, beta=beta, batch=batch, wtype="bf16")
    check_config(synth.make_inputs(cfg, seed), cfg, f"persistent {seed}", max_ties_per_request=2,
                 seed=seed)


@pytest.mark.parametrize("wtype,M,mode", [
    ("bf16", 32, "equal"), ("bf16", 64, "equal"), ("bf16", 128, "equal"),
    ("bf16", 32, "groups"), ("bf16", 64, "groups"), ("f32", 32, "equal"),
    ("f32", 64, "groups"),
])
def test_tied_base_logits(gpu_lib, wtype, M, mode):
    """Exact ties in the base logits (W_lm = 0, so the logits are the bias):
    the Top-M table breaks them by token, and slices with more tied keys
    than a candidate list holds take the exact per-slice path."""
    V = 40000 if wtype == "bf16" else 6000
    cfg = synth.custom_config(cfg_id=9500 + M, d=128 if wtype == "bf16" else 32, V=V, e=64,
                              s=64, r=32, D=4, M=M, K=4, W=8, B=60, beta=-0.05, batch=2,
                              wtype=wtype)
    x = synth.make_inputs(cfg, 3)
    x["weights"]["W_lm"] = np.zeros_like(x["weights"]["W_lm"])
    if mode == "equal":
        x["weights"]["bias"] = np.zeros(V, np.float32)
    else:
        perm = np.random.default_rng(5).permutation(V)
        x["weights"]["bias"] = (-0.25 * np.floor(perm / 97.0)).astype(np.float32)
    check_config(x, cfg, f"tied {wtype} M={M} {mode}")


@pytest.mark.parametrize("M,V,batch,D,mode", [
    (128, 40000, 8, 4, None),     # 32 rows: 320-token tiles, maxima of 80-column groups
    (32, 20011, 8, 4, None),      # odd V: 4-byte logit loads, a ragged last group
    (64, 30000, 12, 12, None),    # 144 rows: 256-token tiles, maxima of 64-column groups
    (32, 20000, 16, 16, None),    # 256 rows: 256 x 256 tiles
    (128, 40000, 8, 4, "equal"),  # every key tied: whole slices reach the bound,
    (32, 40000, 8, 4, "equal"),   #   so every list falls back to the exact search
    (32, 40000, 8, 4, "groups"),  # tied groups of 97 tokens spread over the vocabulary
    (128, 40000, 8, 4, "groups"),
])
def test_row_bound_lists(gpu_lib, M, V, batch, D, mode):
    """Candidate lists from the tiled LM head's logits under the row-wide
    bound (the M-th largest of the per-group logit maxima): every slice
    lists its keys at or above it, or, where those overflow a list, its
    exact M best."""
    cfg = synth.custom_config(cfg_id=9800 + M + D, d=128, V=V, e=64, s=64, r=32, D=D, M=M, K=4,
                              W=8, B=60, beta=-0.05, batch=batch, wtype="bf16")
    x = synth.make_inputs(cfg, 11)
    if mode is not None:
        x["weights"]["W_lm"] = np.zeros_like(x["weights"]["W_lm"])
        if mode == "equal":
            x["weights"]["bias"] = np.zeros(V, np.float32)
        else:
            perm = np.random.default_rng(5).permutation(V)
            x["weights"]["bias"] = (-0.25 * np.floor(perm / 97.0)).astype(np.float32)
        check_config(x, cfg, f"row bound M={M} V={V} {mode}")
    else:
        check_config(x, cfg, f"row bound M={M} V={V}", max_ties_per_request=2, seed=11)


def test_persistent_launch_modes(gpu_lib):
    """The persistent depth loop builds the same round with plain and with
    cooperative launches.  A round whose waits run out (forced from the host
    with a one-poll spin limit, so every kernel still ends normally) reports
    status bit 1, the next call fails loudly, and the context then uses
    cooperative launches and builds correct rounds again."""
    import torch
    from conditional_draft_tree_depth_amd import _lib, runner
    cfg = synth.custom_config(cfg_id=9100, d=128, V=3000, e=128, s=128, r=32, D=5, M=32, K=4,
                              W=8, B=40, beta=-0.05, batch=1, wtype="bf16")
    x = synth.make_inputs(cfg, 0)
    wd, H, root = runner.to_device(x)
    rnd = runner.Round(wd, cfg.wtype, caps_for(cfg), cfg.batch, cfg.D, cfg.M, cfg.K, cfg.W,
                       cfg.B, cfg.beta)
    keys = ("tok", "parent", "depth", "score", "mask")
    try:
        rnd.run(H, root)
        torch.cuda.synchronize()
        plain = rnd.outputs()
        assert rnd.trace(0)["status"] == 0
        _lib.dtree_set_persistent_launch(rnd.ctx, 1)
        rnd.run(H, root)
        torch.cuda.synchronize()
        coop = rnd.outputs()
        for k in keys:
            assert np.array_equal(plain[0][k], coop[0][k]), k
        print("[gpu] forcing a wait to run out (one poll)", flush=True)
        _lib.dtree_set_persistent_launch(rnd.ctx, 0, 1)
        rnd.run(H, root)
        torch.cuda.synchronize()
        assert rnd.trace(0)["status"] & 2
        # the failed round marks itself in its own outputs
        assert rnd.outputs()[0]["n_nodes"] == 0
        _lib.dtree_set_persistent_launch(rnd.ctx, 0, 0)
        with pytest.raises(_lib.DTreeError):
            rnd.run(H, root)
        rnd.run(H, root)
        torch.cuda.synchronize()
        again = rnd.outputs()
        assert rnd.trace(0)["status"] == 0
        for k in keys:
            assert np.array_equal(plain[0][k], again[0][k]), k
        with pytest.raises(_lib.DTreeError):
            _lib.dtree_set_persistent_launch(rnd.ctx, 2)
    finally:
        rnd.close()
    check_config(x, cfg, "persistent launch modes")


@pytest.mark.parametrize("B,beta", [(1200, -0.02), (1500, 0.0)])
def test_large_tree_budget(gpu_lib, B, beta):
    """Budgets past one workgroup's threads: 1364 superarbol nodes, B = 1200
    (three mask bands of rows, rank counts over several passes, emitted nodes
    past the 1024th) and B = 1500 (every node selected, empty tail slots)."""
    cfg = synth.custom_config(cfg_id=9700 + B, d=64, V=600, e=16, s=16, r=8, D=6, M=8, K=4,
                              W=128, B=B, beta=beta, batch=2, wtype="f32")
    check_config(synth.make_inputs(cfg, 3), cfg, f"large budget B={B}")
