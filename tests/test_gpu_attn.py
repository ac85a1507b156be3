"""Tree-attention verification on the GPU vs the attention oracle.

Every element of every row is compared: |O_gpu - O| <= (2^-8 + 2.5e-4)
sum_k w_k |V_k| + 1e-5 (the kernel rounds the softmax weights to bf16 and
sums in fp32), rows past n_nodes exactly 0."""
import numpy as np
import pytest

import synth
from oracle import tree_attention as TA

pytestmark = pytest.mark.gpu


def _masks(x, n_max):
    return np.stack([TA.ancestor_mask(x["parent"][q], int(x["n_nodes"][q]), n_max)
                     for q in range(len(x["n_nodes"]))])


def _check(Og, x, masks, label):
    Oref, absw = TA.tree_attention(x["Q"], x["K"], x["V"], x["prefix_len"], x["n_nodes"], masks,
                                   x["scale"])
    bound = TA.parity_bound(absw)
    err = np.abs(Og.astype(np.float64) - Oref)
    for q, n in enumerate(x["n_nodes"]):
        assert np.all(Og[q, n:] == 0), f"{label}: padding rows of request {q}"
    worst = float(np.max(err / bound))
    print(f"[gpu] {label}: max |err| {err.max():.3e}, max err/bound {worst:.3f}", flush=True)
    assert np.all(np.isfinite(Og)) and worst <= 1.0, label


def _run(x, masks, splits=0):
    from conditional_draft_tree_depth_amd import runner
    import torch
    ta = runner.TreeAttention(x["Q"], x["K"], x["V"], x["prefix_len"], x["n_nodes"], masks,
                              x["scale"], splits)
    ta.run()
    torch.cuda.synchronize()
    return ta.output()


_TINY = [
    ({}, 0), ({}, 1), ({}, 3),
    ({"shape": "recursive"}, 2),
    ({"shape": "chain"}, 0),
    ({"prefix": (0, 3), "n_nodes": (17, 1)}, 1),
    ({"prefix": (0, 3), "n_nodes": (17, 1)}, 4),
    ({"Hq": 8, "Hkv": 1, "dh": 128}, 0),
    ({"Hq": 3, "Hkv": 3, "n_max": 9, "n_nodes": (9, 4)}, 2),
    ({"prefix": (200, 77), "L_cap": 300}, 0),
    ({"prefix": (200, 77), "L_cap": 300}, 5),
]


@pytest.mark.parametrize("over,splits", _TINY)
@pytest.mark.parametrize("seed", [0, 1])
def test_attn_tiny(gpu_lib, over, splits, seed):
    cfg = synth.ATTN_CONFIGS["attn_tiny"].with_(**over)
    x = synth.make_attn_inputs(cfg, seed)
    m = _masks(x, cfg.n_max)
    _check(_run(x, m, splits), x, m, f"attn tiny {over} splits={splits} seed={seed}")


@pytest.mark.parametrize("name", ["attn_qwen3_4b", "attn_wide", "attn_qwen3_8b_x8"])
def test_attn_full_size(gpu_lib, name):
    cfg = synth.ATTN_CONFIGS[name]
    x = synth.make_attn_inputs(cfg, 0)
    m = _masks(x, cfg.n_max)
    _check(_run(x, m), x, m, name)


def test_attn_full_size_one_split(gpu_lib):
    cfg = synth.ATTN_CONFIGS["attn_qwen3_4b"]
    x = synth.make_attn_inputs(cfg, 1)
    m = _masks(x, cfg.n_max)
    _check(_run(x, m, splits=1), x, m, "qwen3_4b one split")


def test_attn_ragged_batch(gpu_lib):
    """Eight requests with different prefix lengths and tree sizes (the
    largest tree 513 nodes, a 4096-token cache)."""
    cfg = synth.AttnConfig("attn_ragged", 44, Hq=32, Hkv=8, dh=128, n_max=513, batch=8,
                           prefix=(0, 1, 63, 64, 65, 1000, 2047, 3583), L_cap=4096,
                           n_nodes=(513, 1, 2, 64, 65, 129, 300, 513), shape="recursive")
    x = synth.make_attn_inputs(cfg, 0)
    m = _masks(x, cfg.n_max)
    for splits in (0, 1, 7):
        _check(_run(x, m, splits), x, m, f"ragged splits={splits}")


def test_attn_bad_request_marked(gpu_lib):
    """A request whose lengths do not fit the cache reads nothing and gets
    NaN rows; the others are unaffected."""
    cfg = synth.ATTN_CONFIGS["attn_tiny"]
    x = synth.make_attn_inputs(cfg, 0)
    m = _masks(x, cfg.n_max)
    good = _run(x, m)
    for bad_prefix, bad_n, splits in ((x["L_cap"], 11, 0), (-1, 11, 3), (40, 0, 1),
                                      (40, cfg.n_max + 1, 2)):
        xb = dict(x, prefix_len=np.array([x["prefix_len"][0], bad_prefix], np.int32),
                  n_nodes=np.array([x["n_nodes"][0], bad_n], np.int32))
        out = _run(xb, m, splits)
        assert np.all(np.isnan(out[1])), (bad_prefix, bad_n)
        np.testing.assert_array_equal(out[0], good[0])


def test_attn_deterministic(gpu_lib):
    from conditional_draft_tree_depth_amd import runner
    import torch
    cfg = synth.ATTN_CONFIGS["attn_qwen3_4b"]
    x = synth.make_attn_inputs(cfg, 2)
    m = _masks(x, cfg.n_max)
    ta = runner.TreeAttention(x["Q"], x["K"], x["V"], x["prefix_len"], x["n_nodes"], m,
                              x["scale"])
    outs = []
    for _ in range(3):
        ta.run()
        torch.cuda.synchronize()
        outs.append(ta.output())
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_round_then_attention(gpu_lib):
    """A GPU round's own mask and n_nodes feed the attention call; the
    oracle attends over the oracle's tree of the same round, which must be
    identical."""
    from conditional_draft_tree_depth_amd import runner
    from gpu_util import caps_for
    from checker import compare_request
    from oracle import dtree_oracle as O
    import torch
    cfg = synth.CONFIGS["qwen3_4b"]
    xr = synth.make_inputs(cfg, 0)
    wd, H, root = runner.to_device(xr)
    rnd = runner.Round(wd, cfg.wtype, caps_for(cfg), cfg.batch, cfg.D, cfg.M, cfg.K, cfg.W,
                       cfg.B, cfg.beta)
    try:
        rnd.run(H, root)
        torch.cuda.synchronize()
        prep = O.prepare_round(xr, cfg.D)
        prm = dict(D=cfg.D, M=cfg.M, K=cfg.K, W=cfg.W, B=cfg.B, beta=cfg.beta)
        res = compare_request(rnd.outputs()[0], rnd.trace(0), prep, 0, prm)
        assert res["exact"], res
        orc = O.build_request(prep, 0, cfg.D, cfg.M, cfg.K, cfg.W, cfg.B, cfg.beta)
        acfg = synth.ATTN_CONFIGS["attn_qwen3_4b"]
        x = synth.make_attn_inputs(acfg, 0)
        x["n_nodes"] = np.array([orc["n_nodes"]], np.int32)
        ta = runner.TreeAttention(x["Q"], x["K"], x["V"], x["prefix_len"], rnd.n_nodes,
                                  rnd.mask, x["scale"])
        ta.run()
        torch.cuda.synchronize()
        _check(ta.output(), x, orc["mask"][None], "round -> attention")
    finally:
        rnd.close()
