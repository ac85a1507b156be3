"""Pins of the tree-attention oracle (CPU).

Tree attention is defined by the tree, not by the mask: every tree token is
a causal sequence of its own -- the verified prefix followed by the tokens on
its root-to-node path ("Resumen Técnico: DominoTree", Componentes
Principales 5).  The oracle takes the mask; these pins rebuild each node's
sequence by walking parent pointers and run torch's own attention routine
on it, so a transposed mask, a wrong head mapping, a dropped prefix or a
wrong scale fails here."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synth
from oracle import dtree_oracle as O
from oracle import tree_attention as TA


def _inputs(name="attn_tiny", seed=0, **over):
    cfg = synth.ATTN_CONFIGS[name].with_(**over) if over else synth.ATTN_CONFIGS[name]
    x = synth.make_attn_inputs(cfg, seed)
    masks = np.stack([TA.ancestor_mask(x["parent"][q], int(x["n_nodes"][q]), cfg.n_max)
                      for q in range(cfg.batch)])
    return cfg, x, masks


def _f64(bits):
    return torch.from_numpy(np.asarray(bits, np.uint16).astype(np.int16)).view(
        torch.bfloat16).to(torch.float64)


def _path(parent, i):
    out = []
    while i >= 0:
        out.append(i)
        i = int(parent[i]) if i > 0 else -1
    return out[::-1]


def _sdpa_per_path(x, q, i):
    """torch SDPA of tree token i over prefix + its root-to-node path."""
    P = int(x["prefix_len"][q])
    idx = list(range(P)) + [P + j for j in _path(x["parent"][q], i)]
    Qt = _f64(x["Q"][q, i])[None, :, None, :]                 # [1, Hq, 1, dh]
    Kt = _f64(x["K"][q][:, idx, :])[None]                     # [1, Hkv, len, dh]
    Vt = _f64(x["V"][q][:, idx, :])[None]
    o = F.scaled_dot_product_attention(Qt, Kt, Vt, scale=x["scale"], enable_gqa=True)
    return o[0, :, 0, :].numpy()                              # [Hq, dh]


@pytest.mark.parametrize("name,over", [
    ("attn_tiny", {}),
    ("attn_tiny", {"shape": "recursive"}),
    ("attn_tiny", {"shape": "chain"}),
    ("attn_tiny", {"prefix": (0, 3), "n_nodes": (17, 1)}),        # no prefix; root only
    ("attn_tiny", {"Hq": 8, "Hkv": 1, "dh": 128}),                 # G = 8
    ("attn_tiny", {"Hq": 3, "Hkv": 3, "n_max": 9, "n_nodes": (9, 4)}),   # G = 1
])
def test_oracle_matches_sdpa_per_path(name, over):
    cfg, x, masks = _inputs(name, 3, **over)
    Ox, _ = TA.tree_attention(x["Q"], x["K"], x["V"], x["prefix_len"], x["n_nodes"], masks,
                              x["scale"])
    for q in range(cfg.batch):
        n = int(x["n_nodes"][q])
        for i in range(n):
            np.testing.assert_allclose(Ox[q, i], _sdpa_per_path(x, q, i), rtol=0, atol=1e-12)
        assert not Ox[q, n:].any()


def test_chain_last_token_sees_everything():
    cfg, x, masks = _inputs("attn_tiny", 1, shape="chain")
    Ox, _ = TA.tree_attention(x["Q"], x["K"], x["V"], x["prefix_len"], x["n_nodes"], masks,
                              x["scale"])
    for q in range(cfg.batch):
        L = int(x["prefix_len"][q] + x["n_nodes"][q])
        i = int(x["n_nodes"][q]) - 1
        Qt = _f64(x["Q"][q, i])[None, :, None, :]
        o = F.scaled_dot_product_attention(Qt, _f64(x["K"][q][:, :L])[None],
                                           _f64(x["V"][q][:, :L])[None], scale=x["scale"],
                                           enable_gqa=True)
        np.testing.assert_allclose(Ox[q, i], o[0, :, 0].numpy(), rtol=0, atol=1e-12)


def test_equal_keys_give_the_mean_of_visible_values():
    cfg, x, masks = _inputs("attn_tiny", 2)
    K0 = np.zeros_like(x["K"])        # all logits 0: uniform weights
    Ox, absw = TA.tree_attention(x["Q"], K0, x["V"], x["prefix_len"], x["n_nodes"], masks,
                                 x["scale"])
    V = _f64(x["V"]).numpy()
    G = cfg.Hq // cfg.Hkv
    for q in range(cfg.batch):
        P = int(x["prefix_len"][q])
        for i in range(int(x["n_nodes"][q])):
            path = _path(x["parent"][q], i)
            for h in range(cfg.Hq):
                rows = np.concatenate([V[q, h // G, :P], V[q, h // G, [P + j for j in path]]])
                np.testing.assert_allclose(Ox[q, i, h], rows.mean(0), atol=1e-13)
                np.testing.assert_allclose(absw[q, i, h], np.abs(rows).mean(0), atol=1e-13)


def test_invisible_positions_do_not_matter():
    """Changing K/V at tree positions off node i's path, and every cache slot
    past the tree, leaves node i's output unchanged."""
    cfg, x, masks = _inputs("attn_tiny", 4, shape="recursive")
    Ox, _ = TA.tree_attention(x["Q"], x["K"], x["V"], x["prefix_len"], x["n_nodes"], masks,
                              x["scale"])
    q, i = 0, int(x["n_nodes"][0]) - 1
    P, n = int(x["prefix_len"][q]), int(x["n_nodes"][q])
    off = [P + j for j in range(n) if j not in _path(x["parent"][q], i)]
    off += list(range(P + n, x["L_cap"]))
    K2, V2 = x["K"].copy(), x["V"].copy()
    rng = np.random.default_rng(0)
    K2[q][:, off] = rng.integers(0, 0x7F00, K2[q][:, off].shape).astype(np.uint16)
    V2[q][:, off] = rng.integers(0, 0x7F00, V2[q][:, off].shape).astype(np.uint16)
    O2, _ = TA.tree_attention(x["Q"], K2, V2, x["prefix_len"], x["n_nodes"], masks, x["scale"])
    np.testing.assert_array_equal(O2[q, i], Ox[q, i])


def test_ancestor_mask_is_the_reachability_closure():
    rng = np.random.default_rng(5)
    for shape in ("levels", "recursive", "chain"):
        for n in (1, 2, 7, 33):
            par = synth.random_parents(40, n, rng, shape)
            m = TA.ancestor_mask(par, n, 40).astype(np.int64)
            # reach = I + A + A^2 + ..., A[i, p] = 1 when p is i's parent
            A = np.zeros((40, 40), np.int64)
            for i in range(1, n):
                A[i, par[i]] = 1
            reach = np.eye(40, dtype=np.int64)
            reach[n:, n:] = 0
            step = reach.copy()
            for _ in range(n):
                step = (step @ A > 0).astype(np.int64)
                reach |= step
            assert np.array_equal(m, reach)


def test_ancestor_mask_agrees_with_the_emitted_tree():
    """The attention oracle's mask and the round oracle's emitted mask are
    the same relation on built trees."""
    cfg = synth.CONFIGS["tiny"]
    for seed in range(4):
        for out in O.build_round(synth.make_inputs(cfg, seed), cfg.D, cfg.M, cfg.K, cfg.W,
                                 cfg.B, cfg.beta):
            m = TA.ancestor_mask(out["parent"], out["n_nodes"], cfg.B + 1)
            assert np.array_equal(m, out["mask"])


def test_bad_lengths_are_rejected():
    cfg, x, masks = _inputs("attn_tiny", 0)
    with pytest.raises(ValueError):
        TA.tree_attention(x["Q"], x["K"], x["V"], np.array([5, x["L_cap"]], np.int32),
                          x["n_nodes"], masks, x["scale"])
    with pytest.raises(ValueError):
        TA.ancestor_mask(np.array([-1, 2, 0], np.int32), 3, 3)
