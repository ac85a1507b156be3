"""Pins of the CPU oracle against facts fixed outside it (CPU only).

Each test checks the oracle against something it does not compute itself:
a library routine the step reduces to, an independent brute-force walk over
every token path, the hand-worked fixtures, the set equality of Lemma 1
(DARTree page, Metodología 2), closed-form special cases, and invariants.
"""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import dtree_oracle as O
from brute import Brute
import fixtures_io


def _run(inputs, cfg, store="f32", **over):
    p = dict(D=cfg.D, M=cfg.M, K=cfg.K, W=cfg.W, B=cfg.B, beta=cfg.beta)
    p.update(over)
    return O.build_round(inputs, store=store, **p)


def _rand_tiny(seed, wtype="f32"):
    rng = np.random.default_rng(seed)
    M = int(rng.integers(2, 7))
    D = int(rng.integers(1, 5))
    K = int(rng.integers(1, M + 1))
    W = int(rng.integers(1, 9))
    V = int(rng.integers(max(M, 8), 65))
    cfg = synth.custom_config(cfg_id=2000 + seed, d=16, V=V, e=8, s=8, r=4, D=D, M=M,
                              K=K, W=W, B=int(rng.integers(1, 40)),
                              beta=float(rng.choice([0.0, -0.05, -0.5])), wtype=wtype)
    return cfg, synth.make_inputs(cfg, seed)


# ---------------------------------------------------------------- formats
def test_bf16_round_matches_torch_cast():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * np.float32(3.0),
        # exact halfway cases: 1 + 2^-8 and 1 + 3*2^-8 (ties to even), negatives
        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 0.0, -0.0,
                  1e-40, -1e-40, 3.0e38, 65504.0], dtype=np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    got = O.bf16_round(x)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_decode_bf16_bits():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0000, 0x8000], dtype=np.uint16)
    assert O.decode(bits, "bf16").tolist() == [1.0, -1.0, 3.140625, 0.0, -0.0]


# ---------------------------------------------------------------- single steps
def test_base_logits_vs_torch_matmul():
    cfg = synth.custom_config(cfg_id=3000, d=256, V=1000, e=8, s=8, r=4, wtype="bf16")
    x = synth.make_inputs(cfg, 1)
    Hq = O.bf16_round(x["H"][0])
    got = O.base_logits(Hq, x["weights"], "bf16", chunk=300)
    W = torch.from_numpy(x["weights"]["W_lm"]).view(torch.bfloat16).to(torch.float64)
    ref = torch.from_numpy(Hq).to(torch.float64) @ W.T + torch.from_numpy(x["weights"]["bias"]).double()
    assert np.max(np.abs(got - ref.numpy())) < 1e-6


def test_top_m_ties_by_token():
    row = np.array([0.5, 2.0, 0.5, 2.0, -1.0, 0.5], dtype=np.float64)
    toks, vals = O.top_m(row, 4)
    assert toks.tolist() == [1, 3, 0, 2]
    ref = sorted(range(6), key=lambda v: (-row[v], v))[:4]
    assert toks.tolist() == ref
    assert vals.tolist() == [2.0, 2.0, 0.5, 0.5]


def test_gru_cell_vs_torch_grucell():
    cfg = synth.custom_config(cfg_id=3001, e=24, s=40)
    x = synth.make_inputs(cfg, 2)
    W = O.OracleWeights(x["weights"], "f32", cfg.d, cfg.s)
    rng = np.random.default_rng(0)
    xin = rng.standard_normal((5, 24))
    h = rng.standard_normal((5, 40)) * 0.3
    got = O.gru_cell(xin, h, W, store="f64")
    g = torch.nn.GRUCell(24, 40, dtype=torch.float64)
    with torch.no_grad():
        g.weight_ih.copy_(torch.from_numpy(W.W_ih))
        g.weight_hh.copy_(torch.from_numpy(W.W_hh))
        g.bias_ih.copy_(torch.from_numpy(W.b_ih))
        g.bias_hh.copy_(torch.from_numpy(W.b_hh))
        ref = g(torch.from_numpy(xin), torch.from_numpy(h)).numpy()
    assert np.max(np.abs(got - ref)) < 1e-12


def test_log_softmax_properties():
    rng = np.random.default_rng(1)
    ell = rng.standard_normal((7, 33)) * 5
    lp = O.log_softmax(ell, store="f64")
    ref = torch.log_softmax(torch.from_numpy(ell), dim=1).numpy()
    assert np.max(np.abs(lp - ref)) < 1e-12
    assert np.all(np.abs(np.exp(lp).sum(1) - 1) < 1e-12)
    lp32 = O.log_softmax(ell.astype(np.float32).astype(np.float64))
    assert np.all(lp32 <= 0.0)


# ---------------------------------------------------------------- brute force
def _check_against_brute(inputs, cfg, req=0):
    res = _run(inputs, cfg, store="f64")[req]
    sa = res["sa"]
    bf = Brute(inputs, req, cfg.D, cfg.M)
    allp = bf.enumerate()
    # candidates per depth
    assert [list(c) for c in sa["C"]] == [list(c) for c in bf.C]
    # every superarbol node's score, recomputed from scratch along its path
    for n in range(1, len(sa["tok"])):
        assert abs(sa["score"][n] - allp[sa["path"][n]]) < 1e-10
    # children of expanded nodes are the Top-K of their M extensions,
    # survivors are the Top-W of each depth's children
    for dd, pdp in enumerate(sa["per_depth"]):
        for p in pdp["frontier"]:
            ext, base = bf.extensions(sa["path"][p])
            want = sorted(ext, key=lambda t: (-ext[t], t))[:cfg.K]
            got = [sa["tok"][c] for c in sa["kids"][p]]
            assert got == want
        ch = pdp["children"]
        want = sorted(ch, key=lambda n: (-allp[sa["path"][n]], sa["path"][n]))[:cfg.W]
        assert set(want) == set(pdp["survivors"])
    return res


@pytest.mark.parametrize("seed", range(6))
def test_oracle_vs_brute_force_tiny(seed):
    cfg = synth.CONFIGS["tiny"]
    _check_against_brute(synth.make_inputs(cfg, seed), cfg)


@pytest.mark.parametrize("seed", range(24))
def test_oracle_vs_brute_force_random_shapes(seed):
    cfg, x = _rand_tiny(seed, "bf16" if seed % 2 else "f32")
    _check_against_brute(x, cfg)


def test_f32_storage_close_to_f64():
    cfg = synth.CONFIGS["tiny"]
    for seed in range(5):
        x = synth.make_inputs(cfg, seed)
        a = _run(x, cfg, store="f32")[0]["sa"]
        b = _run(x, cfg, store="f64")[0]["sa"]
        pa = dict(zip(a["path"], a["score"]))
        pb = dict(zip(b["path"], b["score"]))
        common = set(pa) & set(pb)
        assert len(common) > len(pa) // 2
        assert max(abs(pa[k] - pb[k]) for k in common) < 1e-5


# ---------------------------------------------------------------- Lemma 1
BETAS = [0.0, -0.01, -0.1, -1.0, -10.0]


def test_lemma1_heap_equals_global_top_b_many_seeds():
    cfg = synth.CONFIGS["tiny"]
    n = 0
    for seed in range(1000):
        x = synth.make_inputs(cfg, seed)
        res = _run(x, cfg, check_heap=False)[0]
        sa = res["sa"]
        for beta in BETAS:
            for B in (5, cfg.B, len(sa["tok"]) - 1):
                sel = O.select_global_top_b(sa, B, beta)
                pops = O.select_literal_heap(sa, B, beta)
                assert set(sel) == set(pops), (seed, beta, B)
                O.emit_tree(sa, sel, B)   # raises unless ancestor-closed
                n += 1
    assert n == 1000 * len(BETAS) * 3


def test_lemma1_negative_control_positive_beta():
    """With beta > 0 deeper nodes are favoured: the heap (which can only pop
    what it has reached) and the global Top-B must part ways on some seed."""
    cfg = synth.CONFIGS["tiny"]
    differ = not_closed = 0
    for seed in range(200):
        sa = _run(synth.make_inputs(cfg, seed), cfg, check_heap=False)[0]["sa"]
        sel = O.select_global_top_b(sa, 8, 2.0)
        pops = O.select_literal_heap(sa, 8, 2.0)
        differ += set(sel) != set(pops)
        chosen = set(sel)
        not_closed += any(sa["parent"][n] not in chosen and sa["parent"][n] != 0 for n in sel)
    assert differ > 0 and not_closed > 0


# ---------------------------------------------------------------- special cases
def test_chain_special_case_is_greedy_corrected_path():
    """K = W = 1: a single chain, the greedy argmax of the corrected
    log-probs at each depth (Domino's single-chain drafting)."""
    for seed in range(8):
        cfg = synth.CONFIGS["tiny"].with_(K=1, W=1)
        x = synth.make_inputs(cfg, seed)
        res = _run(x, cfg, store="f64")[0]
        assert res["n_nodes"] == min(cfg.B, cfg.D) + 1
        bf = Brute(x, 0, cfg.D, cfg.M)
        path = ()
        for dd in range(cfg.D):
            ext, _ = bf.extensions(path)
            path = path + (min(ext, key=lambda t: (-ext[t], t)),)
        assert res["tok"][1:cfg.D + 1].tolist() == list(path)
        assert res["parent"][1:cfg.D + 1].tolist() == list(range(cfg.D))


def test_unpruned_tree_equals_top_b_over_all_paths():
    """K = M and W >= M^(D-1): nothing is pruned, so the output is the Top-B
    over every token path, found by brute force (DominoTree's unpruned
    best-first tree)."""
    for seed in range(6):
        cfg = synth.custom_config(cfg_id=4000, d=16, V=40, e=8, s=8, r=4, D=3, M=4, K=4,
                                  W=16, B=20, beta=-0.2)
        x = synth.make_inputs(cfg, seed)
        res = _run(x, cfg, store="f64")[0]
        allp = Brute(x, 0, cfg.D, cfg.M).enumerate()
        assert len(res["sa"]["tok"]) - 1 == len(allp) == 4 + 16 + 64
        ranked = sorted(allp, key=lambda p: (-(allp[p] + cfg.beta * len(p)), len(p), p))
        want = set(ranked[:cfg.B])
        sa = res["sa"]
        got = {sa["path"][n] for n in res["sel"]}
        assert got == want


def test_zero_correction_factorises():
    """W2 = 0: the scores no longer depend on the path (a marginal tree):
    every branch at a depth gets the same children and log-probs."""
    cfg = synth.CONFIGS["tiny"]
    x = synth.make_inputs(cfg, 3)
    x["weights"]["W2"] = np.zeros_like(x["weights"]["W2"])
    sa = _run(x, cfg, store="f64")[0]["sa"]
    for dd, pdp in enumerate(sa["per_depth"]):
        kids = [[sa["tok"][c] for c in sa["kids"][p]] for p in pdp["frontier"]]
        assert all(k == kids[0] for k in kids)
        assert np.allclose(pdp["lp"], pdp["lp"][0:1], atol=0, rtol=0)
        lpm = O.log_softmax(sa["Cl"][dd][None, :], store="f64")[0]
        for p in pdp["frontier"]:
            for c in sa["kids"][p]:
                j = list(sa["C"][dd]).index(sa["tok"][c])
                assert abs(sa["score"][c] - sa["score"][p] - lpm[j]) < 1e-12


def test_very_negative_beta_selects_layer_by_layer():
    cfg = synth.CONFIGS["tiny"]
    for seed in range(10):
        sa = _run(synth.make_inputs(cfg, seed), cfg, check_heap=False)[0]["sa"]
        for B in (3, 7, 12):
            sel = O.select_global_top_b(sa, B, -1e4)
            depths = [sa["depth"][n] for n in sel]
            assert depths == sorted(depths)
            dmax = max(depths)
            n_shallower = sum(1 for dd in sa["depth"][1:] if dd < dmax)
            assert sum(1 for dd in depths if dd < dmax) == n_shallower


def test_budget_equal_superarbol_selects_everything():
    cfg = synth.CONFIGS["tiny"]
    x = synth.make_inputs(cfg, 4)
    res = _run(x, cfg, B=22)[0]
    assert res["n_nodes"] == 23 and len(res["sa"]["tok"]) == 23
    res = _run(x, cfg, B=40)[0]          # more budget than nodes
    assert res["n_nodes"] == 23
    assert np.all(res["tok"][23:] == -1) and np.all(np.isneginf(res["score"][23:]))


# ---------------------------------------------------------------- outputs
def check_output_invariants(out, B, C=None):
    n = out["n_nodes"]
    tok, par, dep, mask = out["tok"], out["parent"], out["depth"], out["mask"]
    assert par[0] == -1 and dep[0] == 0 and out["score"][0] == 0
    for i in range(1, n):
        assert 0 <= par[i] < i
        assert dep[i] == dep[par[i]] + 1
        assert out["score"][i] <= out["score"][par[i]]
        want = mask[par[i]].copy()
        want[i] = 1
        assert np.array_equal(mask[i], want)
        if C is not None:
            assert tok[i] in set(C[dep[i] - 1].tolist())
    assert np.array_equal(mask[:n].sum(1), dep[:n] + 1)
    assert not mask[n:].any() and not mask[:, n:].any()
    sib = {}
    for i in range(1, n):
        sib.setdefault(par[i], []).append(tok[i])
    assert all(len(v) == len(set(v)) for v in sib.values())
    # canonical order: depth, then parent index, then token
    keys = [(dep[i], par[i], tok[i]) for i in range(1, n)]
    assert keys == sorted(keys)


@pytest.mark.parametrize("seed", range(10))
def test_output_invariants(seed):
    cfg = synth.CONFIGS["tiny"]
    out = _run(synth.make_inputs(cfg, seed), cfg)[0]
    check_output_invariants(out, cfg.B, out["sa"]["C"])


# ---------------------------------------------------------------- hand-worked
@pytest.mark.parametrize("name", fixtures_io.fixture_names())
def test_golden_fixture(name):
    g, x, exp = fixtures_io.load(name)
    p = g["params"]
    out = O.build_round(x, **p)[0]
    assert out["n_nodes"] == exp["n_nodes"]
    n = exp["n_nodes"]
    assert out["tok"][:n].tolist() == exp["tok"]
    assert out["parent"][:n].tolist() == exp["parent"]
    assert out["depth"][:n].tolist() == exp["depth"]
    assert np.max(np.abs(out["score"][:n] - np.array(exp["score"]))) < g["score_tol"]
    assert out["mask"][:n, :n].tolist() == exp["mask"]


# ------------------------------------------------------- marginal scoring
def _check_marginal(x, cfg):
    res = _run(x, cfg, store="f64", scoring="marginal")[0]
    sa = res["sa"]
    bf = Brute(x, 0, cfg.D, cfg.M)
    allp = bf.enumerate_marginal()
    assert [list(c) for c in sa["C"]] == [list(c) for c in bf.C]
    for n in range(1, len(sa["tok"])):
        assert abs(sa["score"][n] - allp[sa["path"][n]]) < 1e-10
    for dd, pdp in enumerate(sa["per_depth"]):
        lp = torch.log_softmax(bf.Lb[dd][bf.C[dd]], dim=0).tolist()
        want = [t for _, t in sorted(zip(lp, bf.C[dd]), key=lambda z: (-z[0], z[1]))[:cfg.K]]
        for p in pdp["frontier"]:
            assert [sa["tok"][c] for c in sa["kids"][p]] == want
        ch = pdp["children"]
        surv = sorted(ch, key=lambda n: (-allp[sa["path"][n]], sa["path"][n]))[:cfg.W]
        assert set(surv) == set(pdp["survivors"])
    return res


@pytest.mark.parametrize("seed", range(4))
def test_marginal_scoring_tiny(seed):
    """Marginal (uncorrected) scoring: every node's score is the closed form
    sum of the per-depth log-softmax of the base logits at its tokens, every
    branch of a depth gets the same Top-K children, survivors are the Top-W."""
    cfg = synth.CONFIGS["tiny"]
    _check_marginal(synth.make_inputs(cfg, seed), cfg)


@pytest.mark.parametrize("seed", range(12))
def test_marginal_scoring_random_shapes(seed):
    cfg, x = _rand_tiny(100 + seed, "bf16" if seed % 2 else "f32")
    _check_marginal(x, cfg)


def test_marginal_equals_zero_correction():
    """Marginal scoring builds the same tree as conditional scoring with a
    zero correction head (W2 = 0 makes Delta L vanish on every path)."""
    for seed in range(4):
        cfg = synth.CONFIGS["tiny"]
        x = synth.make_inputs(cfg, seed)
        a = _run(x, cfg, store="f64", scoring="marginal")[0]
        x["weights"]["W2"] = np.zeros_like(x["weights"]["W2"])
        b = _run(x, cfg, store="f64")[0]
        for k in ("tok", "parent", "depth"):
            assert list(a[k]) == list(b[k])
        assert np.max(np.abs(np.asarray(a["score"]) - np.asarray(b["score"]))) < 1e-12
        assert np.array_equal(a["mask"], b["mask"])


def test_marginal_unpruned_top_b_over_all_paths():
    """K = M, W >= M^(D-1) with marginal scoring: the Top-B over all token
    paths by the closed-form marginal score (DDTree's best-first tree)."""
    for seed in range(4):
        cfg = synth.custom_config(cfg_id=4100, d=16, V=40, e=8, s=8, r=4, D=3, M=4, K=4,
                                  W=16, B=20, beta=-0.2)
        x = synth.make_inputs(cfg, seed)
        res = _run(x, cfg, store="f64", scoring="marginal")[0]
        allp = Brute(x, 0, cfg.D, cfg.M).enumerate_marginal()
        ranked = sorted(allp, key=lambda p: (-(allp[p] + cfg.beta * len(p)), len(p), p))
        sa = res["sa"]
        assert {sa["path"][n] for n in res["sel"]} == set(ranked[:cfg.B])


def test_unknown_scoring_rejected():
    cfg = synth.CONFIGS["tiny"]
    with pytest.raises(ValueError):
        _run(synth.make_inputs(cfg, 0), cfg, scoring="no_such_scoring")


# ------------------------------------------------------- Markov scoring
def _check_markov(x, cfg):
    res = _run(x, cfg, store="f64", scoring="markov")[0]
    sa = res["sa"]
    bf = Brute(x, 0, cfg.D, cfg.M)
    allp = bf.enumerate_markov()
    assert [list(c) for c in sa["C"]] == [list(c) for c in bf.C]
    for n in range(1, len(sa["tok"])):
        assert abs(sa["score"][n] - allp[sa["path"][n]]) < 1e-10
    for dd, pdp in enumerate(sa["per_depth"]):
        for p in pdp["frontier"]:
            pth = sa["path"][p]
            ext = {t: allp[pth + (t,)] - (allp[pth] if pth else 0.0) for t in bf.C[dd]}
            want = sorted(ext, key=lambda t: (-ext[t], t))[:cfg.K]
            assert [sa["tok"][c] for c in sa["kids"][p]] == want
        ch = pdp["children"]
        surv = sorted(ch, key=lambda n: (-allp[sa["path"][n]], sa["path"][n]))[:cfg.W]
        assert set(surv) == set(pdp["survivors"])
    return res


@pytest.mark.parametrize("seed", range(4))
def test_markov_scoring_tiny(seed):
    """Markov (parent-token-only) scoring: every node's score equals the sum
    over its path of log-probs recomputed by an independent enumerator that
    runs the GRU one step from a zero state on each node's last token."""
    cfg = synth.CONFIGS["tiny"]
    _check_markov(synth.make_inputs(cfg, seed), cfg)


@pytest.mark.parametrize("seed", range(10))
def test_markov_scoring_random_shapes(seed):
    cfg, x = _rand_tiny(300 + seed, "bf16" if seed % 2 else "f32")
    _check_markov(x, cfg)


def test_markov_children_depend_on_depth_and_token_only():
    """Two expanded branches of one depth ending in the same token get the
    same log-probs under Markov scoring; conditional scoring tells them
    apart (their GRU states differ)."""
    cfg = synth.custom_config(cfg_id=4200, d=16, V=12, e=8, s=8, r=4, D=3, M=3, K=3, W=9,
                              B=30, beta=0.0)
    seen = 0
    for seed in range(6):
        x = synth.make_inputs(cfg, seed)
        for scoring in ("markov", "conditional"):
            sa = _run(x, cfg, store="f64", scoring=scoring)[0]["sa"]
            pdp = sa["per_depth"][2]
            by_tok = {}
            for a, p in enumerate(pdp["frontier"]):
                by_tok.setdefault(sa["tok"][p], []).append(pdp["lp"][a])
            for rows in by_tok.values():
                for r in rows[1:]:
                    same = np.array_equal(r, rows[0])
                    assert same == (scoring == "markov")
                    seen += scoring == "markov"
    assert seen > 0


def test_markov_unpruned_top_b_over_all_paths():
    for seed in range(4):
        cfg = synth.custom_config(cfg_id=4300, d=16, V=40, e=8, s=8, r=4, D=3, M=4, K=4,
                                  W=16, B=20, beta=-0.1)
        x = synth.make_inputs(cfg, seed)
        res = _run(x, cfg, store="f64", scoring="markov")[0]
        allp = Brute(x, 0, cfg.D, cfg.M).enumerate_markov()
        ranked = sorted(allp, key=lambda p: (-(allp[p] + cfg.beta * len(p)), len(p), p))
        sa = res["sa"]
        assert {sa["path"][n] for n in res["sel"]} == set(ranked[:cfg.B])


# ------------------------------------------------ sequential best-first heap
def _heap(x, cfg, store="f64", scoring="conditional", B=None):
    prep = O.prepare_round(x, cfg.D, store)
    return O.build_heap_tree(prep, 0, cfg.D, cfg.M, cfg.K, cfg.B if B is None else B,
                             cfg.beta, scoring=scoring)


@pytest.mark.parametrize("seed", range(8))
@pytest.mark.parametrize("scoring", ["conditional", "markov"])
def test_heap_builder_vs_brute_force(seed, scoring):
    """DominoTree's best-first builder selects the Top-B (key desc, depth
    asc, path asc) of the unpruned K-ary tree in which every node's children
    are the Top-K of its M extensions; brute force rebuilds that tree with
    every score recomputed from the root."""
    cfg, x = _rand_tiny(500 + seed, "bf16" if seed % 2 else "f32")
    cfg = cfg.with_(beta=min(cfg.beta, 0.0))
    res = _heap(x, cfg, scoring=scoring)
    tree = Brute(x, 0, cfg.D, cfg.M).kary_tree(cfg.K, markov=scoring == "markov")
    ranked = sorted(tree, key=lambda p: (-(tree[p] + cfg.beta * len(p)), len(p), p))
    sa = res["sa"]
    got = [sa["path"][n] for n in res["sel"]]
    assert set(got) == set(ranked[:cfg.B])
    for n in res["sel"]:
        assert abs(sa["score"][n] - tree[sa["path"][n]]) < 1e-10
    # pops come out in the selection order itself
    assert got == ranked[:len(got)]


@pytest.mark.parametrize("seed", range(6))
def test_heap_builder_equals_unpruned_depthwise_build(seed):
    """With W >= K^(D-1) the depth-wise build prunes nothing, so by Lemma 1
    its global Top-B is the heap's pop set: same tree, same scores."""
    cfg = synth.custom_config(cfg_id=4400, d=24, V=60, e=8, s=12, r=6, D=4, M=5, K=3,
                              W=27, B=25, beta=[0.0, -0.05, -0.3][seed % 3],
                              wtype="bf16" if seed % 2 else "f32")
    x = synth.make_inputs(cfg, seed)
    a = _heap(x, cfg, store="f32")
    b = _run(x, cfg, store="f32")[0]
    for k in ("tok", "parent", "depth", "mask"):
        assert np.array_equal(a[k], b[k]), k
    assert a["n_nodes"] == b["n_nodes"]
    assert np.max(np.abs(a["score"][:a["n_nodes"]] - b["score"][:b["n_nodes"]])) < 1e-6


def test_heap_builder_chain_special_case():
    """K = 1 (one child per popped node): the heap grows the greedy corrected
    chain, the same tree as the depth-wise build with K = W = 1."""
    for seed in range(5):
        cfg = synth.CONFIGS["tiny"].with_(K=1, W=1)
        x = synth.make_inputs(cfg, seed)
        a = _heap(x, cfg, store="f64")
        b = _run(x, cfg, store="f64")[0]
        assert a["tok"].tolist() == b["tok"].tolist()
        assert a["n_nodes"] == min(cfg.B, cfg.D) + 1


# ---------------------------------------------- decisions and alternatives
def test_default_script_reproduces_the_round():
    """Scripting every decision with its own default selection changes
    nothing; with tol = 0 and no exact ties no decision is ambiguous."""
    cfg = synth.CONFIGS["tiny"]
    for seed in range(5):
        x = synth.make_inputs(cfg, seed)
        prep = O.prepare_round(x, cfg.D)
        a = O.build_request(prep, 0, cfg.D, cfg.M, cfg.K, cfg.W, cfg.B, cfg.beta, tol=0.0)
        decs = a["sa"]["decisions"]
        assert ("B",) in decs and ("W", 3) in decs and ("M", 0) in decs
        assert not any(d["ambiguous"] for d in decs.values())
        script = {k: d["default"] for k, d in decs.items()}
        b = O.build_request(prep, 0, cfg.D, cfg.M, cfg.K, cfg.W, cfg.B, cfg.beta,
                            script=script, tol=0.0)
        for k in ("tok", "parent", "depth", "score", "mask"):
            assert np.array_equal(a[k], b[k])


def test_exact_tie_alternative_is_admissible_and_builds_a_valid_tree():
    """The width-tie fixture has two children with exactly equal scores at
    the Top-W cutoff: the decision is ambiguous, the other choice is an
    admissible alternative the oracle builds itself (a different, valid
    tree), and a set outside the band is refused."""
    g, x, exp = fixtures_io.load("width_tie")
    p = g["params"]
    prep = O.prepare_round(x, p["D"])
    a = O.build_request(prep, 0, p["D"], p["M"], p["K"], p["W"], p["B"], p["beta"])
    amb = [k for k, d in a["sa"]["decisions"].items() if d["ambiguous"]]
    wkeys = [k for k in amb if k[0] == "W"]
    assert wkeys
    k = wkeys[0]
    d = a["sa"]["decisions"][k]
    alts = [X for X in _subsets(d["band"], d["n"] - len(d["sure"]))]
    assert len(alts) >= 2
    other = next(set(d["sure"]) | set(X) for X in alts
                 if set(d["sure"]) | set(X) != d["default"])
    b = O.build_request(prep, 0, p["D"], p["M"], p["K"], p["W"], p["B"], p["beta"],
                        script={k: other}, check_heap=False)
    sa = b["sa"]
    assert {sa["path"][n] for n in sa["per_depth"][k[1] - 1]["survivors"]} == other
    assert not np.array_equal(a["tok"], b["tok"]) or not np.array_equal(a["parent"], b["parent"])
    outside = set(d["default"])
    outside.discard(next(iter(outside - set(d["sure"]))))
    with pytest.raises(O.NotAdmissible):
        O.build_request(prep, 0, p["D"], p["M"], p["K"], p["W"], p["B"], p["beta"],
                        script={k: outside})


def _subsets(items, n):
    import itertools
    return [set(c) for c in itertools.combinations(sorted(items), n)]
