"""The parity checker on the CPU: rounds shaped like the library's outputs
and debug trace are made from oracle runs, and the checker must accept the
oracle's own round, accept an admissible alternative at an exact tie (and
compare that tree to its last node), and reject rounds from an oracle with
a mistake planted in it."""
import numpy as np
import pytest

import synth
import fixtures_io
from oracle import dtree_oracle as O
from checker import compare_request, Mismatch


def as_gpu(res, p):
    """A request's oracle result in the layout of the library's outputs and
    trace (nodes in the oracle's own order; the checker matches by path)."""
    sa = res["sa"]
    D, W, B = p["D"], p["W"], p["B"]
    surv = np.full((D + 1, W), -1, np.int32)
    surv[0, 0] = 0
    for dd, pdp in enumerate(sa["per_depth"]):
        surv[dd + 1, :len(pdp["survivors"])] = pdp["survivors"]
    sel = np.full(B, -1, np.int32)
    sel[:len(res["sel"])] = res["sel"]
    C = np.asarray(sa["C"], np.int32)
    Cl = np.array([[res["Lb"][dd][t] for t in C[dd]] for dd in range(D)], np.float32)
    gout = {k: np.array(res[k]) for k in ("tok", "parent", "depth", "score", "mask")}
    gout["n_nodes"] = res["n_nodes"]
    gtr = dict(C=C, Cl=Cl, node_tok=np.asarray(sa["tok"], np.int32),
               node_parent=np.asarray(sa["parent"], np.int32),
               node_score=np.asarray(sa["score"], np.float32), surv=surv, sel=sel,
               n_sa=len(sa["tok"]), status=0)
    return gout, gtr


def _prm(cfg):
    return dict(D=cfg.D, M=cfg.M, K=cfg.K, W=cfg.W, B=cfg.B, beta=cfg.beta)


@pytest.mark.parametrize("seed", range(6))
def test_oracle_round_is_exact(seed):
    cfg = synth.CONFIGS["tiny"]
    x = synth.make_inputs(cfg, seed)
    prep = O.prepare_round(x, cfg.D)
    res = O.build_request(prep, 0, cfg.D, cfg.M, cfg.K, cfg.W, cfg.B, cfg.beta)
    r = compare_request(*as_gpu(res, _prm(cfg)), prep, 0, _prm(cfg))
    assert r["exact"] and r["nodes"] == res["n_nodes"]


def test_admissible_alternative_is_followed_to_the_last_node():
    g, x, exp = fixtures_io.load("width_tie")
    p = g["params"]
    prep = O.prepare_round(x, p["D"])
    a = O.build_request(prep, 0, p["D"], p["M"], p["K"], p["W"], p["B"], p["beta"])
    k, d = next((k, d) for k, d in a["sa"]["decisions"].items() if d["ambiguous"] and k[0] == "W")
    spare = sorted(d["band"] - d["default"])[0]
    drop = sorted(d["default"] - d["sure"])[0]
    other = (set(d["default"]) - {drop}) | {spare}
    b = O.build_request(prep, 0, p["D"], p["M"], p["K"], p["W"], p["B"], p["beta"],
                        script={k: other}, check_heap=False)
    r = compare_request(*as_gpu(b, p), prep, 0, p)
    assert not r["exact"] and [t["stage"] for t in r["ties"]] == ["W"]
    assert r["nodes"] == b["n_nodes"]
    # the same alternative with one planted score error is still caught
    gout, gtr = as_gpu(b, p)
    gtr["node_score"] = gtr["node_score"].copy()
    last = len(gtr["node_score"]) - 1
    gtr["node_score"][last] -= np.float32(1e-3)
    with pytest.raises(Mismatch):
        compare_request(gout, gtr, prep, 0, p)


def test_planted_mistakes_are_rejected():
    cfg = synth.CONFIGS["tiny"]
    caught = 0
    for seed in range(6):
        x = synth.make_inputs(cfg, seed)
        prep = O.prepare_round(x, cfg.D)
        # (1) a wrong depth bonus in the oracle that made the "GPU" round
        bad = O.build_request(prep, 0, cfg.D, cfg.M, cfg.K, cfg.W, cfg.B, -3.0)
        good = O.build_request(prep, 0, cfg.D, cfg.M, cfg.K, cfg.W, cfg.B, cfg.beta)
        if set(bad["sel"]) != set(good["sel"]):
            with pytest.raises(Mismatch):
                compare_request(*as_gpu(bad, _prm(cfg)), prep, 0, _prm(cfg))
            caught += 1
        # (2) a perturbed correction weight: path scores move by more than 1e-4
        x2 = synth.make_inputs(cfg, seed)
        x2["weights"]["W2"] = x2["weights"]["W2"] * np.float32(1.01)
        prep2 = O.prepare_round(x2, cfg.D)
        res2 = O.build_request(prep2, 0, cfg.D, cfg.M, cfg.K, cfg.W, cfg.B, cfg.beta)
        with pytest.raises(Mismatch):
            compare_request(*as_gpu(res2, _prm(cfg)), prep, 0, _prm(cfg))
        caught += 1
        # (3) a swapped GRU gate order in the drafter the "GPU" ran
        x3 = synth.make_inputs(cfg, seed)
        s = cfg.s
        Wih = x3["weights"]["W_ih"].copy()
        x3["weights"]["W_ih"] = np.concatenate([Wih[s:2 * s], Wih[:s], Wih[2 * s:]])
        prep3 = O.prepare_round(x3, cfg.D)
        res3 = O.build_request(prep3, 0, cfg.D, cfg.M, cfg.K, cfg.W, cfg.B, cfg.beta)
        with pytest.raises(Mismatch):
            compare_request(*as_gpu(res3, _prm(cfg)), prep, 0, _prm(cfg))
        caught += 1
    assert caught >= 13


# ---------------------------------------------------------------------------
# the heap builder's checker
# ---------------------------------------------------------------------------
def heap_as_gpu(res, p):
    sa = res["sa"]
    D, B = p["D"], p["B"]
    sel = np.full(B, -1, np.int32)
    sel[:len(res["sel"])] = res["sel"]
    C = np.asarray(sa["C"], np.int32)
    Cl = np.array([[res["Lb"][dd][t] for t in C[dd]] for dd in range(D)], np.float32)
    gout = {k: np.array(res[k]) for k in ("tok", "parent", "depth", "score", "mask")}
    gout["n_nodes"] = res["n_nodes"]
    gtr = dict(C=C, Cl=Cl, node_tok=np.asarray(sa["tok"], np.int32),
               node_parent=np.asarray(sa["parent"], np.int32),
               node_score=np.asarray(sa["score"], np.float32), sel=sel,
               n_sa=len(sa["tok"]), status=0)
    return gout, gtr


@pytest.mark.parametrize("seed", range(6))
def test_heap_oracle_round_is_exact(seed):
    from checker import compare_heap_request
    cfg = synth.CONFIGS["tiny"]
    x = synth.make_inputs(cfg, seed)
    prep = O.prepare_round(x, cfg.D)
    res = O.build_heap_tree(prep, 0, cfg.D, cfg.M, cfg.K, cfg.B, cfg.beta)
    r = compare_heap_request(*heap_as_gpu(res, _prm(cfg)), prep, 0, _prm(cfg))
    assert r["exact"] and r["nodes"] == res["n_nodes"]


def test_heap_pop_alternative_is_followed():
    """An exact key tie at the last pop: the other admissible pop set is
    followed by the oracle and compared to its last node."""
    from checker import compare_heap_request
    cfg = synth.custom_config(cfg_id=1500, D=3, M=4, K=2, B=3, beta=0.0)
    # equal base logits everywhere and no correction: every child of a node
    # has the same log-prob, so the pop cutoff is a tie
    x = synth.make_inputs(cfg, 0)
    x["weights"]["W_lm"] = np.zeros_like(x["weights"]["W_lm"])
    x["weights"]["bias"] = np.zeros_like(x["weights"]["bias"])
    x["weights"]["W2"] = np.zeros_like(x["weights"]["W2"])
    prep = O.prepare_round(x, cfg.D)
    p = _prm(cfg)
    a = O.build_heap_tree(prep, 0, cfg.D, cfg.M, cfg.K, cfg.B, cfg.beta)
    d = a["sa"]["decisions"][("P",)]
    assert d["ambiguous"]
    # a closed alternative: swap one popped leaf for a tied unpopped sibling
    pops = {a["sa"]["path"][n] for n in a["sel"]}
    leaf = max(pops, key=lambda pth: (len(pth), pth))
    spare = next(pth for pth in sorted(d["band"] - pops) if pth[:-1] in pops | {()}
                 and len(pth) == len(leaf))
    alt = (pops - {leaf}) | {spare}
    b = O.build_heap_tree(prep, 0, cfg.D, cfg.M, cfg.K, cfg.B, cfg.beta, script={("P",): alt})
    r = compare_heap_request(*heap_as_gpu(b, p), prep, 0, p)
    assert not r["exact"] and [t["stage"] for t in r["ties"]] == ["P"]
    assert {b["sa"]["path"][n] for n in b["sel"]} == alt


def test_heap_planted_mistakes_are_rejected():
    from checker import compare_heap_request
    cfg = synth.CONFIGS["tiny"]
    for seed in range(4):
        x = synth.make_inputs(cfg, seed)
        prep = O.prepare_round(x, cfg.D)
        p = _prm(cfg)
        # the depth-wise round is not the heap round (and vice versa for a
        # perturbed drafter)
        x2 = synth.make_inputs(cfg, seed)
        x2["weights"]["W2"] = x2["weights"]["W2"] * np.float32(1.01)
        res2 = O.build_heap_tree(O.prepare_round(x2, cfg.D), 0, cfg.D, cfg.M, cfg.K, cfg.B,
                                 cfg.beta)
        with pytest.raises(Mismatch):
            compare_heap_request(*heap_as_gpu(res2, p), prep, 0, p)
        # Markov scoring instead of conditional
        res3 = O.build_heap_tree(prep, 0, cfg.D, cfg.M, cfg.K, cfg.B, cfg.beta, scoring="markov")
        with pytest.raises(Mismatch):
            compare_heap_request(*heap_as_gpu(res3, p), prep, 0, p)
