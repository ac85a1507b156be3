"""Compares one request's GPU round with the oracle's (tests only).

Parity rule: tree structure (tokens, parents, depths, mask, node count) must
be identical, scores within ``tol`` (1e-4 absolute, fp32 log-prob), and a
selection may differ only where the competing values are within ``tol`` of
the oracle's cutoff (the DominoTree page, Resultados Experimentales: the
method is exact except for floating-point tie-breaking).

How a near-tie is handled.  The oracle records every selection decision of
its own run (Top-M per depth, Top-K per expanded branch, Top-W per depth,
the global Top-B) with the band of items within ``tol`` of its cutoff,
computed from its own values only.  Its admissible alternatives at a
decision are the sets X with  sure <= X <= sure | band,  |X| = n.  The
checker walks the GPU's debug trace stage by stage in the order the round
makes its decisions.  At the first decision where the GPU kept a different
set, that set must be one of the oracle's admissible alternatives there;
the oracle then builds the round again along that alternative -- all of its
arithmetic its own -- and the walk restarts.  When every decision agrees,
the whole tree is compared element by element: every superarbol node's
score, the selected set, and the emitted tokens, parents, depths, mask and
scores, to the last node.  Each followed alternative is reported as a
tolerated tie with its stage and its distance from the cutoff.
"""
import numpy as np

from oracle import dtree_oracle as O


class Mismatch(AssertionError):
    pass


def _paths(tok, par):
    paths = [()] * len(tok)
    for i in range(1, len(tok)):
        p = int(par[i])
        if not 0 <= p < i:
            raise Mismatch(f"superarbol node {i} has parent {p}")
        paths[i] = paths[p] + (int(tok[i]),)
    return paths


def check_invariants(out, B, where=""):
    n = int(out["n_nodes"])
    tok, par, dep, mask, sc = out["tok"], out["parent"], out["depth"], out["mask"], out["score"]
    N = B + 1
    if not 1 <= n <= N:
        raise Mismatch(f"{where}n_nodes {n}")
    if par[0] != -1 or dep[0] != 0 or sc[0] != 0:
        raise Mismatch(f"{where}bad root row")
    for i in range(1, n):
        if not 0 <= par[i] < i or dep[i] != dep[par[i]] + 1 or not sc[i] <= sc[par[i]]:
            raise Mismatch(f"{where}node {i}: parent {par[i]} depth {dep[i]}")
        want = mask[par[i]].copy()
        want[i] = 1
        if not np.array_equal(mask[i], want):
            raise Mismatch(f"{where}mask row {i}")
    if not np.array_equal(mask[0], np.eye(N, dtype=np.uint8)[0]):
        raise Mismatch(f"{where}mask row 0")
    if mask[n:].any() or mask[:, n:].any():
        raise Mismatch(f"{where}mask outside n_nodes")
    if not (np.all(tok[n:] == -1) and np.all(par[n:] == -1) and np.all(dep[n:] == -1)
            and np.all(np.isneginf(sc[n:]))):
        raise Mismatch(f"{where}padding slots")
    keys = [(int(dep[i]), int(par[i]), int(tok[i])) for i in range(1, n)]
    if keys != sorted(keys) or len(set(keys)) != len(keys):
        raise Mismatch(f"{where}not in canonical order")


class _Gpu:
    """The GPU round of one request, indexed by token path."""

    def __init__(self, gout, gtr, B, where):
        check_invariants(gout, B, where)
        if gtr["status"] != 0:
            raise Mismatch(f"{where}device status {gtr['status']}")
        self.paths = _paths(gtr["node_tok"], gtr["node_parent"])
        if len(set(self.paths)) != len(self.paths):
            raise Mismatch(f"{where}GPU superarbol repeats a token path")
        self.id = {p: i for i, p in enumerate(self.paths)}
        self.score = {self.paths[i]: float(gtr["node_score"][i]) for i in range(1, len(self.paths))}
        self.kids = {}
        for i in range(1, len(self.paths)):
            self.kids.setdefault(self.paths[i][:-1], []).append(self.paths[i])
        self.C = [set(int(t) for t in row) for row in gtr["C"]]
        self.Cl = gtr["Cl"]
        self.Ctok = gtr["C"]
        self.surv = [{self.paths[i] for i in row if i >= 0} for row in gtr["surv"]]
        self.sel = {self.paths[int(x)] for x in gtr["sel"] if x >= 0}
        # the emitted tree must be the GPU's own selection in canonical order
        n = int(gout["n_nodes"])
        if n != len(self.sel) + 1:
            raise Mismatch(f"{where}n_nodes {n} vs {len(self.sel)} selected")
        out_paths = _paths(gout["tok"][:n], gout["parent"][:n])
        if set(out_paths[1:]) != self.sel:
            raise Mismatch(f"{where}output is not the GPU's own selection")
        for i in range(1, n):
            if gout["score"][i] != np.float32(self.score[out_paths[i]]):
                raise Mismatch(f"{where}output score differs from trace at {i}")


def _first_divergence(g, orc, prm, tol, where):
    """(decision key, GPU's set) of the first decision where the GPU kept a
    different set than the oracle's build, or None.  Values that are not
    decisions (base logits, scores) must agree within tol on the way."""
    D = prm["D"]
    sa = orc["sa"]
    Lb = orc["Lb"]
    for dd in range(D):
        for j, t in enumerate(g.Ctok[dd]):
            if abs(float(g.Cl[dd][j]) - float(Lb[dd][int(t)])) > tol:
                raise Mismatch(f"{where}base logit of token {t} at depth {dd}")
        if g.C[dd] != set(int(t) for t in sa["C"][dd]):
            return ("M", dd), g.C[dd]
    for dd in range(D):
        pdp = sa["per_depth"][dd]
        o_front = {sa["path"][i] for i in pdp["frontier"]}
        if g.surv[dd] != o_front:
            raise Mismatch(f"{where}expanded set at depth {dd} differs without a decision")
        for p in pdp["frontier"]:
            pp = sa["path"][p]
            g_k = {c[-1] for c in g.kids.get(pp, [])}
            o_k = {sa["tok"][c] for c in sa["kids"][p]}
            if g_k != o_k:
                return ("K", dd, pp), g_k
        for c in pdp["children"]:
            cp = sa["path"][c]
            if cp not in g.score:
                raise Mismatch(f"{where}GPU lacks superarbol node {cp}")
            if abs(g.score[cp] - sa["score"][c]) > tol:
                raise Mismatch(f"{where}score of {cp}: gpu {g.score[cp]} oracle {sa['score'][c]}")
        o_surv = {sa["path"][i] for i in pdp["survivors"]}
        if g.surv[dd + 1] != o_surv:
            return ("W", dd + 1), g.surv[dd + 1]
    if set(g.paths) != set(sa["path"]):
        extra = sorted(set(g.paths) ^ set(sa["path"]))[:3]
        raise Mismatch(f"{where}superarbols differ: {extra}")
    o_sel = {sa["path"][i] for i in orc["sel"]}
    if g.sel != o_sel:
        return ("B",), g.sel
    return None


def _tie_info(key, d, gset):
    diff = set(gset) ^ set(d["default"])
    return {"stage": key[0], "depth": key[1] if len(key) > 1 else None,
            "band": len(d["band"]), "swapped": len(diff) // 2}


def compare_request(gout, gtr, prep, q, prm, tol=O.TIE_TOL, where="", scoring="conditional",
                    max_ties=64):
    """gout: GPU outputs of request q; gtr: its trace; prep: the oracle's
    ``prepare_round`` of the same inputs.  Returns
    {'exact': bool, 'ties': [...], 'ambiguous': int, 'nodes': int}."""
    D, M, K, W, B, beta = prm["D"], prm["M"], prm["K"], prm["W"], prm["B"], prm["beta"]
    g = _Gpu(gout, gtr, B, where)
    script, ties = {}, []
    while True:
        orc = O.build_request(prep, q, D, M, K, W, B, beta, check_heap=not script,
                              scoring=scoring, script=script, tol=tol)
        div = _first_divergence(g, orc, prm, tol, where)
        if div is None:
            break
        key, gset = div
        d = orc["sa"]["decisions"].get(key)
        if d is None:
            raise Mismatch(f"{where}decision {key}: GPU kept {sorted(gset)[:4]}, oracle has no choice")
        if not (len(gset) == d["n"] and d["sure"] <= gset <= (d["sure"] | d["band"])):
            raise Mismatch(f"{where}decision {key} differs beyond tolerance: "
                           f"{sorted(set(gset) ^ d['default'])[:4]}")
        ties.append(_tie_info(key, d, gset))
        if len(ties) > max_ties:
            raise Mismatch(f"{where}more than {max_ties} tolerated ties")
        script[key] = set(gset)

    # every decision agrees: the whole tree element by element
    sa = orc["sa"]
    for n in range(1, len(sa["path"])):
        if abs(g.score[sa["path"][n]] - sa["score"][n]) > tol:
            raise Mismatch(f"{where}score of {sa['path'][n]}")
    n = int(gout["n_nodes"])
    if n != orc["n_nodes"]:
        raise Mismatch(f"{where}n_nodes {n} vs {orc['n_nodes']}")
    for k in ("tok", "parent", "depth", "mask"):
        if not np.array_equal(gout[k], orc[k]):
            raise Mismatch(f"{where}{k} differs")
    if np.max(np.abs(gout["score"][:n] - orc["score"][:n])) > tol:
        raise Mismatch(f"{where}scores differ by more than {tol}")
    amb = sum(1 for d in sa["decisions"].values() if d["ambiguous"])
    return {"exact": not ties, "ties": ties, "ambiguous": amb, "nodes": n,
            "superarbol": len(sa["path"])}


# ---------------------------------------------------------------------------
# the sequential best-first builder
# ---------------------------------------------------------------------------
class _GpuHeap:
    """The GPU heap round of one request: every pushed node by token path,
    the popped set, the emitted tree (checked against the popped set)."""

    def __init__(self, gout, gtr, B, where):
        check_invariants(gout, B, where)
        self.paths = _paths(gtr["node_tok"], gtr["node_parent"])
        if len(set(self.paths)) != len(self.paths):
            raise Mismatch(f"{where}GPU heap pushed a token path twice")
        self.score = {self.paths[i]: float(gtr["node_score"][i]) for i in range(1, len(self.paths))}
        self.kids = {}
        for i in range(1, len(self.paths)):
            self.kids.setdefault(self.paths[i][:-1], set()).add(self.paths[i][-1])
        self.C = [set(int(t) for t in row) for row in gtr["C"]]
        self.Cl = gtr["Cl"]
        self.Ctok = gtr["C"]
        pops = [int(x) for x in gtr["sel"]]
        n = 0
        while n < len(pops) and pops[n] >= 0:
            n += 1
        if any(x >= 0 for x in pops[n:]):
            raise Mismatch(f"{where}pops resume after an empty pop")
        self.pops = [self.paths[x] for x in pops[:n]]
        self.popped = set(self.pops)
        if len(self.popped) != n or () in self.popped:
            raise Mismatch(f"{where}a node was popped twice, or the root")
        nn = int(gout["n_nodes"])
        if nn != n + 1:
            raise Mismatch(f"{where}n_nodes {nn} vs {n} pops")
        out_paths = _paths(gout["tok"][:nn], gout["parent"][:nn])
        if set(out_paths[1:]) != self.popped:
            raise Mismatch(f"{where}output is not the GPU's own pop set")
        for i in range(1, nn):
            if gout["score"][i] != np.float32(self.score[out_paths[i]]):
                raise Mismatch(f"{where}output score differs from trace at {i}")


def _first_heap_divergence(g, orc, D, tol, where):
    sa = orc["sa"]
    by_path = {p: i for i, p in enumerate(sa["path"])}
    for dd in range(D):
        for j, t in enumerate(g.Ctok[dd]):
            if abs(float(g.Cl[dd][j]) - float(orc["Lb"][dd][int(t)])) > tol:
                raise Mismatch(f"{where}base logit of token {t} at depth {dd}")
        if g.C[dd] != set(int(t) for t in sa["C"][dd]):
            return ("M", dd), g.C[dd]
    # expansions of the nodes both builds popped, in the oracle's pop order
    # (the root first)
    o_pops = [sa["path"][n] for n in orc["sel"]]
    for pth in [()] + o_pops:
        if len(pth) >= D or (pth and pth not in g.popped):
            continue
        o_k = {sa["tok"][c] for c in sa["kids"][by_path[pth]]}
        g_k = g.kids.get(pth, set())
        if g_k != o_k:
            return ("K", len(pth), pth), g_k
        for t in o_k:
            c = pth + (t,)
            if abs(g.score[c] - sa["score"][by_path[c]]) > tol:
                raise Mismatch(f"{where}score of {c}: gpu {g.score[c]} oracle {sa['score'][by_path[c]]}")
    if g.popped != set(o_pops):
        return ("P",), g.popped
    return None


def compare_heap_request(gout, gtr, prep, q, prm, tol=O.TIE_TOL, where="",
                         scoring="conditional", max_ties=64):
    """One request of a GPU heap-builder round against the oracle's
    sequential best-first builder, to the last node: candidate sets, every
    expansion's children, every pushed node's score and the pop set, with
    near-ties handled as in compare_request (the oracle's own admissible
    alternatives, then a rebuild along the GPU's choice)."""
    D, M, K, B, beta = prm["D"], prm["M"], prm["K"], prm["B"], prm["beta"]
    g = _GpuHeap(gout, gtr, B, where)
    script, ties = {}, []
    while True:
        orc = O.build_heap_tree(prep, q, D, M, K, B, beta, scoring=scoring, script=script, tol=tol)
        div = _first_heap_divergence(g, orc, D, tol, where)
        if div is None:
            break
        key, gset = div
        d = orc["sa"]["decisions"].get(key)
        if d is None:
            raise Mismatch(f"{where}decision {key}: GPU kept {sorted(gset)[:4]}, oracle has no choice")
        if not (len(gset) == d["n"] and d["sure"] <= gset <= (d["sure"] | d["band"])):
            raise Mismatch(f"{where}decision {key} differs beyond tolerance: "
                           f"{sorted(set(gset) ^ d['default'])[:4]}")
        ties.append(_tie_info(key, d, gset))
        if len(ties) > max_ties:
            raise Mismatch(f"{where}more than {max_ties} tolerated ties")
        script[key] = set(gset)
    sa = orc["sa"]
    if set(g.score) != set(sa["path"][1:]):
        raise Mismatch(f"{where}pushed nodes differ")
    for n in range(1, len(sa["path"])):
        if abs(g.score[sa["path"][n]] - sa["score"][n]) > tol:
            raise Mismatch(f"{where}score of {sa['path'][n]}")
    n = int(gout["n_nodes"])
    if n != orc["n_nodes"]:
        raise Mismatch(f"{where}n_nodes {n} vs {orc['n_nodes']}")
    for k in ("tok", "parent", "depth", "mask"):
        if not np.array_equal(gout[k], orc[k]):
            raise Mismatch(f"{where}{k} differs")
    if np.max(np.abs(gout["score"][:n] - orc["score"][:n])) > tol:
        raise Mismatch(f"{where}scores differ by more than {tol}")
    amb = sum(1 for d in sa["decisions"].values() if d["ambiguous"])
    return {"exact": not ties, "ties": ties, "ambiguous": amb, "nodes": n,
            "superarbol": len(sa["path"])}
