"""Compares one request's GPU round with the oracle's (tests only).

Parity rule: tree structure (tokens, parents, depths, mask, node count) must
be identical, scores within ``tol`` (1e-4 absolute, fp32 log-prob), and a
selection may differ only where the competing values are within ``tol`` of
the oracle's cutoff.  The two sides are compared stage by stage using the
library's debug trace (candidate tables, superarbol, expanded nodes per
depth, selected set), matching nodes by token path.  At the first stage
whose sets differ, every differing item must sit within ``tol`` of the
oracle's cutoff value (a tolerated near-tie); from there on the two runs
legitimately diverge, so the rest of that request is checked for validity
only (output invariants and self-consistency with its own trace).  The
oracle never receives anything computed on the GPU.
"""
import numpy as np


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


def _tie_ok(vals_by_item, diff, cutoff, tol):
    return all(abs(vals_by_item[x] - cutoff) <= tol for x in diff)


def compare_request(gout, gtr, orc, prm, tol=1e-4, where=""):
    """gout: GPU outputs of one request; gtr: its trace; orc: the oracle's
    result for that request.  Returns a dict {'exact': bool, 'tie': str}."""
    D, M, K, W, B = prm["D"], prm["M"], prm["K"], prm["W"], prm["B"]
    sa = orc["sa"]
    check_invariants(gout, B, where)
    if gtr["status"] != 0:
        raise Mismatch(f"{where}device status {gtr['status']}")

    # GPU output must be the GPU's own selection in canonical order
    gpaths = _paths(gtr["node_tok"], gtr["node_parent"])
    n = int(gout["n_nodes"])
    sel_ids = [int(x) for x in gtr["sel"] if x >= 0]
    if n != len(sel_ids) + 1:
        raise Mismatch(f"{where}n_nodes {n} vs {len(sel_ids)} selected")
    out_paths = _paths(gout["tok"][:n], gout["parent"][:n])
    if set(out_paths[1:]) != {gpaths[i] for i in sel_ids}:
        raise Mismatch(f"{where}output is not the GPU's own selection")
    gscore = {gpaths[i]: float(gtr["node_score"][i]) for i in range(1, len(gpaths))}
    for i in range(1, n):
        if gout["score"][i] != np.float32(gscore[out_paths[i]]):
            raise Mismatch(f"{where}output score differs from trace at {i}")

    # stage 1: candidate tables
    for dd in range(D):
        gs, os_ = set(gtr["C"][dd].tolist()), set(int(t) for t in sa["C"][dd])
        lbt, lbv = orc["lb_sorted"][dd]
        lb = {int(t): float(v) for t, v in zip(lbt, lbv)}
        for j, t in enumerate(gtr["C"][dd]):
            if int(t) in lb and abs(float(gtr["Cl"][dd][j]) - lb[int(t)]) > tol:
                raise Mismatch(f"{where}base logit of token {t} at depth {dd}")
        if gs != os_:
            diff = gs ^ os_
            if not all(t in lb for t in diff) or not _tie_ok(lb, diff, float(sa["Cl"][dd][M - 1]), tol):
                raise Mismatch(f"{where}candidates at depth {dd} differ beyond tolerance: {diff}")
            return {"exact": False, "tie": f"top-M at depth {dd}"}

    # stage 2: depth by depth
    opath_id = {p: i for i, p in enumerate(sa["path"])}
    gpath_id = {p: i for i, p in enumerate(gpaths)}
    gkids = {}
    for i in range(1, len(gpaths)):
        gkids.setdefault(int(gtr["node_parent"][i]), []).append(i)
    if set(gpaths) - set(opath_id):
        extra = set(gpaths) - set(opath_id)
    else:
        extra = set()
    for dd in range(D):
        pdp = sa["per_depth"][dd]
        g_front = {gpaths[i] for i in gtr["surv"][dd] if i >= 0}
        o_front = {sa["path"][i] for i in pdp["frontier"]}
        if g_front != o_front:
            raise Mismatch(f"{where}expanded set at depth {dd} differs without a recorded tie")
        for a, p in enumerate(pdp["frontier"]):
            ppath = sa["path"][p]
            o_k = {sa["tok"][c] for c in sa["kids"][p]}
            g_k = {gpaths[c][-1] for c in gkids.get(gpath_id[ppath], [])}
            if g_k != o_k:
                lpm = {int(t): float(v) for t, v in zip(sa["C"][dd], pdp["lp"][a])}
                order = sorted(lpm.values(), reverse=True)
                if not _tie_ok(lpm, g_k ^ o_k, order[K - 1], tol):
                    raise Mismatch(f"{where}children of {ppath} differ beyond tolerance")
                return {"exact": False, "tie": f"top-K at depth {dd}"}
        for c in pdp["children"]:
            cp = sa["path"][c]
            if abs(gscore[cp] - sa["score"][c]) > tol:
                raise Mismatch(f"{where}score of {cp}: gpu {gscore[cp]} oracle {sa['score'][c]}")
        g_surv = {gpaths[i] for i in gtr["surv"][dd + 1] if i >= 0}
        o_surv = {sa["path"][i] for i in pdp["survivors"]}
        if g_surv != o_surv:
            osc = {sa["path"][c]: sa["score"][c] for c in pdp["children"]}
            cut = sorted(osc.values(), reverse=True)[len(o_surv) - 1]
            if not _tie_ok(osc, g_surv ^ o_surv, cut, tol):
                raise Mismatch(f"{where}survivors at depth {dd + 1} differ beyond tolerance")
            return {"exact": False, "tie": f"top-W at depth {dd + 1}"}
    if extra:
        raise Mismatch(f"{where}GPU superarbol has paths the oracle lacks: {sorted(extra)[:3]}")
    if len(gpaths) != len(sa["path"]):
        raise Mismatch(f"{where}superarbol sizes {len(gpaths)} vs {len(sa['path'])}")

    # stage 3: global Top-B
    g_sel = {gpaths[i] for i in sel_ids}
    o_sel = {sa["path"][i] for i in orc["sel"]}
    if g_sel != o_sel:
        beta = np.float32(prm["beta"])
        okey = {sa["path"][i]: float(np.float32(sa["score"][i]) + np.float32(beta * np.float32(sa["depth"][i])))
                for i in range(1, len(sa["path"]))}
        cut = okey[sa["path"][orc["sel"][-1]]]
        if not _tie_ok(okey, g_sel ^ o_sel, cut, tol):
            raise Mismatch(f"{where}selected set differs beyond tolerance")
        return {"exact": False, "tie": "top-B"}

    # stage 4: identical structure, scores within tolerance
    for k in ("tok", "parent", "depth", "mask"):
        if not np.array_equal(gout[k], orc[k]):
            raise Mismatch(f"{where}{k} differs")
    if n != orc["n_nodes"]:
        raise Mismatch(f"{where}n_nodes differs")
    if np.max(np.abs(gout["score"][:n] - orc["score"][:n])) > tol:
        raise Mismatch(f"{where}scores differ by more than {tol}")
    return {"exact": True, "tie": ""}
