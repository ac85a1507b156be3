"""CPU oracle for one round of conditional draft-tree construction.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it, to check and to time against.
It shares no code with the HIP library.

What it computes, step by step, and where the pages define it
-------------------------------------------------------------
Pages cited (each by its title and section):
  * "Resumen Técnico: Domino" -- Metodología 1 (parallel backbone: hidden
    states H for the whole block, base logits through the frozen target LM
    head) and Metodología 2 (Domino head: a GRU summarises the embeddings of
    the preceding draft tokens into a causal state S; a low-rank head maps
    the concatenation [H_i ; S_{i-1}] to rank r and back to vocabulary
    space, giving Delta L_i; final logits L_i = L_base_i + Delta L_i).
  * "Resumen Técnico: DominoTree" -- Componentes Principales 1 (best-first
    max-heap keyed by cumulative path log-probability, children scored by
    the path-specific correction; H is shared by all paths) and 2 (the
    correction is restricted to the Top-M marginal candidates of each depth,
    a 256 x M slice, before the Top-k children are chosen).
  * "DARTree: Speculative Diffusion Decoding with Autoregressive Draft
    Trees" -- Metodología 1 (depth-wise expansion: per-depth candidates from
    the base logits, batched correction of every active branch with its own
    prefix state, scoring by corrected cumulative probability, keep the top
    W branches and carry their states) and Metodología 2 (after the
    fixed-width superarbol is built, one global Top-B over all materialised
    prefixes; Lemma 1: with a non-positive depth bonus beta this equals the
    set a sequential best-first max-heap would pick).

Readings where the pages leave a step open (each also listed in the design
notes): log-softmax over the M candidates only; candidates per depth shared
by all branches; every scored child enters the superarbol, only the top W
are expanded; B excludes the root; key = score + beta * depth; GRU cell =
the PyTorch GRUCell equations with gate blocks (r, z, n); state starts at 0
and first consumes the root (last verified) token; no nonlinearity in the
low-rank head; H[delta] scores the children at depth delta + 1;
tie-breaks are value descending then structural (token ascending for Top-M
and Top-K, lexicographic token path for Top-W, depth then lexicographic
path for Top-B); output in canonical order (depth, lexicographic path);
scores returned without the depth bonus; the mask holds ancestors and self.

Selection decisions and their near-cutoff bands
-----------------------------------------------
Every selection of the round (Top-M per depth, Top-K per expanded branch,
Top-W per depth, the global Top-B) keeps the first n items of a list ranked
by a floating-point value.  The DominoTree page (Resultados Experimentales,
losslessness) notes that the method is exact except for floating-point
tie-breaking.  For each decision the oracle records, from its OWN values:
the cutoff value c (the n-th best), the items surely kept (value > c + tol)
and the band of items within tol of c.  An admissible alternative selection
is any set X with  sure <= X <= sure | band  and |X| = n; when the band
holds more items than the slots left after the sure ones, the decision is
ambiguous.  ``script`` maps a decision's key to one admissible alternative;
the oracle checks admissibility against its own values, follows that
selection and computes everything after it itself.  It never receives a
value computed elsewhere.

Arithmetic: float64 everywhere, with values rounded to float32 at the
storage points marked ``_st`` (``store="f32"``, the default); with
``store="f64"`` nothing is rounded, which is what the brute-force pins use.
In bf16 mode the only bf16 values are the stored weights and Hq = bf16(H).
"""
import heapq

import numpy as np

__all__ = [
    "bf16_round", "decode", "OracleWeights", "base_logits", "top_m",
    "gru_cell", "log_softmax", "build_superarbol", "select_global_top_b",
    "select_literal_heap", "emit_tree", "build_round", "SCORINGS",
    "prepare_round", "build_request", "NotAdmissible", "TIE_TOL",
    "build_heap_tree",
]

TIE_TOL = 1e-4   # the parity tolerance in fp32 log-prob


class NotAdmissible(ValueError):
    """A scripted selection is not an admissible alternative of the oracle's
    own decision (it drops a surely-kept item, adds an item outside the band,
    or has the wrong size)."""


# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------
def bf16_round(x):
    """Round float32 values to the nearest bf16 (ties to even); float32 out.

    bf16 keeps the top 16 bits of an IEEE float32.  Adding 0x7FFF plus the
    lowest kept bit and truncating is round-to-nearest-even.  Inputs are
    finite (the round's inputs must be finite).
    """
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + keep_lsb) >> np.uint64(16)) << np.uint64(16)
    return r.astype(np.uint32).view(np.float32)


def decode(arr, wtype):
    """Stored weights -> float64.  bf16 arrays arrive as uint16 bit patterns."""
    if wtype == "bf16":
        a = np.asarray(arr, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return a.view(np.float32).astype(np.float64)
    return np.asarray(arr, dtype=np.float32).astype(np.float64)


def _storer(store):
    if store == "f32":
        return lambda x: np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    if store == "f64":
        return lambda x: np.asarray(x, dtype=np.float64)
    raise ValueError(store)


class OracleWeights:
    """The shared weights decoded to float64 (the large tables lazily)."""

    def __init__(self, weights, wtype, d, s):
        self.raw = weights
        self.wtype = wtype
        self.d, self.s = d, s
        self.W_ih = decode(weights["W_ih"], wtype)
        self.W_hh = decode(weights["W_hh"], wtype)
        self.b_ih = np.asarray(weights["b_ih"], np.float32).astype(np.float64)
        self.b_hh = np.asarray(weights["b_hh"], np.float32).astype(np.float64)
        W1 = decode(weights["W1"], wtype)
        self.W1_H = W1[:, :d]          # acts on H_i
        self.W1_S = W1[:, d:d + s]     # acts on S_{i-1}
        b = weights.get("bias")
        self.bias = None if b is None else np.asarray(b, np.float32).astype(np.float64)

    def emb_rows(self, toks):
        return decode(self.raw["Emb"][np.asarray(toks, dtype=np.int64)], self.wtype)

    def w2_rows(self, toks):
        return decode(self.raw["W2"][np.asarray(toks, dtype=np.int64)], self.wtype)


# ---------------------------------------------------------------------------
# steps of one round
# ---------------------------------------------------------------------------
def base_logits(Hq, weights, wtype, store="f32", chunk=8192):
    """L_base = Hq . W_lm^T + bias for every row of Hq (rows = depths).

    Domino page, Metodología 1: the base logits come from the backbone's
    hidden states through the frozen target LM head; the Zipf-like unigram
    bias of the synthetic workload is added to them.  Computed one vocabulary
    slab at a time so the float64 copy of W_lm never exists whole.
    """
    st = _storer(store)
    W_lm = weights["W_lm"]
    V = W_lm.shape[0]
    Hq64 = np.asarray(Hq, dtype=np.float64)
    out = np.empty((Hq64.shape[0], V), dtype=np.float64)
    bias = weights.get("bias")
    for lo in range(0, V, chunk):
        hi = min(V, lo + chunk)
        slab = Hq64 @ decode(W_lm[lo:hi], wtype).T
        if bias is not None:
            slab = slab + np.asarray(bias[lo:hi], np.float32).astype(np.float64)
        out[:, lo:hi] = st(slab)
    return out


def top_m(row, M):
    """Top-M tokens of one row of base logits: value descending, token
    ascending on exact ties.  Returns (tokens, values) in that order.

    DominoTree page, Componentes Principales 2; DARTree page, Metodología 1
    (candidate selection from the base logits at each depth).
    """
    toks = np.arange(row.shape[0])
    order = np.lexsort((toks, -row))[:M]
    return order.astype(np.int64), row[order]


def gru_cell(x, h, W, store="f32"):
    """One GRU step, PyTorch GRUCell form, gate blocks (r, z, n).

    Domino page, Metodología 2: a light GRU folds the embedding of each
    preceding draft token into the causal state.  x: [n, e], h: [n, s].
    """
    st = _storer(store)
    s = W.s
    a = x @ W.W_ih.T + W.b_ih          # input part, [n, 3s]
    c = h @ W.W_hh.T + W.b_hh          # state part, [n, 3s]
    r = 1.0 / (1.0 + np.exp(-(a[:, :s] + c[:, :s])))
    z = 1.0 / (1.0 + np.exp(-(a[:, s:2 * s] + c[:, s:2 * s])))
    n = np.tanh(a[:, 2 * s:] + r * c[:, 2 * s:])
    return st((1.0 - z) * n + z * h)


def log_softmax(ell, store="f32"):
    """Row-wise log-softmax over the M candidate columns, max-shifted."""
    st = _storer(store)
    m = ell.max(axis=1, keepdims=True)
    lse = m + np.log(np.exp(ell - m).sum(axis=1, keepdims=True))
    return st(ell - lse)


def _key(score, depth, beta, store):
    """Selection key score + beta * depth (DARTree page, Metodología 2)."""
    if store == "f32":
        return float(np.float32(score) + np.float32(np.float32(beta) * np.float32(depth)))
    return float(score) + float(beta) * float(depth)


# ---------------------------------------------------------------------------
# selection decisions
# ---------------------------------------------------------------------------
def _decide(key, items, values, order_key, n, script, decisions, tol):
    """Keep the first n of ``items`` ranked by (value desc, order_key asc).

    Records the decision's near-cutoff band (see the module docstring) under
    ``key`` in ``decisions``; follows ``script[key]`` if present, after
    checking that it is admissible.  Returns the kept items in rank order.
    """
    ranked = sorted(range(len(items)), key=lambda i: (-values[i], order_key(items[i])))
    if n >= len(items):
        if key in script and set(script[key]) != set(items):
            raise NotAdmissible(f"{key}: every item is kept")
        return [items[i] for i in ranked]
    cut = float(values[ranked[n - 1]])
    sure = {items[i] for i in range(len(items)) if values[i] > cut + tol}
    band = {items[i] for i in range(len(items)) if abs(values[i] - cut) <= tol}
    default = [items[i] for i in ranked[:n]]
    decisions[key] = dict(n=n, cut=cut, sure=sure, band=band, default=set(default),
                          ambiguous=len(band) > n - len(sure))
    if key not in script:
        return default
    X = set(script[key])
    if len(X) != n or not sure <= X or not X <= (sure | band):
        raise NotAdmissible(f"{key}: not an admissible alternative")
    return [items[i] for i in ranked if items[i] in X]


def _decide_top_m(key, row, M, script, decisions, tol):
    """Top-M of one vocabulary row as a recorded decision (vectorised: the
    band is taken over every token of the vocabulary)."""
    toks, vals = top_m(row, M)
    if M >= row.shape[0]:
        return toks, vals
    cut = float(vals[M - 1])
    sure = set(np.nonzero(row > cut + tol)[0].tolist())
    band = set(np.nonzero(np.abs(row - cut) <= tol)[0].tolist())
    decisions[key] = dict(n=M, cut=cut, sure=sure, band=band, default=set(toks.tolist()),
                          ambiguous=len(band) > M - len(sure))
    if key not in script:
        return toks, vals
    X = set(int(t) for t in script[key])
    if len(X) != M or not sure <= X or not X <= (sure | band):
        raise NotAdmissible(f"{key}: not an admissible alternative")
    t = np.array(sorted(X, key=lambda v: (-row[v], v)), dtype=np.int64)
    return t, row[t]


SCORINGS = ("conditional", "marginal", "markov")


def build_superarbol(Hq_req, root_tok, Lb_req, W, D, M, K, Wd, store="f32",
                     scoring="conditional", script=None, tol=TIE_TOL):
    """Depth-wise construction of one request's superarbol.

    DARTree page, Metodología 1, with the Domino head as the corrected
    drafter (Domino page, Metodología 2) and the Top-M restriction
    (DominoTree page, Componentes Principales 2).

    scoring:
      * "conditional" (the method): each branch's own GRU state over its
        whole token path;
      * "marginal": the path-independent base logits alone (Delta L = 0, no
        GRU state): the uncorrected, DDTree-style scoring the pages compare
        against with the same drafter and tree construction (DominoTree page,
        Contribuciones Clave, the conditionality ablation; DARTree page,
        Resultados Experimentales, DDTree as the marginal baseline);
      * "markov": a first-order correction that conditions on the parent
        token only (DARTree page, Resultados Experimentales, Ablación,
        generality: the DSpark drafter with a Markov correction head).
        Reading taken: the causal state of a branch is the GRU applied to
        its last token from a zero state, S = GRU(Emb[token], 0); the root
        is the same as in conditional scoring.

    Hq_req: [D, d] rounded hidden states; Lb_req: [D, V] base logits.
    Wd is the branch width W (the name W is taken by the weights).
    ``script``: {decision key: admissible alternative} (module docstring).
    Returns a dict with the node table, the per-depth intermediates and the
    decision records.
    """
    if scoring not in SCORINGS:
        raise ValueError(f"scoring must be one of {SCORINGS}")
    script = script or {}
    decisions = {}
    marginal = scoring == "marginal"
    st = _storer(store)
    C = np.empty((D, M), dtype=np.int64)
    Cl = np.empty((D, M), dtype=np.float64)
    for dd in range(D):
        C[dd], Cl[dd] = _decide_top_m(("M", dd), Lb_req[dd], M, script, decisions, tol)
    # path-independent part of the low-rank projection, shared by all paths
    uH = st(np.asarray(Hq_req, np.float64) @ W.W1_H.T)          # [D, r]

    tok, par, dep, score, path = [int(root_tok)], [-1], [0], [0.0], [()]
    kids = [[]]
    # the block starts with the last verified token: the GRU consumes it first
    S = None if marginal else gru_cell(W.emb_rows([root_tok]), np.zeros((1, W.s)), W, store)
    frontier = [0]
    per_depth = []
    for dd in range(D):
        A = len(frontier)
        if marginal:
            u = None
            ell = np.repeat(Cl[dd][None, :], A, axis=0)           # [A, M]
        else:
            u = st(uH[dd][None, :] + S @ W.W1_S.T)               # [A, r]
            ell = st(Cl[dd][None, :] + u @ W.w2_rows(C[dd]).T)  # [A, M]
        lp = log_softmax(ell, store)                             # [A, M]
        children = []
        cand = [int(t) for t in C[dd]]
        for a, p in enumerate(frontier):
            # Top-K children of branch p: lp descending, token ascending
            kept = _decide(("K", dd, path[p]), cand, lp[a], lambda t: t, K, script,
                           decisions, tol)
            for t in kept:
                j = cand.index(t)
                nid = len(tok)
                tok.append(t)
                par.append(p)
                dep.append(dd + 1)
                score.append(float(st(score[p] + lp[a, j])))
                path.append(path[p] + (t,))
                kids.append([])
                kids[p].append(nid)
                children.append(nid)
        # Top-W survivors of the depth: score descending, lexicographic path
        surv = _decide_paths(("W", dd + 1), children, score, path, Wd, script,
                             decisions, tol)
        per_depth.append(dict(frontier=list(frontier), u=u, ell=ell, lp=lp,
                              children=children, survivors=surv))
        if dd + 1 < D and not marginal:
            slot = {p: a for a, p in enumerate(frontier)}
            if scoring == "markov":
                h = np.zeros((len(surv), W.s))
            else:
                h = S[[slot[par[c]] for c in surv]]
            S = gru_cell(W.emb_rows([tok[c] for c in surv]), h, W, store)
        frontier = surv
    return dict(tok=tok, parent=par, depth=dep, score=score, path=path,
                kids=kids, C=C, Cl=Cl, uH=uH, per_depth=per_depth, decisions=decisions)


def _decide_paths(key, nodes, score, path, n, script, decisions, tol):
    """A decision over superarbol nodes, with alternatives named by token
    path (node ids are not stable across alternatives)."""
    by_path = {path[v]: v for v in nodes}
    sub = {}
    if key in script:
        sub[key] = set(script[key])
    kept = _decide(key, [path[v] for v in nodes], [score[v] for v in nodes],
                   lambda p: p, n, sub, decisions, tol)
    return [by_path[p] for p in kept]


def _order_key(sa, n, beta, store):
    """Total order used by the selection: key desc, depth asc, path asc."""
    return (-_key(sa["score"][n], sa["depth"][n], beta, store),
            sa["depth"][n], sa["path"][n])


def select_global_top_b(sa, B, beta, store="f32", script=None, tol=TIE_TOL):
    """One global Top-B over every materialised prefix (root excluded).

    DARTree page, Metodología 2 (deferred pruning).  The decision (keys
    against the B-th key) is recorded in sa["decisions"][("B",)]; a scripted
    admissible alternative (a set of token paths) is followed."""
    nodes = list(range(1, len(sa["tok"])))
    keys = [_key(sa["score"][n], sa["depth"][n], beta, store) for n in nodes]
    # items are token paths, ranked by (key desc, depth asc, path asc): a
    # path's depth is its length
    items = [sa["path"][n] for n in nodes]
    dec = sa.setdefault("decisions", {})
    sub = {("B",): set(script[("B",)])} if script and ("B",) in script else {}
    kept = _decide(("B",), items, keys, lambda pth: (len(pth), pth), min(B, len(nodes)),
                   sub, dec, tol)
    by_path = {pth: n for pth, n in zip(items, nodes)}
    return [by_path[pth] for pth in kept]


def select_literal_heap(sa, B, beta, store="f32"):
    """The sequential best-first max-heap over the same superarbol: start
    from the root's children, pop the best node, push its children, repeat.

    DominoTree page, Componentes Principales 1; DARTree page, Planteamiento
    del Problema 3 (the heap loop) -- the definition Lemma 1 compares the
    global Top-B to.
    """
    heap = [(_order_key(sa, c, beta, store), c) for c in sa["kids"][0]]
    heapq.heapify(heap)
    pops = []
    for _ in range(min(B, len(sa["tok"]) - 1)):
        if not heap:
            break
        _, n = heapq.heappop(heap)
        pops.append(n)
        for c in sa["kids"][n]:
            heapq.heappush(heap, (_order_key(sa, c, beta, store), c))
    return pops


def emit_tree(sa, sel, B):
    """Compact tree for verification: the root, then the selected nodes in
    canonical order (depth, lexicographic path); parents re-indexed; the
    ancestor-or-self mask (DominoTree page, Componentes Principales 5: tree
    attention with an ancestor-only mask).  Scores are the raw cumulative
    log-probs.  Raises if the selection is not closed under parents.
    """
    chosen = set(sel)
    for n in sel:
        p = sa["parent"][n]
        if p != 0 and p not in chosen:
            raise AssertionError(f"selection not ancestor-closed at node {n}")
    order = [0] + sorted(sel, key=lambda n: (sa["depth"][n], sa["path"][n]))
    N = B + 1
    n_nodes = len(order)
    idx = {n: i for i, n in enumerate(order)}
    tok = np.full(N, -1, np.int32)
    parent = np.full(N, -1, np.int32)
    depth = np.full(N, -1, np.int32)
    score = np.full(N, -np.inf, np.float32)
    mask = np.zeros((N, N), np.uint8)
    for i, n in enumerate(order):
        tok[i] = sa["tok"][n]
        depth[i] = sa["depth"][n]
        score[i] = np.float32(sa["score"][n])
        parent[i] = -1 if n == 0 else idx[sa["parent"][n]]
        if i > 0:
            mask[i] = mask[parent[i]]
        mask[i, i] = 1
    return dict(tok=tok, parent=parent, depth=depth, score=score, mask=mask,
                n_nodes=n_nodes, order=order)


# ---------------------------------------------------------------------------
# whole rounds
# ---------------------------------------------------------------------------
def prepare_round(inputs, D, store="f32"):
    """The path-independent part shared by every request and every
    alternative: decoded weights, Hq = q(H) and the base logits."""
    wts, wtype = inputs["weights"], inputs["wtype"]
    H = np.asarray(inputs["H"], dtype=np.float32)
    b, Dh, d = H.shape
    assert Dh >= D
    s = wts["W_hh"].shape[1]
    Wo = OracleWeights(wts, wtype, d, s)
    Hq = bf16_round(H[:, :D]) if wtype == "bf16" else H[:, :D]
    Lb = base_logits(Hq.reshape(b * D, d), wts, wtype, store).reshape(b, D, -1)
    return dict(W=Wo, Hq=Hq, Lb=Lb, root=np.asarray(inputs["root"]), D=D, store=store)


def build_request(prep, q, D, M, K, W, B, beta, check_heap=True, scoring="conditional",
                  script=None, tol=TIE_TOL):
    """One request's round: superarbol, global Top-B, emission.  ``script``
    names admissible alternatives at any of the round's decisions."""
    assert D == prep["D"]
    store = prep["store"]
    sa = build_superarbol(prep["Hq"][q], int(prep["root"][q]), prep["Lb"][q], prep["W"],
                          D, M, K, W, store, scoring, script, tol)
    sel = select_global_top_b(sa, B, beta, store, script, tol)
    if check_heap and not (script and ("B",) in script):
        pops = select_literal_heap(sa, B, beta, store)
        if set(pops) != set(sel):
            raise AssertionError("Lemma 1 violated: heap and global Top-B differ")
    out = emit_tree(sa, sel, B)
    out["sa"] = sa
    out["sel"] = sel
    out["Lb"] = prep["Lb"][q]
    return out


def build_round(inputs, D, M, K, W, B, beta, store="f32", check_heap=True,
                scoring="conditional"):
    """Whole round for every request of ``inputs`` (as drawn by ``synth``).

    Returns per-request outputs (tok, parent, depth, score, mask, n_nodes)
    and the superarbol trace used by the checkers.  ``scoring`` as in
    ``build_superarbol``.
    """
    prep = prepare_round(inputs, D, store)
    return [build_request(prep, q, D, M, K, W, B, beta, check_heap, scoring)
            for q in range(prep["Hq"].shape[0])]


# ---------------------------------------------------------------------------
# the sequential best-first builder (DominoTree)
# ---------------------------------------------------------------------------
def build_heap_tree(prep, q, D, M, K, B, beta, scoring="conditional", script=None,
                    tol=TIE_TOL):
    """DominoTree's conditional-scored best-first tree for request q.

    DominoTree page, Componentes Principales 1 and 2: a max-priority queue
    keyed by the cumulative path log-probability; each pop re-runs the GRU
    correction along the popped node's own path and pushes its Top-k
    children, scored over the depth's Top-M candidates; the expensive
    hidden states are shared.  Reading taken: the queue starts with the
    root's Top-K children (the root is the last verified token and is
    expanded first, not counted in B); B pops; nodes at depth D are not
    expanded; the queue order is the selection order of the depth-wise
    build (key = score + beta * depth descending, then depth, then token
    path), so with beta = 0 it is the plain cumulative log-probability; the
    build stops at the B-th pop without expanding it (its children could
    never be popped).

    Returns the same node table as build_superarbol (every node ever
    pushed), with sel = the popped nodes in pop order.  The pop set is a
    recorded decision ("P",) over every pushed node; a scripted admissible
    alternative (a set of token paths closed under parents) is popped first.
    """
    if scoring not in ("conditional", "markov"):
        raise ValueError("the heap builder scores conditionally or with the Markov head")
    script = script or {}
    decisions = {}
    st = _storer(prep["store"])
    W, store = prep["W"], prep["store"]
    Hq, Lb, root_tok = prep["Hq"][q], prep["Lb"][q], int(prep["root"][q])
    C = np.empty((D, M), dtype=np.int64)
    Cl = np.empty((D, M), dtype=np.float64)
    for dd in range(D):
        C[dd], Cl[dd] = _decide_top_m(("M", dd), Lb[dd], M, script, decisions, tol)
    uH = st(np.asarray(Hq, np.float64) @ W.W1_H.T)
    tok, par, dep, score, path, kids = [root_tok], [-1], [0], [0.0], [()], [[]]
    state = {}

    def expand(n, S):
        dd = dep[n]
        u = st(uH[dd][None, :] + S @ W.W1_S.T)
        ell = st(Cl[dd][None, :] + u @ W.w2_rows(C[dd]).T)
        lp = log_softmax(ell, store)[0]
        cand = [int(t) for t in C[dd]]
        kept = _decide(("K", dd, path[n]), cand, lp, lambda t: t, K, script, decisions, tol)
        for t in kept:
            nid = len(tok)
            tok.append(t)
            par.append(n)
            dep.append(dd + 1)
            score.append(float(st(score[n] + lp[cand.index(t)])))
            path.append(path[n] + (t,))
            kids.append([])
            kids[n].append(nid)
        return kids[n]

    # a scripted pop set (an admissible alternative of the ("P",) decision
    # below) is popped first, each part in the builder's order
    forced = set(script[("P",)]) if ("P",) in script else None

    def okey(n):
        k = (-_key(score[n], dep[n], beta, store), dep[n], path[n])
        return k if forced is None else ((0 if path[n] in forced else 1),) + k

    state[0] = gru_cell(W.emb_rows([root_tok]), np.zeros((1, W.s)), W, store)
    heap = [(okey(c), c) for c in expand(0, state[0])]
    heapq.heapify(heap)
    pops = []
    while len(pops) < B and heap:
        _, n = heapq.heappop(heap)
        pops.append(n)
        # the B-th pop ends the build: its children could never be popped
        if dep[n] < D and len(pops) < B:
            h = np.zeros((1, W.s)) if scoring == "markov" else state[par[n]]
            state[n] = gru_cell(W.emb_rows([tok[n]]), h, W, store)
            for c in expand(n, state[n]):
                heapq.heappush(heap, (okey(c), c))
    # The pops come out in the builder's order over every pushed node (keys
    # never grow from a node to its children when beta <= 0), so the popped
    # set is the first len(pops) pushed nodes in that order: recorded as a
    # decision with its near-cutoff band, like the global Top-B.
    nodes = list(range(1, len(tok)))
    items = [path[n] for n in nodes]
    keys = [_key(score[n], dep[n], beta, store) for n in nodes]
    kept = _decide(("P",), items, keys, lambda pth: (len(pth), pth), len(pops), script,
                   decisions, tol)
    if set(kept) != {path[n] for n in pops}:
        raise AssertionError("the pops are not the first pushed nodes in the builder's order")
    sa = dict(tok=tok, parent=par, depth=dep, score=score, path=path, kids=kids, C=C,
              Cl=Cl, uH=uH, decisions=decisions)
    out = emit_tree(sa, pops, B)
    out["sa"] = sa
    out["sel"] = pops
    out["Lb"] = Lb
    return out
