"""Writes the hand-worked fixtures of this folder.

Every expected value below was derived by hand from the method's definition
(the derivation travels with each fixture); this script only serialises
them.  It calls no code of the oracle or of the library.
"""
import json
import math
import os

ln2 = math.log(2.0)
HERE = os.path.dirname(os.path.abspath(__file__))
common_H = [[0.0, ln2, 0.0, -5.0], [ln2, 0.0, 0.0, 0.0]]
eye = [[1.0 if i == j else 0.0 for j in range(4)] for i in range(4)]

g1 = {
    "name": "marginal_ties",
    "cites": ["DARTree page, Methodology 1 (per-depth candidates from base logits, Top-W) "
              "and Methodology 2 (global Top-B with a depth bonus)",
              "DominoTree page, Main components 2 (Top-M then Top-k) and 5 (ancestor-only mask)"],
    "derivation": [
        "W2 = 0 so the correction vanishes and every branch sees the base logits; "
        "W_lm = I and bias = 0 so L_base = H.",
        "Depth 1: L_base = (0, ln2, 0, -5). Top-3 = tok1 (ln2), then the tie at 0 broken by "
        "token: tok0, tok2. log-softmax over {ln2,0,0}: exp sum 4 -> lp(tok1) = -ln2, "
        "lp(tok0) = lp(tok2) = -2ln2. Top-2 children: tok1, then tok0 (tie with tok2 broken by token).",
        "W = 2 keeps both depth-1 nodes. Depth 2: L_base = (ln2,0,0,0): Top-3 = tok0, tok1, tok2 "
        "(tok3 loses the tie by token). lp: tok0 -ln2, tok1 -2ln2. Children of (1): (1,0) -2ln2, "
        "(1,1) -3ln2. Children of (0): (0,0) -3ln2, (0,1) -4ln2.",
        "keys = score - 0.5*depth: (1) -ln2-0.5, (0) -2ln2-0.5, (1,0) -2ln2-1, (1,1) = (0,0) = "
        "-3ln2-1 (equal sums of the same two fp32 log-probs), (0,1) -4ln2-1. Top-4: (1), (0), "
        "(1,0), then the exact tie between (0,0) and (1,1) is broken by depth (equal) and then "
        "lexicographic path: (0,0).",
        "Canonical order: root, (0), (1), (0,0), (1,0)."],
    "params": {"D": 2, "M": 3, "K": 2, "W": 2, "B": 4, "beta": -0.5},
    "weights": {
        "W_lm": eye, "bias": [0.0] * 4, "Emb": [[0.0]] * 4,
        "W_ih": [[0.0]] * 3, "W_hh": [[0.0]] * 3, "b_ih": [0.0] * 3, "b_hh": [0.0] * 3,
        "W1": [[0.0] * 5], "W2": [[0.0]] * 4},
    "H": [common_H], "root": [3],
    "expect": {"n_nodes": 5,
               "tok": [3, 0, 1, 0, 0], "parent": [-1, 0, 0, 1, 2], "depth": [0, 1, 1, 2, 2],
               "score": ["0", "-2*ln2", "-ln2", "-3*ln2", "-2*ln2"],
               "mask": [[1, 0, 0, 0, 0], [1, 1, 0, 0, 0], [1, 0, 1, 0, 0],
                        [1, 1, 0, 1, 0], [1, 0, 1, 0, 1]]},
    "score_tol": 1e-6,
}

w2 = {
    "W_lm": eye, "bias": [0.0] * 4,
    "Emb": [[0.0], [math.atanh(0.5)], [0.0], [0.0]],
    "W_ih": [[0.0], [0.0], [1.0]], "W_hh": [[0.0]] * 3, "b_ih": [0.0] * 3, "b_hh": [0.0] * 3,
    "W1": [[0.0, 0.0, 0.0, 0.0, 1.0]], "W2": [[0.0], [0.0], [8.0 * ln2], [0.0]]}
deriv2 = [
    "GRU with s = e = 1: all gate inputs are 0 except the candidate gate n = tanh(x), so "
    "r = z = 1/2 and h' = tanh(x)/2 + h/2. Emb(tok1) = atanh(1/2), every other embedding is 0.",
    "The root (tok3, embedding 0) gives S_root = 0. W1 = (0,0,0,0 | 1) so u = S; "
    "W2 = (0, 0, 8ln2, 0) so only tok2 is corrected, by 8ln2 * S.",
    "Depth 1 (S = 0): as in marginal_ties, children of the root are tok1 (-ln2) and tok0 (-2ln2).",
    "Branch (1): S = tanh(atanh(1/2))/2 = 1/4, so tok2 gains 2ln2: logits over C = (tok0 ln2, "
    "tok1 0, tok2 2ln2), exp sum 2+1+4 = 7: lp(tok2) = ln(4/7), lp(tok0) = ln(2/7), "
    "lp(tok1) = ln(1/7). Children (1,2) = -ln2 + ln(4/7) = ln(2/7), (1,0) = -ln2 + ln(2/7) = ln(1/7).",
    "Branch (0): S = tanh(0)/2 = 0, no correction: children (0,0) = -3ln2, (0,1) = -4ln2 "
    "(tok1 beats tok2 on the tie at 0 by token)."]
g2 = {
    "name": "path_conditional",
    "cites": ["Domino page, Methodology 2 (GRU causal state, low-rank head on [H_i ; S_{i-1}], "
              "L = L_base + Delta L)",
              "DARTree page, Methodology 1 and 2",
              "DominoTree page, Main components 1 (children scored by the path's own correction)"],
    "derivation": deriv2 + [
        "W = 2, B = 4, beta = -0.5: keys (1) -ln2-0.5, (0) -2ln2-0.5, (1,2) ln(2/7)-1, "
        "(1,0) ln(1/7)-1, (0,0) -3ln2-1, (0,1) -4ln2-1. Top-4: (1), (0), (1,2), (1,0).",
        "Canonical order: root, (0), (1), (1,0), (1,2). Branch (1) and branch (0) chose "
        "different children: the scoring is path-dependent."],
    "params": {"D": 2, "M": 3, "K": 2, "W": 2, "B": 4, "beta": -0.5},
    "weights": w2, "H": [common_H], "root": [3],
    "expect": {"n_nodes": 5,
               "tok": [3, 0, 1, 0, 2], "parent": [-1, 0, 0, 2, 2], "depth": [0, 1, 1, 2, 2],
               "score": ["0", "-2*ln2", "-ln2", "log(1/7)", "log(2/7)"],
               "mask": [[1, 0, 0, 0, 0], [1, 1, 0, 0, 0], [1, 0, 1, 0, 0],
                        [1, 0, 1, 1, 0], [1, 0, 1, 0, 1]]},
    "score_tol": 2e-6,
}
g3 = json.loads(json.dumps(g2))
g3["name"] = "path_conditional_pruned"
g3["params"] = {"D": 2, "M": 3, "K": 2, "W": 1, "B": 3, "beta": -0.5}
g3["derivation"] = deriv2[:3] + [
    "W = 1: only (1) survives depth 1 (score -ln2 beats -2ln2), so only branch (1) is "
    "expanded: " + deriv2[3],
    "The superarbol holds (1), (0), (1,2), (1,0). B = 3, beta = -0.5: keys (1) -ln2-0.5, "
    "(0) -2ln2-0.5, (1,2) ln(2/7)-1, (1,0) ln(1/7)-1; Top-3: (1), (0), (1,2).",
    "Canonical order: root, (0), (1), (1,2)."]
g3["expect"] = {"n_nodes": 4, "tok": [3, 0, 1, 2], "parent": [-1, 0, 0, 2], "depth": [0, 1, 1, 2],
                "score": ["0", "-2*ln2", "-ln2", "log(2/7)"],
                "mask": [[1, 0, 0, 0], [1, 1, 0, 0], [1, 0, 1, 0], [1, 0, 1, 1]]}

g4 = json.loads(json.dumps(g1))
g4["name"] = "width_tie"
g4["params"] = {"D": 2, "M": 3, "K": 3, "W": 2, "B": 5, "beta": -0.5}
g4["derivation"] = [
    "Same weights as marginal_ties (no correction, L_base = H).",
    "Depth 1: log-probs over {tok1 ln2, tok0 0, tok2 0}: tok1 -ln2, tok0 = tok2 = -2ln2 exactly. "
    "K = 3 keeps all three children of the root.",
    "Top-W with W = 2: (1) first; (0) and (2) tie exactly on score and are split by the "
    "lexicographic path, so (0) survives and (2) is never expanded.",
    "Depth 2 log-probs over {tok0 ln2, tok1 0, tok2 0}: tok0 -ln2, tok1 = tok2 = -2ln2. "
    "Children of (1): (1,0) -2ln2, (1,1) -3ln2, (1,2) -3ln2; of (0): (0,0) -3ln2, "
    "(0,1) -4ln2, (0,2) -4ln2.",
    "keys = score - 0.5*depth: (1) -ln2-0.5, (0) = (2) -2ln2-0.5, (1,0) -2ln2-1, then a three-way "
    "exact tie at -3ln2-1 among (0,0), (1,1), (1,2), broken by path: (0,0). B = 5 takes "
    "(1), (0), (2), (1,0), (0,0).",
    "Canonical order: root, (0), (1), (2), (0,0), (1,0)."]
g4["expect"] = {"n_nodes": 6, "tok": [3, 0, 1, 2, 0, 0], "parent": [-1, 0, 0, 0, 1, 2],
                "depth": [0, 1, 1, 1, 2, 2],
                "score": ["0", "-2*ln2", "-ln2", "-2*ln2", "-3*ln2", "-2*ln2"],
                "mask": [[1, 0, 0, 0, 0, 0], [1, 1, 0, 0, 0, 0], [1, 0, 1, 0, 0, 0],
                         [1, 0, 0, 1, 0, 0], [1, 1, 0, 0, 1, 0], [1, 0, 1, 0, 0, 1]]}

if __name__ == "__main__":
    for g in (g1, g2, g3, g4):
        with open(os.path.join(HERE, f"{g['name']}.json"), "w") as f:
            json.dump(g, f, indent=1)
