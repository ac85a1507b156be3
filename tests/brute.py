"""Brute-force path enumerator used to pin the oracle (tests only).

Written independently of ``oracle/``: it uses torch float64 (torch's bf16
cast, ``torch.nn.GRUCell``, ``torch.log_softmax``, the concatenated
[H_i ; S] input of the low-rank head) and walks EVERY token path of length
1..D over the per-depth Top-M candidates, re-running the GRU along each path
from the root, with no state shared between branches of the search except
the prefix it is extending.  Sizes must stay tiny (sum of M^depth paths).
"""
import numpy as np
import torch


def _w(arr, wtype):
    t = torch.from_numpy(np.ascontiguousarray(arr))
    if wtype == "bf16":
        return t.view(torch.bfloat16).to(torch.float64)
    return t.to(torch.float64)


class Brute:
    def __init__(self, inputs, req, D, M):
        w, wtype = inputs["weights"], inputs["wtype"]
        H = torch.from_numpy(np.asarray(inputs["H"][req, :D], np.float32))
        self.Hq = (H.to(torch.bfloat16) if wtype == "bf16" else H).to(torch.float64)
        W_lm = _w(w["W_lm"], wtype)
        self.Lb = self.Hq @ W_lm.T + torch.from_numpy(w["bias"]).to(torch.float64)
        self.V = W_lm.shape[0]
        self.D, self.M = D, M
        # per-depth candidates: plain Python sort, value desc then token asc
        self.C = []
        for dd in range(D):
            row = self.Lb[dd].tolist()
            self.C.append(sorted(range(self.V), key=lambda v: (-row[v], v))[:M])
        s = w["W_hh"].shape[1]
        e = w["W_ih"].shape[1]
        self.gru = torch.nn.GRUCell(e, s, dtype=torch.float64)
        with torch.no_grad():
            self.gru.weight_ih.copy_(_w(w["W_ih"], wtype))
            self.gru.weight_hh.copy_(_w(w["W_hh"], wtype))
            self.gru.bias_ih.copy_(torch.from_numpy(w["b_ih"]).to(torch.float64))
            self.gru.bias_hh.copy_(torch.from_numpy(w["b_hh"]).to(torch.float64))
        self.Emb = _w(w["Emb"], wtype)
        self.W1 = _w(w["W1"], wtype)
        self.W2 = _w(w["W2"], wtype)
        self.root = int(inputs["root"][req])
        self.s = s

    def step_state(self, S, tok):
        with torch.no_grad():
            return self.gru(self.Emb[tok][None, :], S[None, :])[0]

    def child_logprobs(self, dd, S):
        """log-probs over C[dd] for a branch whose causal state is S."""
        u = self.W1 @ torch.cat([self.Hq[dd], S])
        cand = self.C[dd]
        ell = self.Lb[dd][cand] + self.W2[cand] @ u
        return torch.log_softmax(ell, dim=0)

    def enumerate(self):
        """{path tuple: cumulative score} for every path of length 1..D."""
        out = {}
        S0 = self.step_state(torch.zeros(self.s, dtype=torch.float64), self.root)

        def rec(path, S, score, dd):
            if dd == self.D:
                return
            lp = self.child_logprobs(dd, S)
            for j, t in enumerate(self.C[dd]):
                p2 = path + (t,)
                sc = score + float(lp[j])
                out[p2] = sc
                if dd + 1 < self.D:
                    rec(p2, self.step_state(S, t), sc, dd + 1)

        rec((), S0, 0.0, 0)
        return out

    def extensions(self, path):
        """Scores of the M one-token extensions of ``path`` (recomputed from
        the root, GRU re-run along the path)."""
        S = self.step_state(torch.zeros(self.s, dtype=torch.float64), self.root)
        score = 0.0
        for dd, t in enumerate(path):
            lp = self.child_logprobs(dd, S)
            score += float(lp[self.C[dd].index(t)])
            S = self.step_state(S, t)
        lp = self.child_logprobs(len(path), S)
        return {t: float(lp[j]) for j, t in enumerate(self.C[len(path)])}, score

    def enumerate_marginal(self):
        """{path tuple: cumulative score} for every path of length 1..D when
        every branch is scored by the base logits alone (no correction): the
        closed form sum over depths of log_softmax(Lb[dd][C[dd]]) at the
        path's tokens."""
        lps = [torch.log_softmax(self.Lb[dd][self.C[dd]], dim=0) for dd in range(self.D)]
        out = {}

        def rec(path, score, dd):
            if dd == self.D:
                return
            for j, t in enumerate(self.C[dd]):
                p2 = path + (t,)
                out[p2] = score + float(lps[dd][j])
                rec(p2, out[p2], dd + 1)

        rec((), 0.0, 0)
        return out

    def enumerate_markov(self):
        """{path tuple: cumulative score} for every path of length 1..D under
        the first-order (Markov) correction: the children of a node are
        scored with the state the GRU reaches from a zero state after the
        node's own last token alone (the root's token for the root)."""
        zero = torch.zeros(self.s, dtype=torch.float64)
        out = {}

        def rec(path, last_tok, score, dd):
            if dd == self.D:
                return
            lp = self.child_logprobs(dd, self.step_state(zero, last_tok))
            for j, t in enumerate(self.C[dd]):
                p2 = path + (t,)
                out[p2] = score + float(lp[j])
                rec(p2, t, out[p2], dd + 1)

        rec((), self.root, 0.0, 0)
        return out

    def kary_tree(self, K, markov=False):
        """{path: score} of the unpruned K-ary tree of depth D: every node's
        children are the Top-K (log-prob desc, token asc) of its M one-token
        extensions, scores recomputed from scratch along each path."""
        allp = self.enumerate_markov() if markov else self.enumerate()
        out = {}

        def rec(path, dd):
            if dd == self.D:
                return
            ext = {t: allp[path + (t,)] for t in self.C[dd]}
            for t in sorted(ext, key=lambda t: (-ext[t], t))[:K]:
                out[path + (t,)] = ext[t]
                rec(path + (t,), dd + 1)

        rec((), 0)
        return out
