"""CPU oracle for tree-attention verification -- TEST INFRASTRUCTURE ONLY.

Nothing on the product path may import, call or execute this module: only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code with the HIP library.

What it computes.  The draft tree is verified by the target model in one
forward pass with tree attention: every tree token attends to the verified
prefix and to the tree tokens on its own root-to-node path, itself included,
through an ancestor-only mask ("Resumen Técnico: DominoTree", Componentes
Principales 5; "DARTree: Speculative Diffusion Decoding with Autoregressive
Draft Trees", Metodología 2, verification).  This oracle computes one
layer's attention output of that pass for given Q, K, V:

    O[q, i, h] = sum_k  w_k V[q, h // G, k]     over visible keys k,
    w_k = exp(s_k - m) / sum_k' exp(s_k' - m),
    s_k = scale * Q[q, i, h] . K[q, h // G, k],

where key k is visible to tree token i when it is a prefix position
(k < prefix_len[q]) or the tree position prefix_len[q] + j of a node j with
mask[q, i, j] = 1; G = Hq / Hkv query heads share one KV head (grouped-query
attention, query head h reads KV head h // G).  Rows i >= n_nodes[q] are
zero.  float64 throughout; a library matmul is the only primitive.

Along with O it returns  absw[q, i, h, c] = sum_k w_k |V[q, h // G, k, c]|,
the weighted absolute value sum that bounds the effect of rounding the
weights (see ``parity_bound``).
"""
import numpy as np

__all__ = ["ancestor_mask", "tree_attention", "parity_bound", "ATTN_REL_TOL"]

# A kernel that rounds the softmax weights to bf16 (8-bit significand: unit
# roundoff 2^-8, so relative error <= 2^-8) before the weighted sum of V and
# accumulates in fp32 over at most a few thousand keys stays within
# 2^-8 * absw + (fp32 accumulation) of O.
ATTN_REL_TOL = 2.0 ** -8 + 2.5e-4
ATTN_ABS_TOL = 1e-5


def ancestor_mask(parent, n, n_max):
    """Ancestor-or-self mask of a tree in canonical order (parent[i] < i):
    row i holds i and every ancestor of i, the root included; rows and
    columns past n are zero.  Same convention as the round's emitted mask
    (query row, key column)."""
    m = np.zeros((n_max, n_max), np.uint8)
    for i in range(n):
        if i > 0:
            p = int(parent[i])
            if not 0 <= p < i:
                raise ValueError(f"node {i}: parent {p} is not an earlier node")
            m[i] = m[p]
        m[i, i] = 1
    return m


def _bf16(bits):
    a = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return a.view(np.float32).astype(np.float64)


def tree_attention(Q, K, V, prefix_len, n_nodes, mask, scale):
    """Q [b, n_max, Hq, dh], K/V [b, Hkv, L_cap, dh] (float arrays or raw
    bf16 bit patterns as uint16), prefix_len/n_nodes [b], mask
    [b, n_max, n_max].  Returns (O, absw), both [b, n_max, Hq, dh] float64."""
    if np.asarray(Q).dtype == np.uint16:
        Q, K, V = _bf16(Q), _bf16(K), _bf16(V)
    Q, K, V = (np.asarray(x, np.float64) for x in (Q, K, V))
    b, n_max, Hq, dh = Q.shape
    Hkv = K.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    O = np.zeros((b, n_max, Hq, dh))
    absw = np.zeros((b, n_max, Hq, dh))
    for q in range(b):
        P, n = int(prefix_len[q]), int(n_nodes[q])
        L = P + n
        if not (P >= 0 and 1 <= n <= n_max and L <= K.shape[2]):
            raise ValueError(f"request {q}: prefix {P}, nodes {n}")
        visible = np.zeros((n, L), bool)
        visible[:, :P] = True
        visible[:, P:] = np.asarray(mask[q])[:n, :n] != 0
        for h in range(Hq):
            kv = h // G
            s = scale * (Q[q, :n, h, :] @ K[q, kv, :L, :].T)          # [n, L]
            s = np.where(visible, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m)
            w = e / e.sum(axis=1, keepdims=True)
            O[q, :n, h, :] = w @ V[q, kv, :L, :]
            absw[q, :n, h, :] = w @ np.abs(V[q, kv, :L, :])
    return O, absw


def parity_bound(absw):
    """Element-wise tolerance for a kernel that rounds the softmax weights
    to bf16 and accumulates in fp32 (derivation at ATTN_REL_TOL)."""
    return ATTN_REL_TOL * absw + ATTN_ABS_TOL
