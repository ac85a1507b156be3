// K4: deferred pruning and the compact verification tree.
//
// DARTree page, Methodology 2: after the superarbol is built, ONE global
// Top-B over all its materialised prefixes (root excluded) replaces the
// sequential best-first heap; with a non-positive depth bonus beta the key
// score + beta * depth never increases from a node to its children, which
// is why (Lemma 1) the selected set equals the heap's and is closed under
// parents.  The selected nodes are emitted in canonical order (depth, then
// token path), parents re-indexed, with the ancestor-or-self mask that
// tree-attention verification uses ("Resumen Técnico: DominoTree", Main
// components 5).  The closure is checked; a violation sets status bit 0.
#include "common.hpp"
#include "kernels.hpp"

namespace dtree {

constexpr int TB_THREADS = 1024;

__global__ __launch_bounds__(TB_THREADS) void k_topb_emit(int NT, int B, float beta, int Bmax,
                                                          TreeBufs t, int32_t *__restrict__ otok,
                                                          int32_t *__restrict__ opar,
                                                          int32_t *__restrict__ odep,
                                                          float *__restrict__ oscore,
                                                          uint8_t *__restrict__ omask,
                                                          int32_t *__restrict__ on_nodes) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int q = blockIdx.x, tid = threadIdx.x;
  const int Nsa = NT - 1;
  const int Bsel = B < Nsa ? B : Nsa;
  const int npad = next_pow2(Nsa > 1 ? Nsa : 1);
  const int N = B + 1;
  const int nn = Bsel + 1;
  const size_t nb = (size_t)q * t.NT;   // workspace stride (caps), NT = this round's nodes

  uint64_t *keys = reinterpret_cast<uint64_t *>(smem);        // [npad]
  int32_t *ids = reinterpret_cast<int32_t *>(keys + npad);    // [npad]
  int16_t *map = reinterpret_cast<int16_t *>(ids + npad);     // [NT] node -> out index
  int32_t *onode = reinterpret_cast<int32_t *>(map + ((NT + 1) & ~1));  // [N] out -> node
  int32_t *opar_s = onode + N;                                 // [N]
  uint32_t *canon = reinterpret_cast<uint32_t *>(opar_s + N);  // [Bsel]

  // selection keys: fp32 key = score + beta*depth, rounded after each op
  for (int i = tid; i < npad; i += blockDim.x) {
    uint64_t k = 0;
    if (i < Nsa) {
      const int n = i + 1;
      const int dep = t.n_dep[nb + n];
      const float key = __fadd_rn(t.n_score[nb + n], __fmul_rn(beta, (float)dep));
      k = make_key(key, ((uint32_t)dep << 27) | t.n_lex[nb + n]);
    }
    keys[i] = k;
    ids[i] = i + 1;
  }
  for (int i = tid; i < NT; i += blockDim.x) map[i] = -1;
  __syncthreads();
  block_bitonic_desc(keys, ids, npad);

  // canonical order of the selected nodes: (depth, lexicographic path)
  for (int i = tid; i < Bsel; i += blockDim.x) {
    const int n = ids[i];
    canon[i] = ((uint32_t)t.n_dep[nb + n] << 27) | t.n_lex[nb + n];
    t.sel[(size_t)q * Bmax + i] = n;
  }
  for (int i = Bsel + tid; i < Bmax; i += blockDim.x) t.sel[(size_t)q * Bmax + i] = -1;
  __syncthreads();
  for (int i = tid; i < Bsel; i += blockDim.x) {
    const uint32_t ci = canon[i];
    int rank = 0;
    for (int j = 0; j < Bsel; ++j) rank += canon[j] < ci;
    map[ids[i]] = (int16_t)(1 + rank);
    onode[1 + rank] = ids[i];
  }
  if (tid == 0) { map[0] = 0; onode[0] = 0; }
  __syncthreads();

  // outputs, parent re-indexing and the closure check
  for (int i = tid; i < N; i += blockDim.x) {
    const size_t o = (size_t)q * N + i;
    if (i < nn) {
      const int n = onode[i];
      const int pn = t.n_par[nb + n];
      int pi = -1;
      if (i > 0) {
        pi = map[pn];
        if (pi < 0) atomicOr(t.status, 1u);
      }
      otok[o] = t.n_tok[nb + n];
      opar[o] = pi;
      odep[o] = t.n_dep[nb + n];
      oscore[o] = t.n_score[nb + n];
      opar_s[i] = pi;
    } else {
      otok[o] = -1; opar[o] = -1; odep[o] = -1; oscore[o] = -INFINITY;
      opar_s[i] = -1;
    }
  }
  if (tid == 0) on_nodes[q] = nn;
  __syncthreads();

  // mask[i][j] = 1 iff j is i or an ancestor of i (one wave per row)
  const int lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
  uint8_t *mq = omask + (size_t)q * N * N;
  for (int i = wave; i < N; i += nw) {
    int chain[32];
    int len = 0;
    if (i < nn) {
      int x = i;
      while (x >= 0 && len < 32) { chain[len++] = x; x = opar_s[x]; }
    }
    for (int j = lane; j < N; j += 64) {
      uint8_t v = 0;
      for (int c = 0; c < len; ++c) v |= (uint8_t)(chain[c] == j);
      mq[(size_t)i * N + j] = v;
    }
  }
}

size_t topb_smem(int NT, int B) {
  const int Nsa = NT - 1;
  int npad = 1;
  while (npad < Nsa) npad <<= 1;
  const int N = B + 1;
  return (size_t)npad * 12 + (size_t)((NT + 1) & ~1) * 2 + (size_t)N * 8 + (size_t)B * 4 + 16;
}

hipError_t topb_prepare(size_t smem) {
  return hipFuncSetAttribute(reinterpret_cast<const void *>(&k_topb_emit),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
}

hipError_t launch_topb_emit(int b, int NT, int B, float beta, int Bmax, const TreeBufs &t,
                            int32_t *tok, int32_t *parent, int32_t *depth, float *score,
                            uint8_t *mask, int32_t *n_nodes, hipStream_t st) {
  hipLaunchKernelGGL(k_topb_emit, dim3(b), dim3(TB_THREADS), topb_smem(NT, B), st, NT, B, beta,
                     Bmax, t, tok, parent, depth, score, mask, n_nodes);
  return hipGetLastError();
}

}  // namespace dtree
