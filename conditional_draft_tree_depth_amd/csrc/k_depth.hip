// Per-depth kernels of the depth-wise build (DARTree page, Methodology 1):
// batched correction of every active branch, per-branch log-softmax and
// Top-K children, and the Top-W survivors of the depth.
//
// Node ids of one request's superarbol: 0 is the root; the children created
// at depth delta+1 occupy [off, off + A*K), child (a, k) = off + a*K + k for
// expanded branch slot a and rank k.  Each node keeps a lexicographic key
// lex = (rank of its parent's token path among that depth's expanded
// nodes) << 18 | token, which orders same-depth nodes by token path.
#include "common.hpp"
#include "kernels.hpp"

namespace dtree {

constexpr int SEL_THREADS = 256;
constexpr int SEL_MAXZ = 1024;   // children per request and depth
constexpr int SEL_MAXW = 512;

// Corrected logits of the depth's candidates for every expanded branch:
//   ell[a][j] = Cl[j] + W2[C[j]] . u_a
// ("Resumen Técnico: Domino", Methodology 2: L = L_base + Delta L with the
// low-rank map back to the vocabulary; "Resumen Técnico: DominoTree", Main
// components 2: only the r x M slice of W2 for the Top-M candidates is
// used).  One workgroup per request stages that slice and the branches' u
// vectors in LDS.
template <typename WT>
__global__ __launch_bounds__(256) void k_corr_logits(int A, int M, int r, int D, int delta,
                                                     const WT *__restrict__ W2,
                                                     const int32_t *__restrict__ C,
                                                     const float *__restrict__ Cl,
                                                     const float *__restrict__ u,
                                                     float *__restrict__ ell) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int q = blockIdx.x;
  const int rs = r + (sizeof(WT) == 2 ? 2 : 1);   // skewed row stride
  WT *W2s = reinterpret_cast<WT *>(smem);
  size_t w2bytes = ((size_t)M * rs * sizeof(WT) + 15) & ~(size_t)15;
  float *us = reinterpret_cast<float *>(smem + w2bytes);
  const int32_t *toks = C + ((size_t)q * D + delta) * M;
  for (int i = threadIdx.x; i < M * r; i += blockDim.x) {
    const int j = i / r, tt = i - j * r;
    const int tk = toks[j] < 0 ? 0 : toks[j];   // an empty slot never reaches here
    W2s[j * rs + tt] = W2[(size_t)tk * r + tt];
  }
  const float *uq = u + (size_t)q * A * r;
  for (int i = threadIdx.x; i < A * r; i += blockDim.x) us[i] = uq[i];
  __syncthreads();
  const float *clq = Cl + ((size_t)q * D + delta) * M;
  for (int o = threadIdx.x; o < A * M; o += blockDim.x) {
    const int a = o / M, j = o - a * M;
    const WT *w = W2s + j * rs;
    const float *ua = us + a * r;
    float acc = 0.f;
    for (int tt = 0; tt < r; ++tt) acc += wload(w, tt) * ua[tt];
    ell[((size_t)q * A + a) * M + j] = clq[j] + acc;
  }
}

size_t corr_logits_smem(int A, int M, int r, int wtype) {
  const size_t es = wtype == WT_BF16 ? 2 : 4;
  const size_t rs = r + (wtype == WT_BF16 ? 2 : 1);
  return (((size_t)M * rs * es + 15) & ~(size_t)15) + (size_t)A * r * 4;
}

hipError_t corr_logits_prepare(int wtype, size_t smem) {
  if (wtype == WT_BF16)
    return hipFuncSetAttribute(reinterpret_cast<const void *>(&k_corr_logits<uint16_t>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  return hipFuncSetAttribute(reinterpret_cast<const void *>(&k_corr_logits<float>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
}

hipError_t launch_corr_logits(int b, int A, int M, int r, int D, int delta, const void *W2,
                              int wtype, const int32_t *C, const float *Cl, const float *u,
                              float *ell, hipStream_t st) {
  const size_t sm = corr_logits_smem(A, M, r, wtype);
  if (wtype == WT_BF16)
    hipLaunchKernelGGL(k_corr_logits<uint16_t>, dim3(b), dim3(256), sm, st, A, M, r, D, delta,
                       static_cast<const uint16_t *>(W2), C, Cl, u, ell);
  else
    hipLaunchKernelGGL(k_corr_logits<float>, dim3(b), dim3(256), sm, st, A, M, r, D, delta,
                       static_cast<const float *>(W2), C, Cl, u, ell);
  return hipGetLastError();
}

// Selection of one depth for one request (one workgroup each):
//  1. per expanded branch (one wave each): log-softmax over the M corrected
//     logits, Top-K children (log-prob desc, token asc), child score =
//     parent score + log-prob; every child is appended to the superarbol
//     ("Resumen Técnico: DominoTree", Main components 2; DARTree page,
//     Methodology 1, scoring by corrected cumulative probability);
//  2. Top-W of the depth's children by (score desc, token path asc) become
//     the next expanded branches (DARTree page, Methodology 1, retention);
//  3. the survivors' lexicographic ranks among themselves, and the gathers
//     the GRU step needs (token and parent state slot).
__global__ __launch_bounds__(SEL_THREADS) void k_select(int A, int M, int K, int W, int D,
                                                        int delta, int off,
                                                        const int32_t *__restrict__ C,
                                                        const float *__restrict__ ell,
                                                        TreeBufs t) {
  __shared__ uint64_t ckey[SEL_MAXZ];
  __shared__ uint32_t clex[SEL_MAXZ];
  __shared__ uint32_t slex[SEL_MAXW];
  const int q = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const int32_t *cq = C + ((size_t)q * D + delta) * M;
  const size_t nb = (size_t)q * t.NT;
  const int Z = A * K;
  const int An = Z < W ? Z : W;

  for (int a = wave; a < A; a += nw) {
    const int p = t.surv_node[(size_t)q * t.Wmax + a];
    const uint32_t prank = (uint32_t)t.surv_rank[(size_t)q * t.Wmax + a];
    const float pscore = t.n_score[nb + p];
    const float *la = ell + ((size_t)q * A + a) * M;
    const bool h0 = lane < M, h1 = lane + 64 < M;
    const float l0 = h0 ? la[lane] : -INFINITY;
    const float l1 = h1 ? la[lane + 64] : -INFINITY;
    const float m = wave_max_f32(fmaxf(l0, l1));
    const float e = (h0 ? expf(l0 - m) : 0.f) + (h1 ? expf(l1 - m) : 0.f);
    const float lse = m + logf(wave_sum_f32(e));
    uint64_t k0 = h0 ? make_key(l0 - lse, (uint32_t)cq[lane]) : 0ull;
    uint64_t k1 = h1 ? make_key(l1 - lse, (uint32_t)cq[lane + 64]) : 0ull;
    for (int k = 0; k < K; ++k) {
      const uint64_t top = group_max_u64<64>(k0 > k1 ? k0 : k1);
      if (k0 == top) k0 = 0ull;
      if (k1 == top) k1 = 0ull;
      if (lane == 0) {
        const uint32_t tok = key_tie(top);
        const float lp = key_val(top);
        const float sc = __fadd_rn(pscore, lp);
        const uint32_t lex = (prank << 18) | tok;
        const int c = a * K + k;
        const size_t id = nb + off + c;
        t.n_tok[id] = (int32_t)tok;
        t.n_par[id] = p;
        t.n_dep[id] = delta + 1;
        t.n_score[id] = sc;
        t.n_lex[id] = lex;
        ckey[c] = make_key(sc, lex);
        clex[c] = lex;
      }
    }
  }
  __syncthreads();

  // Top-W by rank: keys are distinct (distinct token paths)
  for (int c = threadIdx.x; c < Z; c += blockDim.x) {
    const uint64_t kc = ckey[c];
    int rank = 0;
    for (int c2 = 0; c2 < Z; ++c2) rank += ckey[c2] > kc;
    if (rank < An) {
      const size_t sl = (size_t)q * t.Wmax + rank;
      t.nsurv_node[sl] = off + c;
      slex[rank] = clex[c];
      t.gidx_tok[(size_t)q * An + rank] = (int32_t)(clex[c] & 0x3FFFFu);
      t.gidx_par[(size_t)q * An + rank] = q * A + c / K;
      t.surv_hist[((size_t)q * (D + 1) + delta + 1) * t.Wmax + rank] = off + c;
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < An; i += blockDim.x) {
    const uint32_t li = slex[i];
    int rank = 0;
    for (int j = 0; j < An; ++j) rank += slex[j] < li;
    t.nsurv_rank[(size_t)q * t.Wmax + i] = rank;
  }
}

hipError_t launch_select(int b, int A, int M, int K, int W, int D, int delta, int off,
                         const int32_t *C, const float *ell, const TreeBufs &t,
                         hipStream_t st) {
  hipLaunchKernelGGL(k_select, dim3(b), dim3(SEL_THREADS), 0, st, A, M, K, W, D, delta, off, C,
                     ell, t);
  return hipGetLastError();
}

}  // namespace dtree
