// Per-depth kernels of the depth-wise build (DARTree page, Metodología 1):
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

constexpr int SEL_THREADS = 1024;
constexpr int SEL_MAXZ = 1024;   // children per request and depth
constexpr int SEL_MAXW = 512;
constexpr int CL_BR = 4;         // expanded branches per correction workgroup

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
__device__ __forceinline__ f32x4 cl_mfma(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Corrected logits of the depth's candidates for every expanded branch:
//   ell[a][j] = Cl[j] + W2[C[j]] . u_a
// ("Resumen Técnico: Domino", Metodología 2: L = L_base + Delta L with the
// low-rank map back to the vocabulary; "Resumen Técnico: DominoTree", Main
// components 2: only the r x M slice of W2 for the Top-M candidates is
// used).  One workgroup per (request, group of CL_BR branches) stages that
// slice and its branches' u vectors in LDS; with bf16 rows of a multiple of
// 8 the slice moves in 16-byte pieces and every output reads 8 weights at
// a time.
template <typename WT>
__global__ __launch_bounds__(256) void k_corr_logits(int A, int M, int r, int D, int delta,
                                                     int vec, const WT *__restrict__ W2,
                                                     const int32_t *__restrict__ C,
                                                     const float *__restrict__ Cl,
                                                     const float *__restrict__ u, int ldu,
                                                     float *__restrict__ ell) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int q = blockIdx.x, a0 = blockIdx.y * CL_BR;
  const int na = min(CL_BR, A - a0);
  constexpr bool B16 = sizeof(WT) == 2;   // vec: bf16, r % 8 == 0, W2 16-byte aligned
  const int rs = vec ? r + 8 : r + (B16 ? 2 : 1);   // row stride (skewed when scalar)
  WT *W2s = reinterpret_cast<WT *>(smem);
  size_t w2bytes = ((size_t)M * rs * sizeof(WT) + 15) & ~(size_t)15;
  float *us = reinterpret_cast<float *>(smem + w2bytes);
  const int32_t *toks = C + ((size_t)q * D + delta) * M;
  if (vec) {
    const int r8 = r >> 3;
    for (int i = threadIdx.x; i < M * r8; i += blockDim.x) {
      const int j = i / r8, c8 = i - j * r8;
      const int tk = toks[j] < 0 ? 0 : toks[j];   // an empty slot never reaches here
      *reinterpret_cast<uint4 *>(W2s + j * rs + 8 * c8) =
          *reinterpret_cast<const uint4 *>(W2 + (size_t)tk * r + 8 * c8);
    }
  } else {
    for (int i = threadIdx.x; i < M * r; i += blockDim.x) {
      const int j = i / r, tt = i - j * r;
      const int tk = toks[j] < 0 ? 0 : toks[j];
      W2s[j * rs + tt] = W2[(size_t)tk * r + tt];
    }
  }
  const float *uq = u + ((size_t)q * A + a0) * ldu;
  for (int i = threadIdx.x; i < na * r; i += blockDim.x) {
    const int a = i / r;
    us[i] = uq[(size_t)a * ldu + (i - a * r)];
  }
  __syncthreads();
  const float *clq = Cl + ((size_t)q * D + delta) * M;
  for (int o = threadIdx.x; o < na * M; o += blockDim.x) {
    const int a = o / M, j = o - a * M;
    const WT *w = W2s + j * rs;
    const float *ua = us + a * r;
    float acc = 0.f;
    if (vec) {
      for (int c8 = 0; c8 < r; c8 += 8) {
        const uint4 wv = *reinterpret_cast<const uint4 *>(w + c8);
        const float4 u0 = *reinterpret_cast<const float4 *>(ua + c8);
        const float4 u1 = *reinterpret_cast<const float4 *>(ua + c8 + 4);
        acc += __uint_as_float(wv.x << 16) * u0.x;
        acc += __uint_as_float(wv.x & 0xFFFF0000u) * u0.y;
        acc += __uint_as_float(wv.y << 16) * u0.z;
        acc += __uint_as_float(wv.y & 0xFFFF0000u) * u0.w;
        acc += __uint_as_float(wv.z << 16) * u1.x;
        acc += __uint_as_float(wv.z & 0xFFFF0000u) * u1.y;
        acc += __uint_as_float(wv.w << 16) * u1.z;
        acc += __uint_as_float(wv.w & 0xFFFF0000u) * u1.w;
      }
    } else {
      for (int tt = 0; tt < r; ++tt) acc += wload(w, tt) * ua[tt];
    }
    ell[((size_t)q * A + a0 + a) * M + j] = clq[j] + acc;
  }
}

// The same logits on the matrix cores (bf16 W2 with 16-byte rows, r a
// multiple of 8): workgroups of 4 waves per (request, 16 branches, 64
// candidates), one 16 x 16 tile (candidates x branches) per wave.  A wave
// issues the u values and W2 fragments of up to 8 k steps of 32 at once
// (straight from memory: W2 rows by candidate token), then splits each
// lane's 8 u values exactly into three bf16 terms (W2 is bf16, so every
// product is exact in fp32) and runs the MFMAs.
constexpr int CLM_KB = 8;   // k steps per batch of loads
__global__ __launch_bounds__(256) void k_corr_logits_mfma(int A, int M, int r, int D, int delta,
                                                          const uint16_t *__restrict__ W2,
                                                          const int32_t *__restrict__ C,
                                                          const float *__restrict__ Cl,
                                                          const float *__restrict__ u, int ldu,
                                                          float *__restrict__ ell) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, lr = lane & 15, g = lane >> 4;
  const int q = blockIdx.x, a = blockIdx.y * 16 + lr, jt = blockIdx.z * 4 + wave;
  if (jt * 16 >= M) return;   // (no barrier in this kernel)
  const int32_t *toks = C + ((size_t)q * D + delta) * M;
  const float *clq = Cl + ((size_t)q * D + delta) * M;
  const float *ua = u + ((size_t)q * A + min(a, A - 1)) * ldu;
  const int j = min(jt * 16 + lr, M - 1);
  const uint16_t *wr = W2 + (size_t)max(toks[j], 0) * r;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < r; k0 += 32 * CLM_KB) {
    // loads from clamped addresses, always in bounds, then masked: no
    // branch between them
    float x[CLM_KB][8];
    uint4 wa[CLM_KB];
#pragma unroll
    for (int st = 0; st < CLM_KB; ++st) {
      const int kk = k0 + 32 * st + 8 * g;   // r % 8 == 0: 8 elements all in or all out
      const int kc = min(kk, r - 8);
      const bool in = kk < r;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = ua[kc + e];
        x[st][e] = (in && a < A) ? v : 0.f;
      }
      const uint4 w = *reinterpret_cast<const uint4 *>(wr + kc);
      wa[st] = in ? w : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int st = 0; st < CLM_KB; ++st) {
      uint4 t3[3];
      split3_bf16(x[st], t3);
#pragma unroll
      for (int tq = 0; tq < 3; ++tq) acc = cl_mfma(wa[st], t3[tq], acc);
    }
  }
  // lane holds D[candidate 4 g + t][branch lr]
  if (a < A) {
    float *eq = ell + ((size_t)q * A + a) * M;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const int jj = jt * 16 + 4 * g + tt;
      if (jj < M) eq[jj] = clq[jj] + acc[tt];
    }
  }
}

size_t corr_logits_smem(int A, int M, int r, int wtype) {
  const size_t es = wtype == WT_BF16 ? 2 : 4;
  const size_t rs = wtype == WT_BF16 ? (r % 8 == 0 ? r + 8 : r + 2) : r + 1;
  return (((size_t)M * rs * es + 15) & ~(size_t)15) + (size_t)(A < CL_BR ? A : CL_BR) * r * 4;
}

hipError_t corr_logits_prepare(int wtype, size_t lds_bytes) {
  if (wtype == WT_BF16)
    return set_lds_limit(reinterpret_cast<const void *>(&k_corr_logits<uint16_t>), lds_bytes);
  return set_lds_limit(reinterpret_cast<const void *>(&k_corr_logits<float>), lds_bytes);
}

hipError_t launch_corr_logits(int b, int A, int M, int r, int D, int delta, const void *W2,
                              int wtype, const int32_t *C, const float *Cl, const float *u,
                              int ldu, float *ell, hipStream_t st) {
  const size_t sm = corr_logits_smem(A, M, r, wtype);
  const dim3 grid(b, (A + CL_BR - 1) / CL_BR);
  const int vec = wtype == WT_BF16 && r % 8 == 0 && reinterpret_cast<uintptr_t>(W2) % 16 == 0;
  if (vec) {
    hipLaunchKernelGGL(k_corr_logits_mfma, dim3(b, (A + 15) / 16, (M + 63) / 64), dim3(256), 0, st,
                       A, M, r, D, delta, static_cast<const uint16_t *>(W2), C, Cl, u, ldu, ell);
    return hipGetLastError();
  }
  if (wtype == WT_BF16)
    hipLaunchKernelGGL(k_corr_logits<uint16_t>, grid, dim3(256), sm, st, A, M, r, D, delta, vec,
                       static_cast<const uint16_t *>(W2), C, Cl, u, ldu, ell);
  else
    hipLaunchKernelGGL(k_corr_logits<float>, grid, dim3(256), sm, st, A, M, r, D, delta, 0,
                       static_cast<const float *>(W2), C, Cl, u, ldu, ell);
  return hipGetLastError();
}

// Ranks of one branch's candidates, held by one wave (lane l: candidate l
// in k0, candidate l + 64 in k1; keys are distinct): the keys go through
// the wave's LDS row wk and every lane counts the larger ones.
__device__ __forceinline__ void branch_ranks(uint64_t k0, uint64_t k1, bool h0, bool h1, int M,
                                             uint64_t *wk, int lane, int &r0, int &r1) {
  if (h0) wk[lane] = k0;
  if (h1) wk[lane + 64] = k1;
  // LDS accesses of one wave take effect in issue order
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  r0 = 0;
  r1 = 0;
  int j = 0;
  for (; j + 8 <= M; j += 8) {
    uint64_t v[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) v[t] = wk[j + t];
#pragma unroll
    for (int t = 0; t < 8; ++t) { r0 += v[t] > k0; r1 += v[t] > k1; }
  }
  for (; j < M; ++j) { const uint64_t v = wk[j]; r0 += v > k0; r1 += v > k1; }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Number of the n keys in LDS greater than kc (8 loads in flight at a time).
template <class T>
__device__ __forceinline__ int count_greater(const T *keys, int n, T kc) {
  int r = 0, j = 0;
  for (; j + 8 <= n; j += 8) {
    T v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = keys[j + u];
#pragma unroll
    for (int u = 0; u < 8; ++u) r += v[u] > kc;
  }
  for (; j < n; ++j) r += keys[j] > kc;
  return r;
}

// Selection of one depth for one request (one workgroup each):
//  0. the expanded branches' node ids, lexicographic ranks and scores are
//     gathered into LDS once (two dependent loads for all branches at once);
//  1. per expanded branch (one wave each; the next branch's logits are
//     loaded while the current one is processed): log-softmax over the M
//     corrected logits, Top-K children (log-prob desc, token asc) by rank
//     counting, child score = parent score + log-prob; every child is
//     appended to the
//     superarbol ("Resumen Técnico: DominoTree", Componentes Principales 2; DARTree
//     page, Metodología 1, scoring by corrected cumulative probability);
//  2. Top-W of the depth's children by (score desc, token path asc) become
//     the next expanded branches (DARTree page, Metodología 1, retention);
//  3. the survivors' lexicographic ranks among themselves, and the gathers
//     the GRU step needs (token and parent state slot).
__global__ __launch_bounds__(SEL_THREADS) void k_select(int A, int M, int K, int W, int D,
                                                        int delta, int off,
                                                        const int32_t *__restrict__ C,
                                                        const float *__restrict__ ell, long ldq,
                                                        int lda, TreeBufs t) {
  __shared__ uint64_t ckey[SEL_MAXZ];
  __shared__ uint32_t clex[SEL_MAXZ];
  __shared__ uint32_t slex[SEL_MAXW];
  __shared__ int32_t pnode[SEL_MAXW];
  __shared__ uint32_t prank[SEL_MAXW];
  __shared__ float pscore[SEL_MAXW];
  __shared__ int32_t ctok[128];
  __shared__ uint64_t wkeys[(SEL_THREADS / 64) * 128];   // one row of keys per wave
  __shared__ int16_t cidx[SEL_MAXZ];                      // children's candidate index
  const int q = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int nw = blockDim.x >> 6;
  const int32_t *cq = C + ((size_t)q * D + delta) * M;
  const size_t nb = (size_t)q * t.NT;
  const int Z = A * K;
  const int An = Z < W ? Z : W;

  for (int a = tid; a < A; a += blockDim.x) {
    const int p = t.surv_node[(size_t)q * t.Wmax + a];
    pnode[a] = p;
    prank[a] = (uint32_t)t.surv_rank[(size_t)q * t.Wmax + a];
    pscore[a] = t.n_score[nb + p];
  }
  for (int j = tid; j < M; j += blockDim.x) ctok[j] = cq[j];
  const bool h0 = lane < M, h1 = lane + 64 < M;
  float l0 = -INFINITY, l1 = -INFINITY;
  if (wave < A) {
    const float *la = ell + q * ldq + (size_t)wave * lda;
    if (h0) l0 = la[lane];
    if (h1) l1 = la[lane + 64];
  }
  __syncthreads();
  for (int a = wave; a < A; a += nw) {
    float n0 = -INFINITY, n1 = -INFINITY;   // the wave's next branch, in flight meanwhile
    if (a + nw < A) {
      const float *ln = ell + q * ldq + (size_t)(a + nw) * lda;
      if (h0) n0 = ln[lane];
      if (h1) n1 = ln[lane + 64];
    }
    const int p = pnode[a];
    const uint32_t pr = prank[a];
    const float ps = pscore[a];
    const float m = wave_max_f32(fmaxf(l0, l1));
    const float e = (h0 ? expf(l0 - m) : 0.f) + (h1 ? expf(l1 - m) : 0.f);
    const float lse = m + logf(wave_sum_f32(e));
    const uint64_t k0 = h0 ? make_key(l0 - lse, (uint32_t)ctok[lane]) : 0ull;
    const uint64_t k1 = h1 ? make_key(l1 - lse, (uint32_t)ctok[lane + 64]) : 0ull;
    // Top-K by rank; each selected candidate's lane writes its child
    int r0, r1;
    branch_ranks(k0, k1, h0, h1, M, wkeys + wave * 128, lane, r0, r1);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint64_t kk = h ? k1 : k0;
      const int rk = h ? r1 : r0;
      if ((h ? h1 : h0) && rk < K) {
        const uint32_t tok = key_tie(kk);
        const float lp = key_val(kk);
        const float sc = __fadd_rn(ps, lp);
        const uint32_t lex = (pr << 18) | tok;
        const int c = a * K + rk;
        const size_t id = nb + off + c;
        t.n_tok[id] = (int32_t)tok;
        t.n_par[id] = p;
        t.n_dep[id] = delta + 1;
        t.n_score[id] = sc;
        t.n_lex[id] = lex;
        ckey[c] = make_key(sc, lex);
        clex[c] = lex;
        cidx[c] = (int16_t)(lane + 64 * h);
      }
    }
    l0 = n0;
    l1 = n1;
  }
  __syncthreads();

  // Top-W by rank: keys are distinct (distinct token paths)
  for (int c = tid; c < Z; c += blockDim.x) {
    const uint64_t kc = ckey[c];
    const int rank = count_greater<uint64_t>(ckey, Z, kc);
    if (rank < An) {
      const size_t sl = (size_t)q * t.Wmax + rank;
      t.nsurv_node[sl] = off + c;
      slex[rank] = clex[c];
      t.gidx_tok[(size_t)q * An + rank] = (int32_t)(clex[c] & 0x3FFFFu);
      t.gidx_par[(size_t)q * An + rank] = q * A + c / K;
      if (t.gidx_cand) t.gidx_cand[(size_t)q * An + rank] = (q * D + delta) * M + cidx[c];
      t.surv_hist[((size_t)q * (D + 1) + delta + 1) * t.Wmax + rank] = off + c;
    }
  }
  __syncthreads();
  for (int i = tid; i < An; i += blockDim.x) {
    const uint32_t li = slex[i];
    const int rank = An - 1 - count_greater<uint32_t>(slex, An, li);   // lex keys are distinct
    t.nsurv_rank[(size_t)q * t.Wmax + i] = rank;
  }
}

// ---------------------------------------------------------------- batched selection
// The selection of one depth spread over many workgroups (bf16 W2 with
// 16-byte rows, r a multiple of 8 up to 512, M <= 128):
//  k_branch_topk, one workgroup per (request, BS_BR expanded branches), one
//    wave per branch: the branches' correction logits on the matrix cores,
//    log-softmax over the M candidates and the Top-K children, appended to
//    the superarbol, each child's (score, token path) key written out;
//  then the last of a request's workgroups to finish takes the Top-W
//    survivors among those keys (no second launch: a launch costs several
//    microseconds here, more than the arrival count and the reload).
// Same arithmetic, keys and tie-breaks as k_select
// ("Resumen Técnico: DominoTree", Componentes Principales 2; DARTree page,
// Metodología 1).
// (8 branches per workgroup: the wide tree's depth loop took 362 us, 392 us
// with 16, whose single workgroup per request at 16 branches saved nothing on
// the 8B x 8 shape)
constexpr int BS_BR = 8;
constexpr int SEL_FLAGS = 64;   // arrival flags per request (at least SEL_MAXW / BS_BR)

// Ranks of the K best of a wave's candidates, by log-prob descending and
// token ascending (the order of make_key(lp, token)); lane l holds
// candidates l (v0, t0) and l + 64 (v1, t1), absent ones as -inf.  K rounds:
// the wave-wide maximum of the lanes' best remaining log-probs, the lanes
// holding it, and among several such lanes the smallest token (tokens of a
// depth's candidates are distinct).  r0 / r1 = K when not among the K best.
__device__ __forceinline__ void wave_topk(float v0, uint32_t t0, float v1, uint32_t t1, int K,
                                          int &r0, int &r1) {
  const int lane = threadIdx.x & 63;
  int a0 = K, a1 = K;
  for (int rk = 0; rk < K; ++rk) {
    const bool s1 = v1 > v0 || (v1 == v0 && t1 < t0);
    const float bv = s1 ? v1 : v0;
    const uint32_t bt = s1 ? t1 : t0;
    const float m = __builtin_bit_cast(
        float, __builtin_amdgcn_readfirstlane(__float_as_uint(wave_max_f32_full(bv))));
    if (m == -INFINITY) break;
    uint64_t at = __ballot(bv == m);
    if (__popcll(at) > 1) {   // equal log-probs: the smallest token first
      uint32_t tt = bv == m ? bt : 0xFFFFFFFFu;
      tt = min(tt, xchg_u32<1>(tt));
      tt = min(tt, xchg_u32<2>(tt));
      tt = min(tt, xchg_u32<4>(tt));
      tt = min(tt, xchg_u32<8>(tt));
      tt = min(tt, xchg_u32<16>(tt));
      tt = min(tt, xchg_u32<32>(tt));
      at = __ballot(bv == m && bt == tt);
    }
    const bool win = lane == (int)__builtin_ctzll(at);
    a0 = win && !s1 ? rk : a0;
    a1 = win && s1 ? rk : a1;
    v0 = win && !s1 ? -INFINITY : v0;
    v1 = win && s1 ? -INFINITY : v1;
  }
  r0 = a0;
  r1 = a1;
}

// Top-W of one request's Z = A K children by (score desc, token path asc),
// by the NT threads of one workgroup.  The An-th largest key is at least tau, the An-th largest among
// the first m = ceil(An / A) children of every branch (A m >= An keys), so
// only the keys >= tau are ranked: with full-width depths tau is the weakest
// of the branches' best children.
struct TopwLds {
  uint64_t key[SEL_MAXZ];   // the request's children's keys
  uint64_t pk[SEL_MAXZ];
  int16_t cc[SEL_MAXZ];     // their candidate indices
  int16_t pc[SEL_MAXZ];
  uint32_t slex[SEL_MAXW];  // survivors by slot: token path
  int16_t sc[SEL_MAXW];     //   and child index
  uint64_t tau;
  int np;
};
// (the caller has put the Z keys and candidate indices into L.key / L.cc
// and cleared L.tau and L.np, all before a barrier)
template <int NT>
__device__ void topw_request(int q, int A, int K, int W, int D, int delta, int off, int M,
                             const TreeBufs &t, TopwLds &L) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int Z = A * K, An = Z < W ? Z : W;
  uint64_t tau = 0ull;
  if (An < Z && An == A) {
    // full width (m = 1): tau is the weakest of the branches' best children,
    // found by every wave on its own (no barrier)
    uint64_t v = ~0ull;
    for (int a2 = lane; a2 < A; a2 += 64) {
      const uint64_t k = L.key[a2 * K];
      v = k < v ? k : v;
    }
    v = ~group_max_u64<16>(~v);
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const uint32_t hi = (uint32_t)(v >> 32), lo = (uint32_t)v;
      const auto h = x ? __builtin_amdgcn_permlane32_swap(hi, hi, false, false)
                       : __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
      const auto l = x ? __builtin_amdgcn_permlane32_swap(lo, lo, false, false)
                       : __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
      const uint64_t k0 = ((uint64_t)h[0] << 32) | l[0], k1 = ((uint64_t)h[1] << 32) | l[1];
      v = k0 < k1 ? k0 : k1;
    }
    tau = v;
  } else if (An < Z) {
    const int m = (An + A - 1) / A, ns = A * m;
    for (int i = tid; i < ns; i += NT) L.pk[i] = L.key[(i / m) * K + i % m];
    __syncthreads();
    const int tpn = split_width(ns, NT), part = tid & (tpn - 1);
    for (int b0 = 0; b0 < ns; b0 += NT / tpn) {
      const int i = b0 + tid / tpn;
      const uint64_t kc = i < ns ? L.pk[i] : 0ull;
      int cnt = i < ns ? count_split<true>(L.pk, ns, kc, part, tpn) : 0;
      cnt = sum_adjacent(cnt, tpn);
      if (i < ns && part == 0 && cnt == An - 1) L.tau = kc;   // keys are distinct: one thread
    }
    __syncthreads();
    tau = L.tau;
  }
  for (int c0 = 0; c0 < Z; c0 += NT) {
    const int c = c0 + tid;
    const bool keep = c < Z && L.key[c] >= tau;
    const uint64_t bal = __ballot(keep);
    int base = 0;
    if (lane == 0 && bal) base = atomicAdd(&L.np, __popcll(bal));
    base = __shfl(base, 0);
    if (keep) {
      const int at = base + __popcll(bal & ((1ull << lane) - 1ull));
      L.pk[at] = L.key[c];
      L.pc[at] = (int16_t)c;
    }
  }
  __syncthreads();
  const int np = L.np;
  const int tpn = split_width(np, NT), part = tid & (tpn - 1);
  for (int b0 = 0; b0 < np; b0 += NT / tpn) {
    const int i = b0 + tid / tpn;
    const uint64_t ki = i < np ? L.pk[i] : 0ull;
    int rank = i < np ? count_split<true>(L.pk, np, ki, part, tpn) : 0;
    rank = sum_adjacent(rank, tpn);
    if (i < np && part == 0 && rank < An) {
      L.slex[rank] = key_tie(ki);
      L.sc[rank] = L.pc[i];
    }
  }
  __syncthreads();
  // the survivors in slot order, in coalesced stores
  for (int i = tid; i < An; i += NT) {
    const int c = L.sc[i];
    const uint64_t ki = L.key[c];
    const uint32_t li = L.slex[i];
    const size_t sl = (size_t)q * t.Wmax + i;
    t.nsurv_node[sl] = off + c;
    t.nsurv_score[sl] = key_val(ki);
    t.gidx_tok[(size_t)q * An + i] = (int32_t)(li & 0x3FFFFu);
    t.gidx_par[(size_t)q * An + i] = q * A + c / K;
    if (t.gidx_cand) t.gidx_cand[(size_t)q * An + i] = (q * D + delta) * M + L.cc[c];
    t.surv_hist[((size_t)q * (D + 1) + delta + 1) * t.Wmax + i] = off + c;
    t.nsurv_rank[sl] = An - 1 - count_greater<uint32_t>(L.slex, An, li);   // lex keys are distinct
  }
}

__global__ __launch_bounds__(64 * BS_BR) void k_branch_topk(
    int A, int M, int K, int W, int D, int delta, int off, int r, int uvec,
    const uint16_t *__restrict__ W2, const int32_t *__restrict__ C, const float *__restrict__ Cl,
    const float *__restrict__ u, int ldu, TreeBufs t, uint64_t *__restrict__ ckey,
    int32_t *__restrict__ ccand) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ float ell_s[BS_BR][128];
  __shared__ int32_t ctok[128];
  __shared__ float clv[128];
  __shared__ int32_t pnode[BS_BR];
  __shared__ uint32_t prank[BS_BR];
  __shared__ float pscore[BS_BR];
  __shared__ __align__(16) TopwLds tw;
  __shared__ bool last_s;
  // u's three bf16 terms as B-fragment rows: row tq BS_BR + b for branch b,
  // row 3 BS_BR all zeros (the unused branch columns); rows zero-padded to
  // whole chunks of four k steps, so the fragment reads need no masks
  const int nch = (r + 127) >> 7;   // chunks of four k steps of 32
  const int rp = nch * 128 + 8;     // row pitch (+8: rows start 16 bytes apart in the banks)
  uint16_t *us = reinterpret_cast<uint16_t *>(smem);   // [3 BS_BR + 1][rp]
  const int q = blockIdx.x, a0 = blockIdx.y * BS_BR, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, lr = lane & 15, g = lane >> 4;
  const size_t cb = ((size_t)q * D + delta) * M;
  const size_t nb = (size_t)q * t.NT;
  const int Z = A * K;
  const int r8 = r >> 3;
  // this wave's 16 candidates: token, then its W2 row as A fragments (the
  // token load goes first, so waiting for it leaves the others in flight)
  const int jt = wave;
  const bool tile = jt * 16 < M;
  const int jw = min(jt * 16 + lr, M - 1);
  const int tokw = max(C[cb + jw], 0);   // an empty slot never reaches here
  // u of the workgroup's branches, 8 values per thread (BS_BR r / 8 <= 512
  // threads), coalesced
  const int ub = tid / r8, uc = tid - ub * r8;
  const bool uin = ub < BS_BR && a0 + ub < A;
  float x[8];
  {
    const float *up = u + ((size_t)q * A + (uin ? a0 + ub : a0)) * ldu + (uin ? 8 * uc : 0);
    if (uvec) {
      const float4 v0 = reinterpret_cast<const float4 *>(up)[0];
      const float4 v1 = reinterpret_cast<const float4 *>(up)[1];
      x[0] = v0.x; x[1] = v0.y; x[2] = v0.z; x[3] = v0.w;
      x[4] = v1.x; x[5] = v1.y; x[6] = v1.z; x[7] = v1.w;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = up[e];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = uin ? x[e] : 0.f;
  }
  for (int j = tid; j < M; j += blockDim.x) {
    ctok[j] = C[cb + j];
    clv[j] = Cl[cb + j];
  }
  if (tid < BS_BR && a0 + tid < A) {
    pnode[tid] = t.surv_node[(size_t)q * t.Wmax + a0 + tid];
    prank[tid] = (uint32_t)t.surv_rank[(size_t)q * t.Wmax + a0 + tid];
    pscore[tid] = t.surv_score[(size_t)q * t.Wmax + a0 + tid];
  }
  // W2 fragments of every k step (past the row's end: its last piece again,
  // finite bf16 weights that meet zero B rows)
  uint4 wa[16];
  {
    const uint16_t *wr = W2 + (size_t)tokw * r;
#pragma unroll
    for (int ch = 0; ch < 4; ++ch)
      if (ch < nch) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          wa[4 * ch + i] = *reinterpret_cast<const uint4 *>(wr + min(128 * ch + 32 * i + 8 * g, r - 8));
      }
  }
  if (ub < BS_BR) {
    uint4 t3[3];
    split3_bf16(x, t3);   // exact: W2 is bf16, so every MFMA product below is exact in fp32
#pragma unroll
    for (int tq = 0; tq < 3; ++tq)
      *reinterpret_cast<uint4 *>(us + ((size_t)tq * BS_BR + ub) * rp + 8 * uc) = t3[tq];
  }
  {
    const int padc = (rp - r) >> 3;   // zero 8-element pieces past r in each of the 3 BS_BR rows
    for (int i = tid; i < 3 * BS_BR * padc + rp / 8; i += blockDim.x) {
      const int row = i < 3 * BS_BR * padc ? i / padc : 3 * BS_BR;
      const int col = i < 3 * BS_BR * padc ? r + 8 * (i - row * padc) : 8 * (i - 3 * BS_BR * padc);
      *reinterpret_cast<uint4 *>(us + (size_t)row * rp + col) = make_uint4(0u, 0u, 0u, 0u);
    }
  }
  __syncthreads();
  // one 16 x 16 tile (candidates x branch columns, BS_BR of them used) per
  // wave: ell_s[branch][j] = Cl[j] + W2[C[j]] . u_branch, k steps in order,
  // the B fragments of four steps read at a time
  if (tile) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const uint16_t *brow[3];
#pragma unroll
    for (int tq = 0; tq < 3; ++tq)
      brow[tq] = us + (size_t)(lr < BS_BR ? tq * BS_BR + lr : 3 * BS_BR) * rp + 8 * g;
#pragma unroll
    for (int ch = 0; ch < 4; ++ch)
      if (ch < nch) {
        uint4 bq[4][3];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int tq = 0; tq < 3; ++tq)
            bq[i][tq] = *reinterpret_cast<const uint4 *>(brow[tq] + 128 * ch + 32 * i);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int tq = 0; tq < 3; ++tq) acc = cl_mfma(wa[4 * ch + i], bq[i][tq], acc);
      }
    // lane holds D[candidate 4 g + tt][branch column lr]
    if (lr < BS_BR) {
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const int jj = jt * 16 + 4 * g + tt;
        if (jj < M) ell_s[lr][jj] = clv[jj] + acc[tt];
      }
    }
  }
  __syncthreads();
  const int a = a0 + wave;
  if (a < A) {
    const bool h0 = lane < M, h1 = lane + 64 < M;
    const float l0 = h0 ? ell_s[wave][lane] : -INFINITY;
    const float l1 = h1 ? ell_s[wave][lane + 64] : -INFINITY;
    const uint32_t pr = prank[wave];
    const float ps = pscore[wave];
    const float m = wave_max_f32_full(fmaxf(l0, l1));
    const float e = (h0 ? expf(l0 - m) : 0.f) + (h1 ? expf(l1 - m) : 0.f);
    const float lse = m + logf(wave_sum_f32_full(e));
    const float lp0 = h0 ? l0 - lse : -INFINITY, lp1 = h1 ? l1 - lse : -INFINITY;
    const uint32_t tk0 = h0 ? (uint32_t)ctok[lane] : 0u, tk1 = h1 ? (uint32_t)ctok[lane + 64] : 0u;
    int r0, r1;
    wave_topk(lp0, tk0, lp1, tk1, K, r0, r1);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int rk = h ? r1 : r0;
      if (rk < K) {
        const uint32_t tok = h ? tk1 : tk0;
        const float sc = __fadd_rn(ps, h ? lp1 : lp0);
        const uint32_t lex = (pr << 18) | tok;
        const int c = a * K + rk;
        tw.key[c] = make_key(sc, lex);
        tw.cc[c] = (int16_t)(lane + 64 * h);
      }
    }
  }
  if (tid == 0) { tw.tau = 0ull; tw.np = 0; }
  __syncthreads();
  // the workgroup's children are nodes off + [c0, c1): their records in
  // coalesced stores
  const int c0 = a0 * K, c1 = min(A, a0 + BS_BR) * K;
  for (int c = c0 + tid; c < c1; c += blockDim.x) {
    const uint64_t kc = tw.key[c];
    const uint32_t lex = key_tie(kc);
    const size_t id = nb + off + c;
    t.n_tok[id] = (int32_t)(lex & 0x3FFFFu);
    t.n_par[id] = pnode[c / K - a0];
    t.n_dep[id] = delta + 1;
    t.n_score[id] = key_val(kc);
    t.n_lex[id] = lex;
  }
  // Hand-off to the request's last workgroup (several workgroups): wave 0
  // publishes the workgroup's children keys with device-coherent stores,
  // waits until they have completed, raises the workgroup's flag (the depth
  // number plus one; the round start clears the flags) and reads all of the
  // request's flags.  The workgroup whose flag landed last sees them all
  // raised and loads the other workgroups' keys; one that raced it may see
  // them all too and then ranks the same complete keys into the same
  // outputs.  No workgroup waits for another.
  if (gridDim.y > 1) {
    uint32_t *fl = t.selflag + (size_t)q * SEL_FLAGS;
    const uint32_t ep = (uint32_t)delta + 1u;
    if (wave == 0) {
      for (int c = c0 + lane; c < c1; c += 64) {
        __hip_atomic_store(ckey + (size_t)q * Z + c, tw.key[c], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(ccand + (size_t)q * Z + c, (int32_t)tw.cc[c], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
      __builtin_amdgcn_s_waitcnt(0);
      if (lane == 0) {
        __hip_atomic_store(fl + blockIdx.y, ep, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_s_waitcnt(0);
      }
      const bool up = lane >= (int)gridDim.y ||
                      __hip_atomic_load(fl + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == ep;
      const bool all = __all(up);
      if (lane == 0) last_s = all;
    }
    __syncthreads();
    if (!last_s) return;
    for (int c = tid; c < Z; c += blockDim.x)
      if (c < c0 || c >= c1) {
        tw.key[c] = __hip_atomic_load(ckey + (size_t)q * Z + c, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
        tw.cc[c] = (int16_t)__hip_atomic_load(ccand + (size_t)q * Z + c, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
      }
    __syncthreads();
  }
  topw_request<64 * BS_BR>(q, A, K, W, D, delta, off, M, t, tw);
}

hipError_t branch_select_prepare(size_t lds_bytes) {
  return set_lds_limit(reinterpret_cast<const void *>(&k_branch_topk), lds_bytes);
}

size_t branch_select_smem(int r) { return (size_t)(3 * BS_BR + 1) * (((r + 127) >> 7) * 128 + 8) * 2; }

hipError_t launch_branch_select(int b, int A, int M, int K, int W, int D, int delta, int off,
                                int r, const void *W2, const int32_t *C, const float *Cl,
                                const float *u, int ldu, const TreeBufs &t, uint64_t *ckey,
                                int32_t *ccand, hipStream_t st) {
  if (r % 8 || r > 512 || M > 128 || A * K > SEL_MAXZ || W > SEL_MAXW ||
      reinterpret_cast<uintptr_t>(W2) % 16)
    return hipErrorInvalidValue;
  const int uvec = ldu % 4 == 0 && reinterpret_cast<uintptr_t>(u) % 16 == 0;
  hipLaunchKernelGGL(k_branch_topk, dim3(b, (A + BS_BR - 1) / BS_BR), dim3(64 * BS_BR),
                     branch_select_smem(r), st, A, M, K, W, D, delta, off, r, uvec,
                     static_cast<const uint16_t *>(W2), C, Cl, u, ldu, t, ckey, ccand);
  return hipGetLastError();
}

// The whole depth loop under marginal scoring, one workgroup per request:
// with no correction every branch of a depth sees the same M log-probs (the
// log-softmax of the depth's base logits), so the depth's ranks are found
// once; each expanded branch a gets children a * K + k, k < K, with the
// candidate of rank k and score fp32(score(a) + lp); then the Top-W
// survivors and their lexicographic ranks, carried to the next depth in LDS.
// Same rules and tie-breaks as k_select (DARTree page, Metodología 1;
// "Resumen Técnico: DominoTree", Componentes Principales 2).
__global__ __launch_bounds__(SEL_THREADS) void k_select_marginal(int M, int K, int W, int D,
                                                                 const int32_t *__restrict__ C,
                                                                 const float *__restrict__ Cl,
                                                                 TreeBufs t) {
  __shared__ uint64_t ckey[SEL_MAXZ];
  __shared__ uint32_t clex[SEL_MAXZ];
  __shared__ uint32_t slex[SEL_MAXW];
  __shared__ int32_t pnode[2][SEL_MAXW];
  __shared__ uint32_t prank[2][SEL_MAXW];
  __shared__ float pscore[2][SEL_MAXW];
  __shared__ int32_t ktok[128];     // the depth's candidates by rank: token
  __shared__ float klp[128];        //   and log-prob
  __shared__ uint64_t wkeys[128];
  __shared__ int32_t ctab[32 * 128];   // every depth's candidates (D <= 31, M <= 128)
  __shared__ float ltab[32 * 128];     //   and their base logits
  const int q = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t nb = (size_t)q * t.NT;
  for (int i = tid; i < D * M; i += blockDim.x) {
    ctab[i] = C[(size_t)q * D * M + i];
    ltab[i] = Cl[(size_t)q * D * M + i];
  }
  if (tid == 0) { pnode[0][0] = 0; prank[0][0] = 0u; pscore[0][0] = 0.f; }
  __syncthreads();
  int A = 1, off = 1, cur = 0;
  for (int dd = 0; dd < D; ++dd) {
    const int Z = A * K, An = Z < W ? Z : W;
    if (wave == 0) {
      const int32_t *cq = ctab + dd * M;
      const float *lq = ltab + dd * M;
      const bool h0 = lane < M, h1 = lane + 64 < M;
      const float l0 = h0 ? lq[lane] : -INFINITY, l1 = h1 ? lq[lane + 64] : -INFINITY;
      const int32_t t0 = h0 ? cq[lane] : 0, t1 = h1 ? cq[lane + 64] : 0;
      const float m = wave_max_f32(fmaxf(l0, l1));
      const float e = (h0 ? expf(l0 - m) : 0.f) + (h1 ? expf(l1 - m) : 0.f);
      const float lse = m + logf(wave_sum_f32(e));
      const uint64_t k0 = h0 ? make_key(l0 - lse, (uint32_t)t0) : 0ull;
      const uint64_t k1 = h1 ? make_key(l1 - lse, (uint32_t)t1) : 0ull;
      int r0, r1;
      branch_ranks(k0, k1, h0, h1, M, wkeys, lane, r0, r1);
      if (h0 && r0 < K) { ktok[r0] = t0; klp[r0] = key_val(k0); }
      if (h1 && r1 < K) { ktok[r1] = t1; klp[r1] = key_val(k1); }
    }
    __syncthreads();
    for (int c = tid; c < Z; c += blockDim.x) {
      const int a = c / K, k = c - a * K;
      const uint32_t tok = (uint32_t)ktok[k];
      const float sc = __fadd_rn(pscore[cur][a], klp[k]);
      const uint32_t lex = (prank[cur][a] << 18) | tok;
      const size_t id = nb + off + c;
      t.n_tok[id] = (int32_t)tok;
      t.n_par[id] = pnode[cur][a];
      t.n_dep[id] = dd + 1;
      t.n_score[id] = sc;
      t.n_lex[id] = lex;
      ckey[c] = make_key(sc, lex);
      clex[c] = lex;
    }
    __syncthreads();
    // Top-W by rank: keys are distinct (distinct token paths)
    for (int c = tid; c < Z; c += blockDim.x) {
      const uint64_t kc = ckey[c];
      const int rank = count_greater<uint64_t>(ckey, Z, kc);
      if (rank < An) {
        pnode[cur ^ 1][rank] = off + c;
        pscore[cur ^ 1][rank] = key_val(kc);
        slex[rank] = clex[c];
        t.surv_hist[((size_t)q * (D + 1) + dd + 1) * t.Wmax + rank] = off + c;
      }
    }
    __syncthreads();
    for (int i = tid; i < An; i += blockDim.x) {
      const uint32_t li = slex[i];
      const int rank = An - 1 - count_greater<uint32_t>(slex, An, li);   // lex keys are distinct
      prank[cur ^ 1][i] = (uint32_t)rank;
    }
    __syncthreads();
    cur ^= 1;
    off += Z;
    A = An;
  }
}

hipError_t launch_select_marginal(int b, int M, int K, int W, int D, const int32_t *C,
                                  const float *Cl, const TreeBufs &t, hipStream_t st) {
  hipLaunchKernelGGL(k_select_marginal, dim3(b), dim3(SEL_THREADS), 0, st, M, K, W, D, C, Cl, t);
  return hipGetLastError();
}

hipError_t launch_select(int b, int A, int M, int K, int W, int D, int delta, int off,
                         const int32_t *C, const float *ell, long ldq, int lda,
                         const TreeBufs &t, hipStream_t st) {
  hipLaunchKernelGGL(k_select, dim3(b), dim3(SEL_THREADS), 0, st, A, M, K, W, D, delta, off, C,
                     ell, ldq, lda, t);
  return hipGetLastError();
}

}  // namespace dtree
