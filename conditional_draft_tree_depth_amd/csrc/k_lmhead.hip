// K1 / K1b: shared base logits and the per-depth Top-M candidate table.
//
// Base logits L_base = Hq . W_lm^T (+ bias) come from the backbone's shared
// hidden states through the frozen target LM head ("Resumen Técnico:
// Domino", Methodology 1); they are path-independent, so one pass serves
// every branch ("Resumen Técnico: DominoTree", Main components 1).  Only the
// Top-M of each row is kept ("Resumen Técnico: DominoTree", Main
// components 2; DARTree page, Methodology 1, candidate selection): the
// vocabulary-wide logits are never written to memory.
//
// bf16 path: every wave multiplies 16-token tiles of W_lm (MFMA A operand,
// streamed from HBM with one chunk of prefetch) by the 16 rounded hidden
// rows held in LDS (B operand) with v_mfma_f32_16x16x32_bf16, fp32
// accumulation.  Inside one MFMA the k index pairs lane (i + 16g) element t
// of A with lane (j + 16g) element t of B, so any assignment of k to (g, t)
// that both operands share is valid; here lane group g reads 32 contiguous
// k per 128-wide chunk (64-byte row segments of W_lm).  A workgroup owns a
// contiguous slice of tiles; after its GEMM it re-uses the LDS of the hidden
// rows to stage its logits and extracts each row's best M keys.
#include "common.hpp"
#include "kernels.hpp"

namespace dtree {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int K1_WAVES = 8;                 // waves per workgroup (bf16 path)
constexpr int K1_TPW = 8;                   // max 16-token tiles per wave
constexpr int K1_MAXCOLS = K1_WAVES * K1_TPW * 16;  // 1024 tokens per WG
constexpr int K1F_THREADS = 256;            // fp32 path
constexpr int K1F_MAXCOLS = 256;

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// Each half-wave takes one row of the staged logits Ls[row][0..ncols) and
// writes that row's M best keys (value desc, token asc), best first, to
// out[row * ostride + m].  Keys within a row are distinct (distinct tokens),
// so the m-th best is the largest key strictly below the (m-1)-th.
template <int MAXC>
__device__ void wg_topm_epilogue(const float *Ls, int lstride, int ncols, int col0,
                                 int nrow, int M, uint64_t *out, size_t ostride) {
  constexpr int KPL = MAXC / 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6, hl = lane & 31;
  for (int rb = wave * 2; rb < nrow; rb += 2 * nw) {
    const int r = rb + (lane >> 5);
    const bool active = r < nrow;
    uint64_t keys[KPL];
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
      const int c = hl + 32 * i;
      uint64_t k = 0;
      if (active && c < ncols) k = make_key(Ls[r * lstride + c], (uint32_t)(col0 + c));
      keys[i] = k;
      best = k > best ? k : best;
    }
    for (int m = 0; m < M; ++m) {
      const uint64_t top = group_max_u64<32>(best);
      if (active && hl == 0) out[(size_t)r * ostride + m] = top;
      if (best == top && top != 0) {
        uint64_t nb = 0;
#pragma unroll
        for (int i = 0; i < KPL; ++i) {
          const uint64_t k = keys[i];
          nb = (k < top && k > nb) ? k : nb;
        }
        best = nb;
      }
    }
  }
}

__global__ __launch_bounds__(K1_WAVES * 64) void k1_lmhead_bf16(
    const float *__restrict__ H, int rows, int d, const uint16_t *__restrict__ W, int V,
    const float *__restrict__ bias, int M, uint64_t *__restrict__ part) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int P = gridDim.y, y = blockIdx.y;
  const int row0 = blockIdx.x * 16;
  const int nrow = min(16, rows - row0);
  const int HS = d + 8;  // bf16 elements per LDS row (16-byte skew)
  uint16_t *Hs = reinterpret_cast<uint16_t *>(smem);

  // Hq = bf16_rne(H) for the 16 rows of this block (zeros past `rows`)
  for (int i = threadIdx.x; i < 16 * d; i += blockDim.x) {
    const int rr = i / d, k = i - rr * d;
    const float v = rr < nrow ? H[(size_t)(row0 + rr) * d + k] : 0.f;
    Hs[rr * HS + k] = f32_to_bf16_rne(v);
  }
  __syncthreads();

  const int ntiles = (V + 15) >> 4;
  const int t0 = (int)((long long)ntiles * y / P);
  const int t1 = (int)((long long)ntiles * (y + 1) / P);
  const int nt = t1 - t0;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lr = lane & 15, g = lane >> 4;
  const uint16_t *hp = Hs + lr * HS + g * 32;

  float vals[K1_TPW][4];
#pragma unroll
  for (int i = 0; i < K1_TPW; i += 2) {
    const int ltA = wave + K1_WAVES * i;
    const int ltB = ltA + K1_WAVES;
    if (ltA < nt) {
      const int ltB2 = ltB < nt ? ltB : ltA;
      const int vA = min((t0 + ltA) * 16 + lr, V - 1);
      const int vB = min((t0 + ltB2) * 16 + lr, V - 1);
      const uint4 *pa = reinterpret_cast<const uint4 *>(W + (size_t)vA * d + g * 32);
      const uint4 *pb = reinterpret_cast<const uint4 *>(W + (size_t)vB * d + g * 32);
      f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accB = {0.f, 0.f, 0.f, 0.f};
      uint4 ca[4], cb[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) { ca[j] = pa[j]; cb[j] = pb[j]; }
      for (int kc = 0; kc < d; kc += 128) {
        uint4 na[4], nb[4];
        if (kc + 128 < d) {
#pragma unroll
          for (int j = 0; j < 4; ++j) { na[j] = pa[(kc + 128) / 8 + j]; nb[j] = pb[(kc + 128) / 8 + j]; }
        }
        const uint4 *h4 = reinterpret_cast<const uint4 *>(hp + kc);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bf16x8 hb = as_bf16x8(h4[j]);
          accA = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ca[j]), hb, accA, 0, 0, 0);
          accB = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(cb[j]), hb, accB, 0, 0, 0);
        }
        if (kc + 128 < d) {
#pragma unroll
          for (int j = 0; j < 4; ++j) { ca[j] = na[j]; cb[j] = nb[j]; }
        }
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) { vals[i][t] = accA[t]; vals[i + 1][t] = accB[t]; }
    }
  }
  __syncthreads();  // every wave is done with Hs: re-use it for the logits

  float *Ls = reinterpret_cast<float *>(smem);
  constexpr int LSTR = K1_MAXCOLS;
  if (lr < nrow) {
#pragma unroll
    for (int i = 0; i < K1_TPW; ++i) {
      const int lt = wave + K1_WAVES * i;
      if (lt < nt) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int c = lt * 16 + 4 * g + t;
          const int v = t0 * 16 + c;
          if (v < V) Ls[lr * LSTR + c] = vals[i][t] + (bias ? bias[v] : 0.f);
        }
      }
    }
  }
  __syncthreads();
  const int ncols = min(nt * 16, V - t0 * 16);
  wg_topm_epilogue<K1_MAXCOLS>(Ls, LSTR, ncols, t0 * 16, nrow, M,
                               part + ((size_t)row0 * P + y) * M, (size_t)P * M);
}

// fp32 weights: plain VALU dot products (small workloads only).
__global__ __launch_bounds__(K1F_THREADS) void k1_lmhead_f32(
    const float *__restrict__ H, int rows, int d, const float *__restrict__ W, int V,
    const float *__restrict__ bias, int M, uint64_t *__restrict__ part) {
  __shared__ float Ls[16 * K1F_MAXCOLS];
  const int P = gridDim.y, y = blockIdx.y;
  const int row0 = blockIdx.x * 16;
  const int nrow = min(16, rows - row0);
  const int ntiles = (V + 15) >> 4;
  const int t0 = (int)((long long)ntiles * y / P);
  const int t1 = (int)((long long)ntiles * (y + 1) / P);
  const int col0 = t0 * 16;
  const int ncols = min((t1 - t0) * 16, V - col0);
  for (int c = threadIdx.x; c < ncols; c += blockDim.x) {
    const float *wr = W + (size_t)(col0 + c) * d;
    for (int rr = 0; rr < nrow; ++rr) {
      const float *hr = H + (size_t)(row0 + rr) * d;
      float acc = 0.f;
      for (int k = 0; k < d; ++k) acc += hr[k] * wr[k];
      Ls[rr * K1F_MAXCOLS + c] = acc + (bias ? bias[col0 + c] : 0.f);
    }
  }
  __syncthreads();
  wg_topm_epilogue<K1F_MAXCOLS>(Ls, K1F_MAXCOLS, ncols, col0, nrow, M,
                                part + ((size_t)row0 * P + y) * M, (size_t)P * M);
}

// K1b: one workgroup per row merges that row's P partial lists.  A lower
// bound on the row's M-th best key is the largest M-th key of any partial
// list; only keys at or above it can be in the result.
constexpr int K1B_THREADS = 256;
constexpr int K1B_CAP = 2048;

__global__ __launch_bounds__(K1B_THREADS) void k1b_topm_merge(
    const uint64_t *__restrict__ part, int P, int M, int32_t *__restrict__ C,
    float *__restrict__ Cl) {
  __shared__ uint64_t cand[K1B_CAP];
  __shared__ int32_t dummy[K1B_CAP];
  __shared__ uint64_t red[K1B_THREADS / 64];
  __shared__ int cnt;
  const int row = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const uint64_t *pk = part + (size_t)row * P * M;
  const int total = P * M;

  uint64_t t = 0;
  for (int p = tid; p < P; p += K1B_THREADS) {
    const uint64_t k = pk[(size_t)p * M + M - 1];
    t = k > t ? k : t;
  }
  t = group_max_u64<64>(t);
  if (lane == 0) red[wave] = t;
  if (tid == 0) cnt = 0;
  __syncthreads();
  t = red[0];
  for (int w = 1; w < K1B_THREADS / 64; ++w) t = red[w] > t ? red[w] : t;
  if (t == 0) t = 1;  // never admit empty slots
  for (int i = tid; i < total; i += K1B_THREADS) {
    const uint64_t k = pk[i];
    if (k >= t) {
      const int pos = atomicAdd(&cnt, 1);
      if (pos < K1B_CAP) cand[pos] = k;
    }
  }
  __syncthreads();
  const int n = cnt;
  if (n <= K1B_CAP) {
    const int np2 = next_pow2(n > M ? n : M);
    for (int i = n + tid; i < np2; i += K1B_THREADS) cand[i] = 0;
    __syncthreads();
    block_bitonic_desc(cand, dummy, np2);
    for (int j = tid; j < M; j += K1B_THREADS) {
      const uint64_t k = cand[j];
      C[(size_t)row * M + j] = k ? (int32_t)key_tie(k) : -1;
      Cl[(size_t)row * M + j] = key_val(k);
    }
  } else {
    // Many keys above the bound: take the M best one at a time.
    uint64_t prev = ~0ull;
    for (int j = 0; j < M; ++j) {
      uint64_t b = 0;
      for (int i = tid; i < total; i += K1B_THREADS) {
        const uint64_t k = pk[i];
        b = (k < prev && k > b) ? k : b;
      }
      b = group_max_u64<64>(b);
      __syncthreads();
      if (lane == 0) red[wave] = b;
      __syncthreads();
      b = red[0];
      for (int w = 1; w < K1B_THREADS / 64; ++w) b = red[w] > b ? red[w] : b;
      if (tid == 0) {
        C[(size_t)row * M + j] = b ? (int32_t)key_tie(b) : -1;
        Cl[(size_t)row * M + j] = key_val(b);
      }
      prev = b;
    }
  }
}

// ----------------------------------------------------------------- host side
int lmhead_partitions(int V, int wtype) {
  const int ntiles = (V + 15) / 16;
  const int per_wg = wtype == WT_BF16 ? K1_MAXCOLS / 16 : K1F_MAXCOLS / 16;
  int P = (ntiles + per_wg - 1) / per_wg;   // enough slices to fit the LDS
  if (P < 256) P = ntiles < 256 ? ntiles : 256;   // at least one per CU
  return P;
}

size_t lmhead_smem(int d, int wtype) {
  if (wtype != WT_BF16) return 0;
  const size_t hs = (size_t)16 * (d + 8) * 2;
  const size_t ls = (size_t)16 * K1_MAXCOLS * 4;
  return hs > ls ? hs : ls;
}

hipError_t lmhead_prepare(int wtype, size_t smem) {
  if (wtype != WT_BF16) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void *>(&k1_lmhead_bf16),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
}

hipError_t launch_lmhead(const LMHeadArgs &a, hipStream_t st) {
  dim3 grid((a.rows + 15) / 16, a.P);
  if (a.wtype == WT_BF16) {
    hipLaunchKernelGGL(k1_lmhead_bf16, grid, dim3(K1_WAVES * 64), lmhead_smem(a.d, a.wtype), st,
                       a.H, a.rows, a.d, static_cast<const uint16_t *>(a.W), a.V, a.bias, a.M,
                       a.part);
  } else {
    hipLaunchKernelGGL(k1_lmhead_f32, grid, dim3(K1F_THREADS), 0, st, a.H, a.rows, a.d,
                       static_cast<const float *>(a.W), a.V, a.bias, a.M, a.part);
  }
  return hipGetLastError();
}

hipError_t launch_topm_merge(const uint64_t *part, int P, int M, int rows, int32_t *C,
                             float *Cl, hipStream_t st) {
  hipLaunchKernelGGL(k1b_topm_merge, dim3(rows), dim3(K1B_THREADS), 0, st, part, P, M, C, Cl);
  return hipGetLastError();
}

}  // namespace dtree
