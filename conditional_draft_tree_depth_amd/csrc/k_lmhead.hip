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
#ifndef K1_TPI
#define K1_TPI 1      // tiles in flight per wave
#endif
#ifndef K1_PF
#define K1_PF 4       // k chunks prefetched per tile
#endif
#ifndef K1_CL
#define K1_CL 0       // lane-contiguous k layout
#endif
constexpr int K1_GROUP = 16;                // workgroups per first-level merge
constexpr int K1F_THREADS = 256;            // fp32 path
constexpr int K1F_MAXCOLS = 256;

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// Each half-wave takes one row of the staged logits Ls[row][0..ncols) and
// writes that row's M best keys (value desc, token asc), best first, to
// out[row * ostride + m].  Keys within a row are distinct (distinct tokens).
// Every lane keeps its own best EPI_T keys in a short sorted list; each of
// the M rounds takes the half-wave maximum of the list heads and the winning
// lane pops its head.  A lane whose list runs dry refills it with its next
// best keys (those below the last one it gave).
constexpr int EPI_T = 4;
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
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
      const int c = hl + 32 * i;
      uint64_t k = 0;
      if (active && c < ncols) k = make_key(Ls[r * lstride + c], (uint32_t)(col0 + c));
      keys[i] = k;
    }
    // best EPI_T keys below `below`, descending (insertion network)
    uint64_t loc[EPI_T];
    auto refill = [&](uint64_t below) {
#pragma unroll
      for (int t = 0; t < EPI_T; ++t) loc[t] = 0;
#pragma unroll
      for (int i = 0; i < KPL; ++i) {
        uint64_t x = keys[i] < below ? keys[i] : 0ull;
#pragma unroll
        for (int t = 0; t < EPI_T; ++t) {
          const uint64_t hi = x > loc[t] ? x : loc[t];
          x = x > loc[t] ? loc[t] : x;
          loc[t] = hi;
        }
      }
    };
    refill(~0ull);
    for (int m = 0; m < M; ++m) {
      const uint64_t top = group_max_u64<32>(loc[0]);
      if (active && hl == 0)   // read by another workgroup: device-coherent store
        __hip_atomic_store(out + (size_t)r * ostride + m, top, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      if (loc[0] == top && top != 0) {
#pragma unroll
        for (int t = 0; t + 1 < EPI_T; ++t) loc[t] = loc[t + 1];
        loc[EPI_T - 1] = 0;
        if (loc[0] == 0) refill(top);
      }
    }
  }
}

// Top-M merge of at most 16 sorted lists per row.  For each of nr rows,
// lists 0 .. nl-1 (descending, M keys, 0 = empty) sit at src + row * rstride
// + list * lstride (written by other workgroups: read with device-coherent
// loads) and are staged in LDS.  Sixteen lanes take a row, one list each,
// with the list's next four keys in registers; each of the M rounds takes
// the 16-lane maximum (DPP only) and the winning lane pops its head and
// fetches the key four places further on from LDS.  emit(row, m, key) gets
// the row's m-th best key.  At most 4 * waves rows per call; all threads of
// the block call it.
constexpr int K1_MLISTS = 16;
template <class Emit>
__device__ void lds_merge_lists(uint64_t *L, const uint64_t *src, size_t rstride, int lstride,
                                int nl, int nr, int M, Emit emit) {
  const int tid = threadIdx.x;
  constexpr int NT = K1_WAVES * 64;
  const int tot = nr * K1_MLISTS * M;
  for (int i0 = tid; i0 < tot; i0 += 8 * NT) {   // 8 loads in flight per thread
    uint64_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * NT, rl = i / M, k = i - rl * M, row = rl / K1_MLISTS;
      const int l = rl - row * K1_MLISTS;
      v[u] = 0ull;
      if (i < tot && l < nl)
        v[u] = __hip_atomic_load(src + row * rstride + (size_t)l * lstride + k, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (i0 + u * NT < tot) L[i0 + u * NT] = v[u];
  }
  __syncthreads();
  const int lane = tid & 63, wave = tid >> 6;
  const int row = wave * 4 + (lane >> 4), li = lane & 15;
  const bool act = row < nr;
  const uint64_t *lst = L + ((size_t)(act ? row : 0) * K1_MLISTS + li) * M;
  uint64_t buf[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) buf[t] = (act && t < M) ? lst[t] : 0ull;
  int cur = 0;   // index of buf[0] in the list
  for (int m = 0; m < M; ++m) {
    const uint64_t top = group_max_u64<16>(buf[0]);
    if (act && li == 0) emit(row, m, top);
    if (buf[0] == top && top != 0) {
      buf[0] = buf[1];
      buf[1] = buf[2];
      buf[2] = buf[3];
      ++cur;
      buf[3] = cur + 3 < M ? lst[cur + 3] : 0ull;
    }
  }
  __syncthreads();
}

// LDS of the bf16 kernel: the hidden rows [16][d + 8] bf16, later re-used
// for the logits [16][K1_MAXCOLS] fp32; then the slice's bias.
__host__ __device__ inline size_t lmhead_smem_body(int d) {
  const size_t hs = (size_t)16 * (d + 8) * 2;
  const size_t ls = (size_t)16 * K1_MAXCOLS * 4;
  return ((hs > ls ? hs : ls) + 15) & ~(size_t)15;
}

// Tiles [0, ntV) are 16-token slabs of W_lm; when W1 is given, tiles
// [ntV, ntV + ntU) are 16-row slabs of W1[:, :d] and produce the
// path-independent projection uH = W1[:, :d] Hq for the same rows (the same
// B operand), written straight to uH.  A wave keeps TPI tiles in flight and
// PF 128-wide k chunks of each prefetched in registers.
template <int TPI, int PF, int CL>
__global__ __launch_bounds__(K1_WAVES * 64) void k1_lmhead_bf16(
    const float *__restrict__ H, int rows, int d, const uint16_t *__restrict__ W, int V,
    const float *__restrict__ bias, int M, uint64_t *__restrict__ part,
    const uint16_t *__restrict__ W1, int ldw1, int r, float *__restrict__ uH,
    uint32_t *__restrict__ cnt, uint64_t *__restrict__ part2, int32_t *__restrict__ C,
    float *__restrict__ Cl, const int32_t *__restrict__ root, int b, int Dp1, TreeBufs tb) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int P = gridDim.y, y = blockIdx.y;
  if (root && blockIdx.x == 0)
    for (int q = y; q < b; q += P) init_round_request(q, root, tb, Dp1, threadIdx.x, K1_WAVES * 64);
  const int row0 = blockIdx.x * 16;
  const int nrow = min(16, rows - row0);
  const int HS = d + 8;  // bf16 elements per LDS row (16-byte skew)
  uint16_t *Hs = reinterpret_cast<uint16_t *>(smem);

  const int ntV = (V + 15) >> 4;
  const int ntU = W1 ? (r + 15) >> 4 : 0;
  const int T = ntV + ntU;
  const int t0 = (int)((long long)T * y / P);
  const int t1 = (int)((long long)T * (y + 1) / P);
  const int nt = t1 - t0;
  const int nch = d >> 7;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lr = lane & 15, g = lane >> 4;
  // CL: lane group g takes k = 32 j + 8 g + (0..7) of MFMA j (a row's four
  // lanes read 64 contiguous bytes per load); else k = 32 g + 8 j + (0..7)
  const uint16_t *hp = Hs + lr * HS + g * (CL ? 8 : 32);
  const uint4 *ptr[TPI];
  uint4 ring[PF][TPI][4];
  // pointers of the tiles lt0 + K1_WAVES u and the first PF chunks of them
  auto start_tiles = [&](int lt0) {
#pragma unroll
    for (int u = 0; u < TPI; ++u) {
      const int lt = lt0 + K1_WAVES * u < nt ? lt0 + K1_WAVES * u : lt0;
      const int tt = t0 + lt;
      const uint16_t *rp = tt < ntV ? W + (size_t)min(tt * 16 + lr, V - 1) * d
                                    : W1 + (size_t)min((tt - ntV) * 16 + lr, r - 1) * ldw1;
      ptr[u] = reinterpret_cast<const uint4 *>(rp + g * (CL ? 8 : 32));
    }
#pragma unroll
    for (int pp = 0; pp < PF; ++pp)
      if (pp < nch) {
#pragma unroll
        for (int u = 0; u < TPI; ++u)
#pragma unroll
          for (int j = 0; j < 4; ++j) ring[pp][u][j] = ptr[u][pp * 16 + j * (CL ? 4 : 1)];
      }
  };
  // the first tiles' loads are in flight while the hidden rows are staged
  if (wave < nt) start_tiles(wave);

  // bias of this slice's vocabulary columns, staged once (behind the larger
  // of the hidden-row and logit buffers)
  float *bs = reinterpret_cast<float *>(smem + lmhead_smem_body(d));
  {
    const int c0 = t0 * 16, nc = min(min(t1, ntV) * 16, V) - c0;
    for (int c = threadIdx.x; c < nc; c += K1_WAVES * 64) bs[c] = bias ? bias[c0 + c] : 0.f;
  }
  // Hq = bf16_rne(H) for the 16 rows of this block (zeros past `rows`)
  {
    const int q4 = d >> 2;   // float4 per row
#pragma unroll 4
    for (int i = threadIdx.x; i < 16 * q4; i += K1_WAVES * 64) {
      const int rr = i / q4, k = (i - rr * q4) * 4;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (rr < nrow) v = *reinterpret_cast<const float4 *>(H + (size_t)(row0 + rr) * d + k);
      const uint32_t lo = (uint32_t)f32_to_bf16_rne(v.x) | ((uint32_t)f32_to_bf16_rne(v.y) << 16);
      const uint32_t hi = (uint32_t)f32_to_bf16_rne(v.z) | ((uint32_t)f32_to_bf16_rne(v.w) << 16);
      *reinterpret_cast<uint2 *>(Hs + rr * HS + k) = make_uint2(lo, hi);
    }
  }
  __syncthreads();

  float vals[K1_TPW][4];
#pragma unroll
  for (int i = 0; i < K1_TPW; i += TPI) {
    const int lt0 = wave + K1_WAVES * i;
    if (lt0 < nt) {
      if (i > 0) start_tiles(lt0);
      f32x4 acc[TPI];
#pragma unroll
      for (int u = 0; u < TPI; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int c0 = 0; c0 < nch; c0 += PF) {
#pragma unroll
        for (int pp = 0; pp < PF; ++pp) {
          const int c = c0 + pp;
          if (c < nch) {
            const uint4 *h4 = reinterpret_cast<const uint4 *>(hp + c * 128);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const bf16x8 hb = as_bf16x8(h4[j * (CL ? 4 : 1)]);
#pragma unroll
              for (int u = 0; u < TPI; ++u)
                acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ring[pp][u][j]), hb,
                                                                 acc[u], 0, 0, 0);
            }
            if (c + PF < nch) {
#pragma unroll
              for (int u = 0; u < TPI; ++u)
#pragma unroll
                for (int j = 0; j < 4; ++j) ring[pp][u][j] = ptr[u][(c + PF) * 16 + j * (CL ? 4 : 1)];
            }
          }
        }
      }
#pragma unroll
      for (int u = 0; u < TPI; ++u)
#pragma unroll
        for (int t = 0; t < 4; ++t) vals[i + u][t] = acc[u][t];
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
        const int tt = t0 + lt;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          if (tt < ntV) {
            const int c = lt * 16 + 4 * g + t;
            const int v = t0 * 16 + c;
            if (v < V) Ls[lr * LSTR + c] = vals[i][t] + bs[c];
          } else {
            const int uc = (tt - ntV) * 16 + 4 * g + t;
            if (uc < r) uH[(size_t)(row0 + lr) * r + uc] = vals[i][t];
          }
        }
      }
    }
  }
  __syncthreads();
  const int vend = min(min(t1, ntV) * 16, V);
  const int ncols = vend > t0 * 16 ? vend - t0 * 16 : 0;
  wg_topm_epilogue<K1_MAXCOLS>(Ls, LSTR, ncols, t0 * 16, nrow, M,
                               part + ((size_t)row0 * P + y) * M, (size_t)P * M);
  if (!cnt) return;

  // Fused merge.  Workgroups y come in groups of K1_GROUP; the last one of a
  // group to finish (counted by an ever-growing counter: every round adds the
  // group size) merges the group's lists into part2, and the last group
  // merger of this row block merges the groups' lists into C / Cl.  Lists
  // travel through device-coherent stores and loads; each thread's stores
  // have completed before its workgroup counts itself in.
  const int NG = (P + K1_GROUP - 1) / K1_GROUP, grp = y / K1_GROUP;
  const int gsz = min(K1_GROUP, P - grp * K1_GROUP);
  uint32_t *cb = cnt + (size_t)blockIdx.x * (NG + 1);
  int *flag = reinterpret_cast<int *>(bs);
  uint64_t *L = reinterpret_cast<uint64_t *>(smem);
  // rows per merge call: the staged lists fit in LDS, 4 rows per wave
  const int rpb = min(4 * K1_WAVES, max(1, (int)(lmhead_smem_body(d) / 8) / (K1_MLISTS * M)));
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(cb + grp, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    flag[0] = (old + 1) % (uint32_t)gsz == 0;
  }
  __syncthreads();
  if (!flag[0]) return;
  for (int rb = 0; rb < nrow; rb += rpb) {
    const int nr = min(rpb, nrow - rb);
    lds_merge_lists(L, part + ((size_t)(row0 + rb) * P + grp * K1_GROUP) * M, (size_t)P * M, M,
                    gsz, nr, M, [&](int rr, int m, uint64_t key) {
                      __hip_atomic_store(part2 + ((size_t)(row0 + rb + rr) * NG + grp) * M + m, key,
                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    });
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(cb + NG, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    flag[0] = (old + 1) % (uint32_t)NG == 0;
  }
  __syncthreads();
  if (!flag[0]) return;
  for (int rb = 0; rb < nrow; rb += rpb) {
    const int nr = min(rpb, nrow - rb);
    lds_merge_lists(L, part2 + (size_t)(row0 + rb) * NG * M, (size_t)NG * M, M, NG, nr, M,
                    [&](int rr, int m, uint64_t key) {
                      const size_t o = (size_t)(row0 + rb + rr) * M + m;
                      C[o] = key ? (int32_t)key_tie(key) : -1;
                      Cl[o] = key_val(key);
                    });
  }
}

// fp32 weights: plain VALU dot products (small workloads only).
__global__ __launch_bounds__(K1F_THREADS) void k1_lmhead_f32(
    const float *__restrict__ H, int rows, int d, const float *__restrict__ W, int V,
    const float *__restrict__ bias, int M, uint64_t *__restrict__ part,
    const int32_t *__restrict__ root, int b, int Dp1, TreeBufs tb) {
  __shared__ float Ls[16 * K1F_MAXCOLS];
  const int P = gridDim.y, y = blockIdx.y;
  if (root && blockIdx.x == 0)
    for (int q = y; q < b; q += P) init_round_request(q, root, tb, Dp1, threadIdx.x, K1F_THREADS);
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

// K1b: one workgroup per row merges that row's P partial lists (each sorted
// best-first, padded with empty keys to Mp = next_pow2(M)) by a bitonic
// tournament: for two descending lists A and B, max(A[k], B[Mp-1-k]) holds
// the Mp best keys of A and B as a bitonic sequence, which a half-cleaner
// cascade sorts back into descending order.  Lists are paired level by level
// in LDS (no data movement: at level l the live lists sit at slots that are
// multiples of 2^l); with more lists than fit, batches of G-1 lists are
// reduced together with the running result in slot 0.
constexpr int K1B_THREADS = 512;
constexpr int K1B_CAP = 16384;   // keys in LDS (128 KiB)

__global__ __launch_bounds__(K1B_THREADS) void k1b_topm_merge(
    const uint64_t *__restrict__ part, int P, int M, int32_t *__restrict__ C,
    float *__restrict__ Cl) {
  extern __shared__ __align__(16) uint8_t smem[];
  uint64_t *L = reinterpret_cast<uint64_t *>(smem);
  const int row = blockIdx.x, tid = threadIdx.x, nt = blockDim.x;
  const uint64_t *pk = part + (size_t)row * P * M;
  const int Mp = next_pow2(M);
  const int lm = __builtin_ctz((unsigned)Mp);         // log2(Mp)
  const int G = K1B_CAP >> lm;                         // lists per batch (power of two, >= 2)
  for (int i = tid; i < Mp; i += nt) L[i] = 0ull;     // running result, slot 0
  for (int p0 = 0; p0 < P; p0 += G - 1) {
    const int nl = min(G - 1, P - p0);                 // fresh lists in this batch
    const int nslots = next_pow2(nl + 1);
    for (int i = Mp + tid; i < (nslots << lm); i += nt) {
      const int sl = (i >> lm) - 1, k = i & (Mp - 1);
      L[i] = (sl < nl && k < M) ? pk[(size_t)(p0 + sl) * M + k] : 0ull;
    }
    __syncthreads();
    for (int ls = 0; (1 << ls) < nslots; ++ls) {
      const int npairs = nslots >> (ls + 1);
      const int pshift = ls + 1 + lm;                  // log2 of a pair's span in keys
      // max against the reversed partner: bitonic, holds the best Mp
      for (int i = tid; i < (npairs << lm); i += nt) {
        const int pr = i >> lm, k = i & (Mp - 1);
        uint64_t *A = L + ((size_t)pr << pshift);
        const uint64_t *Bv = A + ((size_t)1 << (ls + lm));
        const uint64_t a = A[k], b = Bv[Mp - 1 - k];
        A[k] = a > b ? a : b;
      }
      __syncthreads();
      for (int lj = lm - 1; lj >= 0; --lj) {
        const int j = 1 << lj;
        for (int i = tid; i < (npairs << (lm - 1)); i += nt) {
          const int pr = i >> (lm - 1), h = i & ((Mp >> 1) - 1);
          uint64_t *A = L + ((size_t)pr << pshift);
          const int lo = ((h >> lj) << (lj + 1)) | (h & (j - 1)), hi = lo + j;
          const uint64_t a = A[lo], b = A[hi];
          if (a < b) { A[lo] = b; A[hi] = a; }
        }
        __syncthreads();
      }
    }
  }
  for (int j = tid; j < M; j += nt) {
    const uint64_t k = L[j];
    C[(size_t)row * M + j] = k ? (int32_t)key_tie(k) : -1;
    Cl[(size_t)row * M + j] = key_val(k);
  }
}

// ----------------------------------------------------------------- host side
int lmhead_partitions(int V, int wtype, int extra_tiles) {
  const int ntiles = (V + 15) / 16 + (wtype == WT_BF16 ? extra_tiles : 0);
  const int per_wg = wtype == WT_BF16 ? K1_MAXCOLS / 16 : K1F_MAXCOLS / 16;
  int P = (ntiles + per_wg - 1) / per_wg;   // enough slices to fit the LDS
  if (P < 256) P = ntiles < 256 ? ntiles : 256;   // at least one per CU
  return P;
}

bool lmhead_fused_merge(int P, int M, int d, int wtype) {
  if (wtype != WT_BF16 || (P + K1_GROUP - 1) / K1_GROUP > K1_MLISTS) return false;
  return (size_t)K1_MLISTS * M * 8 <= lmhead_smem_body(d);
}
int lmhead_groups(int P) { return (P + K1_GROUP - 1) / K1_GROUP; }

size_t lmhead_smem(int d, int wtype) {
  if (wtype != WT_BF16) return 0;
  return lmhead_smem_body(d) + (size_t)K1_MAXCOLS * 4;
}

hipError_t lmhead_prepare(int wtype, size_t smem) {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k1b_topm_merge),
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)(K1B_CAP * sizeof(uint64_t)));
  if (e != hipSuccess || wtype != WT_BF16) return e;
  return hipFuncSetAttribute(reinterpret_cast<const void *>(&k1_lmhead_bf16<K1_TPI, K1_PF, K1_CL>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
}

hipError_t launch_lmhead(const LMHeadArgs &a, hipStream_t st) {
  dim3 grid((a.rows + 15) / 16, a.P);
  if (a.wtype == WT_BF16) {
    hipLaunchKernelGGL((k1_lmhead_bf16<K1_TPI, K1_PF, K1_CL>), grid, dim3(K1_WAVES * 64),
                       lmhead_smem(a.d, a.wtype), st, a.H, a.rows, a.d,
                       static_cast<const uint16_t *>(a.W), a.V, a.bias, a.M, a.part,
                       static_cast<const uint16_t *>(a.W1), a.ldw1, a.r, a.uH, a.cnt, a.part2,
                       a.C, a.Cl, a.root, a.b, a.Dp1, a.t);
  } else {
    hipLaunchKernelGGL(k1_lmhead_f32, grid, dim3(K1F_THREADS), 0, st, a.H, a.rows, a.d,
                       static_cast<const float *>(a.W), a.V, a.bias, a.M, a.part, a.root, a.b,
                       a.Dp1, a.t);
  }
  return hipGetLastError();
}

hipError_t launch_topm_merge(const uint64_t *part, int P, int M, int rows, int32_t *C,
                             float *Cl, hipStream_t st) {
  const size_t sm = (size_t)K1B_CAP * sizeof(uint64_t);
  hipLaunchKernelGGL(k1b_topm_merge, dim3(rows), dim3(K1B_THREADS), sm, st, part, P, M, C, Cl);
  return hipGetLastError();
}

}  // namespace dtree
