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
constexpr int K1_TPW = 5;                   // max 16-token tiles per wave
constexpr int K1_MAXCOLS = K1_WAVES * K1_TPW * 16;  // 640 tokens per WG
constexpr int K1_PF = 4;                    // register path: k chunks prefetched per tile
constexpr int K1F_THREADS = 256;            // fp32 path
constexpr int K1F_MAXCOLS = 256;

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// ---- per-row Top-M of the staged logits (one row per half-wave)

// u64 exchange with lane ^ J inside groups of 32 lanes
template <int J>
__device__ __forceinline__ uint64_t xor_u64(uint64_t v) {
  auto x32 = [](uint32_t u) -> uint32_t {
    if constexpr (J == 1) return dpp_u32<0xB1>(u);
    else if constexpr (J == 2) return dpp_u32<0x4E>(u);
    else if constexpr (J == 4) return (uint32_t)__builtin_amdgcn_ds_swizzle((int)u, 0x101F);
    else if constexpr (J == 8) return (uint32_t)__builtin_amdgcn_ds_swizzle((int)u, 0x201F);
    else return (uint32_t)__builtin_amdgcn_ds_swizzle((int)u, 0x401F);
  };
  return ((uint64_t)x32((uint32_t)(v >> 32)) << 32) | x32((uint32_t)v);
}

// Bitonic sort (descending) of 32 NR keys held NR per lane by a half-wave,
// element e = 32 h + lane in register h.  Merge step (K, J): e is compared
// with e ^ J; blocks with (e & K) == 0 are ordered descending.
template <int NR, int K, int J>
__device__ __forceinline__ void bitonic_step(uint64_t (&v)[NR], int hl) {
  if constexpr (J >= 32) {
    constexpr int HJ = J / 32;
#pragma unroll
    for (int h = 0; h < NR; ++h) {
      if ((h & HJ) == 0) {
        const uint64_t a = v[h], b = v[h | HJ];
        const bool desc = ((32 * h + hl) & K) == 0;
        const bool sw = desc ? a < b : a > b;
        v[h] = sw ? b : a;
        v[h | HJ] = sw ? a : b;
      }
    }
  } else {
#pragma unroll
    for (int h = 0; h < NR; ++h) {
      const uint64_t o = xor_u64<J>(v[h]);
      const bool keepmax = ((hl & J) == 0) == (((32 * h + hl) & K) == 0);
      v[h] = keepmax ? (o > v[h] ? o : v[h]) : (o < v[h] ? o : v[h]);
    }
  }
  if constexpr (J > 1) bitonic_step<NR, K, J / 2>(v, hl);
}
template <int NR, int K>
__device__ __forceinline__ void bitonic_sort32(uint64_t (&v)[NR], int hl) {
  bitonic_step<NR, K, K / 2>(v, hl);
  if constexpr (K < 32 * NR) bitonic_sort32<NR, 2 * K>(v, hl);
}

// the lane's NR best keys, descending (insertion network)
template <int KPL, int NR>
__device__ __forceinline__ void lane_best(const uint64_t (&keys)[KPL], uint64_t below,
                                          uint64_t (&v)[NR]) {
#pragma unroll
  for (int t = 0; t < NR; ++t) v[t] = 0;
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    uint64_t x = keys[i] < below ? keys[i] : 0ull;
#pragma unroll
    for (int t = 0; t < NR; ++t) {
      const uint64_t hi = x > v[t] ? x : v[t];
      x = x > v[t] ? v[t] : x;
      v[t] = hi;
    }
  }
}

// Each lane holds KPL keys of the row (0 = empty; keys of a row are
// distinct).  S = the NR best keys of every lane (32 NR >= M of them); tau,
// the M-th largest key of S, has at least M keys of the row at or above it,
// so the row's M best are among the keys >= tau, usually only a few more
// than M.  Those are compacted into cand (the row's own LDS, already read)
// and each one's rank among them is counted.  Returns false, having written
// nothing, when more than min(32 CAP, capmax) keys reach tau.
template <int KPL, int NR, int CAP>
__device__ __forceinline__ bool row_topm_fast(const uint64_t (&keys)[KPL], int hl, bool active,
                                              int M, uint64_t *cand, int capmax, uint64_t *outr) {
  uint64_t v[NR];
  lane_best<KPL, NR>(keys, ~0ull, v);
  bitonic_sort32<NR, 2>(v, hl);
  uint64_t x = v[0];
#pragma unroll
  for (int h = 1; h < NR; ++h)
    if (((M - 1) >> 5) == h) x = v[h];
  const int src = (int)(threadIdx.x & 32) + ((M - 1) & 31);
  const uint64_t tau = ((uint64_t)(uint32_t)__shfl((int)(uint32_t)(x >> 32), src) << 32) |
                       (uint32_t)__shfl((int)(uint32_t)x, src);
  int cnt = 0;
#pragma unroll
  for (int i = 0; i < KPL; ++i) cnt += (keys[i] >= tau && keys[i] != 0ull) ? 1 : 0;
  // inclusive prefix of the counts over the half-wave, and its total
  int incl = cnt, tot = cnt, y;
  y = (int)dpp_u32<0xB1>((uint32_t)tot); if (hl & 1) incl += y; tot += y;
  y = (int)dpp_u32<0x4E>((uint32_t)tot); if (hl & 2) incl += y; tot += y;
  y = __builtin_amdgcn_ds_swizzle(tot, 0x101F); if (hl & 4) incl += y; tot += y;
  y = __builtin_amdgcn_ds_swizzle(tot, 0x201F); if (hl & 8) incl += y; tot += y;
  y = __builtin_amdgcn_ds_swizzle(tot, 0x401F); if (hl & 16) incl += y; tot += y;
  if (tot > 32 * CAP || tot > capmax) return false;
  if (active) {
    int pos = incl - cnt;
#pragma unroll
    for (int i = 0; i < KPL; ++i)
      if (keys[i] >= tau && keys[i] != 0ull) cand[pos++] = keys[i];
  }
  uint64_t mine[CAP];
  int rk[CAP];
#pragma unroll
  for (int w = 0; w < CAP; ++w) {
    mine[w] = hl + 32 * w < tot ? cand[hl + 32 * w] : 0ull;
    rk[w] = 0;
  }
  for (int j = 0; j < tot; j += 8) {
    uint64_t c[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) c[u] = j + u < tot ? cand[j + u] : 0ull;
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int w = 0; w < CAP; ++w) rk[w] += c[u] > mine[w] ? 1 : 0;
  }
  if (active) {
#pragma unroll
    for (int w = 0; w < CAP; ++w)
      if (hl + 32 * w < tot && rk[w] < M) outr[rk[w]] = mine[w];
    for (int m = tot + hl; m < M; m += 32) outr[m] = 0ull;
  }
  return true;
}

// The same result by M rounds of a half-wave maximum over the lanes' sorted
// lists of their best EPI_T keys; the winning lane pops its head, and a lane
// whose list runs dry refills it with its next best keys.
constexpr int EPI_T = 4;
template <int KPL>
__device__ __forceinline__ void row_topm_rounds(const uint64_t (&keys)[KPL], int hl, bool active,
                                                int M, uint64_t *outr) {
  uint64_t loc[EPI_T];
  lane_best<KPL, EPI_T>(keys, ~0ull, loc);
  for (int m = 0; m < M; ++m) {
    const uint64_t top = group_max_u64<32>(loc[0]);
    if (active && hl == 0) outr[m] = top;
    if (loc[0] == top && top != 0) {
#pragma unroll
      for (int t = 0; t + 1 < EPI_T; ++t) loc[t] = loc[t + 1];
      loc[EPI_T - 1] = 0;
      if (loc[0] == 0) lane_best<KPL, EPI_T>(keys, top, loc);
    }
  }
}

// Each half-wave takes one row of the staged logits Ls[row][0..ncols) and
// writes that row's M best keys (value desc, token asc), best first, to
// out[row * ostride + m] (0 = empty).  The row's LDS is scratch afterwards.
template <int MAXC>
__device__ __forceinline__ void wg_topm_epilogue(float *Ls, int lstride, int ncols, int col0,
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
    uint64_t *cand = reinterpret_cast<uint64_t *>(Ls + r * lstride);
    uint64_t *outr = out + (size_t)r * ostride;
    const int capmax = lstride / 2;
    const bool done = M <= 64 && row_topm_fast<KPL, 2, 4>(keys, hl, active, M, cand, capmax, outr);
    if (!done) row_topm_rounds<KPL>(keys, hl, active, M, outr);
  }
}

// LDS of the bf16 kernel: the hidden rows [16][d + 8] bf16, later re-used
// for the logits [16][K1_MAXCOLS] fp32; then (ring path) each wave's ring of
// W_lm chunks; then the slice's bias.
__host__ __device__ inline size_t lmhead_smem_body(int d) {
  const size_t hs = (size_t)16 * (d + 8) * 2;
  const size_t ls = (size_t)16 * K1_MAXCOLS * 4;
  return ((hs > ls ? hs : ls) + 15) & ~(size_t)15;
}
constexpr int K1_CHUNK = 4096;   // one ring buffer: 16 rows x 128 k bf16

__device__ __forceinline__ void k1_wait_vm(int n) {   // vmcnt <= n (n <= 63)
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    case 4: __builtin_amdgcn_s_waitcnt(0x0F74); break;
    case 8: __builtin_amdgcn_s_waitcnt(0x0F78); break;
    case 12: __builtin_amdgcn_s_waitcnt(0x0F7C); break;
    default: __builtin_amdgcn_s_waitcnt(0x0F70); break;
  }
}

// Tiles [0, ntV) are 16-token slabs of W_lm; when W1 is given, tiles
// [ntV, ntV + ntU) are 16-row slabs of W1[:, :d] and produce the
// path-independent projection uH = W1[:, :d] Hq for the same rows (the same
// B operand), written straight to uH.
//
// RING > 0: every wave streams its tiles' 128-wide k chunks (16 rows x 256
// bytes) into a ring of RING LDS buffers with global_load_lds, each load
// instruction covering four whole 256-byte row segments (full cache lines;
// loads that hand each lane a piece of a different row reach much less of
// the HBM bandwidth).  Buffer slot (row q, 16-byte segment x) holds segment
// x ^ q, so the MFMA A-fragment reads (16 rows, same segment) hit distinct
// banks.  The ring runs across tile boundaries.
// RING == 0 (hidden rows too large for a ring beside them): every lane loads
// its own row's A fragments straight into registers, K1_PF chunks ahead.
template <int RING>
__global__ __launch_bounds__(K1_WAVES * 64) void k1_lmhead_bf16(
    const float *__restrict__ H, int rows, int d, const uint16_t *__restrict__ W, int V,
    const float *__restrict__ bias, int M, uint64_t *__restrict__ part,
    const uint16_t *__restrict__ W1, int ldw1, int r, float *__restrict__ uH,
    const int32_t *__restrict__ root, int b, int Dp1, TreeBufs tb) {
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
  // source row rr of tile lt (clamped into the matrix)
  auto tile_row = [&](int lt, int rr) -> const uint16_t * {
    const int tt = t0 + lt;
    return tt < ntV ? W + (size_t)min(tt * 16 + rr, V - 1) * d
                    : W1 + (size_t)min((tt - ntV) * 16 + rr, r - 1) * ldw1;
  };
  // tiles of this wave: lt = wave + K1_WAVES * i, i < ntw
  const int ntw = nt > wave ? min(K1_TPW, (nt - wave + K1_WAVES - 1) / K1_WAVES) : 0;

  // ---- ring state (RING > 0): chunk z = i * nch + c goes to buffer z % RING
  uint4 *ring = reinterpret_cast<uint4 *>(smem + lmhead_smem_body(d)) + wave * RING * (K1_CHUNK / 16);
  const int Z = ntw * nch;
  int zi = 0, ii = 0, ic = 0;   // next chunk to issue, its tile and k chunk
  const uint4 *rq[4];           // this lane's source rows 4 k + lane / 16 of tile ii (swizzled slot)
  auto ring_rows = [&](int i) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int q = 4 * k + g;
      rq[k] = reinterpret_cast<const uint4 *>(tile_row(wave + K1_WAVES * i, q)) + (lr ^ q);
    }
  };
  auto ring_issue = [&]() {
    if (zi < Z) {
      uint4 *dst = ring + (zi % (RING > 0 ? RING : 1)) * (K1_CHUNK / 16);
#pragma unroll
      for (int k = 0; k < 4; ++k)
        __builtin_amdgcn_global_load_lds(rq[k] + ic * 16,
                                         (__attribute__((address_space(3))) void *)(dst + k * 64),
                                         16, 0, 0);
      ++zi;
      if (++ic == nch) {
        ic = 0;
        if (++ii < ntw) ring_rows(ii);
      }
    }
  };
  // ---- register state (RING == 0): lane group g takes k = 32 g + 8 j + (0..7)
  // of MFMA j in each 128-wide chunk
  const uint16_t *hp = Hs + lr * HS + g * (RING > 0 ? 8 : 32);
  const uint4 *ptr = nullptr;
  uint4 regs[RING > 0 ? 1 : K1_PF][4];
  auto reg_start = [&](int i) {
    ptr = reinterpret_cast<const uint4 *>(tile_row(wave + K1_WAVES * i, lr) + g * 32);
#pragma unroll
    for (int pp = 0; pp < (RING > 0 ? 1 : K1_PF); ++pp)
      if (pp < nch) {
#pragma unroll
        for (int j = 0; j < 4; ++j) regs[pp][j] = ptr[pp * 16 + j];
      }
  };
  // the first loads are in flight while the hidden rows are staged
  if (ntw > 0) {
    if constexpr (RING > 0) {
      ring_rows(0);
#pragma unroll
      for (int p0 = 0; p0 < RING; ++p0) ring_issue();
    } else {
      reg_start(0);
    }
  }

  // bias of this slice's vocabulary columns, staged once
  float *bs = reinterpret_cast<float *>(smem + lmhead_smem_body(d) + (size_t)K1_WAVES * RING * K1_CHUNK);
  {
    const int c0 = t0 * 16, nc = min(min(t1, ntV) * 16, V) - c0;
    for (int c = threadIdx.x; c < nc; c += K1_WAVES * 64) bs[c] = bias ? bias[c0 + c] : 0.f;
  }
  // Hq = bf16_rne(H) for the 16 rows of this block (zeros past `rows`)
  {
    // all of a thread's loads in flight at once (16 per batch)
    const int q4 = d >> 2;   // float4 per row
    constexpr int NB = 16, NTH = K1_WAVES * 64;
    for (int i0 = threadIdx.x; i0 < 16 * q4; i0 += NB * NTH) {
      float4 v[NB];
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const int i = i0 + u * NTH, rr = i / q4, k = (i - rr * q4) * 4;
        v[u] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (i < 16 * q4 && rr < nrow) v[u] = *reinterpret_cast<const float4 *>(H + (size_t)(row0 + rr) * d + k);
      }
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const int i = i0 + u * NTH, rr = i / q4, k = (i - rr * q4) * 4;
        const uint32_t lo = (uint32_t)f32_to_bf16_rne(v[u].x) | ((uint32_t)f32_to_bf16_rne(v[u].y) << 16);
        const uint32_t hi = (uint32_t)f32_to_bf16_rne(v[u].z) | ((uint32_t)f32_to_bf16_rne(v[u].w) << 16);
        if (i < 16 * q4) *reinterpret_cast<uint2 *>(Hs + rr * HS + k) = make_uint2(lo, hi);
      }
    }
  }
  __syncthreads();

  float vals[K1_TPW][4];
#pragma unroll
  for (int i = 0; i < K1_TPW; ++i) {
    if (i < ntw) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (RING > 0) {
        for (int c = 0; c < nch; ++c) {
          const int z = i * nch + c;
          k1_wait_vm(z + RING - 1 < Z ? 4 * (RING - 1) : 0);
          const uint4 *buf = ring + (z % RING) * (K1_CHUNK / 16) + lr * 16;
          const uint4 *h4 = reinterpret_cast<const uint4 *>(hp + c * 128);
          uint4 av[4], hv[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            av[j] = buf[(4 * j + g) ^ lr];
            hv[j] = h4[4 * j];
          }
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av[j]), as_bf16x8(hv[j]), acc,
                                                         0, 0, 0);
          // this buffer's reads have landed before the next chunk overwrites it
          __builtin_amdgcn_s_waitcnt(0xC07F);
          ring_issue();
        }
      } else {
        if (i > 0) reg_start(i);
        for (int c0 = 0; c0 < nch; c0 += K1_PF) {
#pragma unroll
          for (int pp = 0; pp < K1_PF; ++pp) {
            const int c = c0 + pp;
            if (c < nch) {
              const uint4 *h4 = reinterpret_cast<const uint4 *>(hp + c * 128);
#pragma unroll
              for (int j = 0; j < 4; ++j)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(regs[pp][j]),
                                                             as_bf16x8(h4[j]), acc, 0, 0, 0);
              if (c + K1_PF < nch) {
#pragma unroll
                for (int j = 0; j < 4; ++j) regs[pp][j] = ptr[(c + K1_PF) * 16 + j];
              }
            }
          }
        }
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) vals[i][t] = acc[t];
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
// best first, M keys, 0 = empty) into the row's M best.
//
// Every list holds M keys at least as large as its M-th, and the M largest
// list heads are M distinct keys, so the row's M best are all >= tau, the
// larger of the largest M-th key of a list and the M-th largest head.
// Usually only a few more than M keys qualify: they are gathered in LDS and each one's rank
// among them is counted.  With more than K1B_FAST of them, the lists are
// merged by a bitonic tournament instead: for two descending lists A and B,
// max(A[k], B[Mp-1-k]) holds the Mp best keys of A and B as a bitonic
// sequence (Mp = next_pow2(M), lists padded with empty keys), which a
// half-cleaner cascade sorts back into descending order.  Lists are paired
// level by level in LDS (at level l the live lists sit at slots that are
// multiples of 2^l); with more lists than fit, batches of G-1 lists are
// reduced together with the running result in slot 0.
constexpr int K1B_THREADS = 512;
constexpr int K1B_CAP = 16384;   // tournament: keys in LDS (128 KiB)
constexpr int K1B_FAST = 2048;   // gathered candidates

__global__ __launch_bounds__(K1B_THREADS) void k1b_topm_merge(
    const uint64_t *__restrict__ part, int P, int M, int32_t *__restrict__ C,
    float *__restrict__ Cl) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ uint64_t red[K1B_THREADS / 64];
  __shared__ int ncand;
  uint64_t *L = reinterpret_cast<uint64_t *>(smem);
  const int row = blockIdx.x, tid = threadIdx.x, nt = blockDim.x;
  const uint64_t *pk = part + (size_t)row * P * M;
  {
    uint64_t t = 0;
    for (int l = tid; l < P; l += nt) {
      const uint64_t v = pk[(size_t)l * M + M - 1];
      t = v > t ? v : t;
    }
    // the lists' heads are distinct keys too: the M-th largest head is
    // another lower bound of the row's M-th key (0 if fewer than M heads)
    uint64_t *heads = L;
    for (int l = tid; l < P; l += nt) heads[l] = pk[(size_t)l * M];
    if (tid == 0) ncand = 0;
    __syncthreads();
    if (M <= P) {
      for (int l = tid; l < P; l += nt) {
        const uint64_t h = heads[l];
        int rk = 0;
        for (int j = 0; j < P; ++j) rk += heads[j] > h ? 1 : 0;
        if (rk == M - 1 && h > t) t = h;
      }
    }
    t = group_max_u64<64>(t);
    if ((tid & 63) == 0) red[tid >> 6] = t;
    __syncthreads();
    uint64_t tau = 0;
    for (int w = 0; w < nt / 64; ++w) tau = red[w] > tau ? red[w] : tau;
    const int tot = P * M;
    for (int i0 = tid; i0 < tot; i0 += 8 * nt) {
      uint64_t v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = i0 + u * nt < tot ? pk[i0 + u * nt] : 0ull;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (v[u] >= tau && v[u] != 0ull) {
          const int at = atomicAdd(&ncand, 1);
          if (at < K1B_FAST) L[at] = v[u];
        }
    }
    __syncthreads();
    const int n = ncand;
    if (n <= K1B_FAST) {
      for (int i = tid; i < n; i += nt) {
        const uint64_t k = L[i];
        int rk = 0;
        for (int j = 0; j < n; ++j) rk += L[j] > k ? 1 : 0;
        if (rk < M) {
          C[(size_t)row * M + rk] = (int32_t)key_tie(k);
          Cl[(size_t)row * M + rk] = key_val(k);
        }
      }
      for (int m = n + tid; m < M; m += nt) {
        C[(size_t)row * M + m] = -1;
        Cl[(size_t)row * M + m] = key_val(0ull);
      }
      return;
    }
    __syncthreads();
  }
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


size_t lmhead_smem(int d, int wtype, int ring) {
  if (wtype != WT_BF16) return 0;
  return lmhead_smem_body(d) + (size_t)K1_WAVES * ring * K1_CHUNK + (size_t)K1_MAXCOLS * 4;
}

int lmhead_ring(int d, int wtype, size_t lds_max) {
  if (wtype != WT_BF16) return 0;
  for (int ring = 2; ring > 0; --ring)
    if (lmhead_smem(d, wtype, ring) <= lds_max) return ring;
  return 0;
}

template <int RING>
static const void *k1_fn() { return reinterpret_cast<const void *>(&k1_lmhead_bf16<RING>); }

hipError_t lmhead_prepare(int wtype, int ring, size_t smem) {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k1b_topm_merge),
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)(K1B_CAP * sizeof(uint64_t)));
  if (e != hipSuccess || wtype != WT_BF16) return e;
  const void *fn = ring == 2 ? k1_fn<2>() : ring == 1 ? k1_fn<1>() : k1_fn<0>();
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
}

hipError_t launch_lmhead(const LMHeadArgs &a, hipStream_t st) {
  dim3 grid((a.rows + 15) / 16, a.P);
  if (a.wtype == WT_BF16) {
    const size_t sm = lmhead_smem(a.d, a.wtype, a.ring);
#define K1_LAUNCH(RING)                                                                         \
  hipLaunchKernelGGL((k1_lmhead_bf16<RING>), grid, dim3(K1_WAVES * 64), sm, st, a.H, a.rows, a.d, \
                     static_cast<const uint16_t *>(a.W), a.V, a.bias, a.M, a.part,               \
                     static_cast<const uint16_t *>(a.W1), a.ldw1, a.r, a.uH, a.root, a.b, a.Dp1, a.t)
    if (a.ring == 2) K1_LAUNCH(2);
    else if (a.ring == 1) K1_LAUNCH(1);
    else K1_LAUNCH(0);
#undef K1_LAUNCH
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
