// K1 / K1b: shared base logits and the per-depth Top-M candidate table.
//
// Base logits L_base = Hq . W_lm^T (+ bias) come from the backbone's shared
// hidden states through the frozen target LM head ("Resumen Técnico:
// Domino", Metodología 1); they are path-independent, so one pass serves
// every branch ("Resumen Técnico: DominoTree", Componentes Principales 1).  Only the
// Top-M of each row is kept ("Resumen Técnico: DominoTree", Main
// components 2; DARTree page, Metodología 1, candidate selection): the
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
#include <hip/hip_ext.h>
#include <type_traits>

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

// ---- per-row candidate lists of the staged logits (one row per half-wave)
//
// Every workgroup leaves, for each of its rows, a list at part + row *
// rstride: K1_LCAP key slots, then tau, head and count.  The list holds
// `count` keys (any order) that include the slice's M best, every slice key
// >= tau is in it, at least min(M, slice size) slice keys are >= tau (so the
// row's M-th best key is >= tau), and head is the slice's best key.

// u32 exchange with lane ^ J inside groups of 32 lanes
template <int J>
__device__ __forceinline__ uint32_t xor_u32(uint32_t u) {
  if constexpr (J == 1) return dpp_u32<0xB1>(u);
  else if constexpr (J == 2) return dpp_u32<0x4E>(u);
  else if constexpr (J == 4) return (uint32_t)__builtin_amdgcn_ds_swizzle((int)u, 0x101F);
  else if constexpr (J == 8) return (uint32_t)__builtin_amdgcn_ds_swizzle((int)u, 0x201F);
  else return (uint32_t)__builtin_amdgcn_ds_swizzle((int)u, 0x401F);
}

// Bitonic sort (descending) of 32 NR values held NR per lane by a half-wave,
// element e = NR lane + h in register h (NR a power of two): the low index
// bits stay inside a lane, so fewer steps need a lane exchange.  Merge step
// (K, J): e is compared with e ^ J; blocks with (e & K) == 0 are ordered
// descending.
template <int NR, int K, int J>
__device__ __forceinline__ void bitonic_step(uint32_t (&v)[NR], int hl) {
  if constexpr (J < NR) {
#pragma unroll
    for (int h = 0; h < NR; ++h) {
      if ((h & J) == 0) {
        const uint32_t a = v[h], b = v[h | J];
        const bool desc = ((NR * hl + h) & K) == 0;
        v[h] = desc ? max(a, b) : min(a, b);
        v[h | J] = desc ? min(a, b) : max(a, b);
      }
    }
  } else {
    constexpr int LJ = J / NR;
#pragma unroll
    for (int h = 0; h < NR; ++h) {
      const uint32_t o = xor_u32<LJ>(v[h]);
      const bool keepmax = ((hl & LJ) == 0) == (((NR * hl + h) & K) == 0);
      v[h] = keepmax ? max(o, v[h]) : min(o, v[h]);
    }
  }
  if constexpr (J > 1) bitonic_step<NR, K, J / 2>(v, hl);
}
template <int NR, int K>
__device__ __forceinline__ void bitonic_sort32(uint32_t (&v)[NR], int hl) {
  bitonic_step<NR, K, K / 2>(v, hl);
  if constexpr (K < 32 * NR) bitonic_sort32<NR, 2 * K>(v, hl);
}
// element e of the sorted values (all lanes of the half-wave get it)
template <int NR>
__device__ __forceinline__ uint32_t bitonic_elem(const uint32_t (&v)[NR], int e) {
  uint32_t x = v[0];
#pragma unroll
  for (int h = 1; h < NR; ++h)
    if ((e & (NR - 1)) == h) x = v[h];
  return (uint32_t)__shfl((int)x, (int)(threadIdx.x & 32) + e / NR);
}

// the lane's EPI_T best keys below `below`, descending (insertion network)
constexpr int EPI_T = 4;
template <int KPL>
__device__ __forceinline__ void lane_best(const uint64_t (&keys)[KPL], uint64_t below,
                                          uint64_t (&v)[EPI_T]) {
#pragma unroll
  for (int t = 0; t < EPI_T; ++t) v[t] = 0;
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    uint64_t x = keys[i] < below ? keys[i] : 0ull;
#pragma unroll
    for (int t = 0; t < EPI_T; ++t) {
      const uint64_t hi = x > v[t] ? x : v[t];
      x = x > v[t] ? v[t] : x;
      v[t] = hi;
    }
  }
}

// Each lane holds KPL ordered values of the row (hv, 0 = empty) for columns
// hl + 32 i.  Fast path (M <= 64): S = every lane's two best values (four
// when M > 32); tau, the M-th largest of S, has at least M keys of the row at
// or above it, so
// the row's M best are among the keys with value >= tau, usually only a few
// more than M.  Those are written unsorted.  With more than K1_LCAP of them
// (ties) or M > 64, the row's exact M best are written instead, by M rounds
// of a half-wave maximum over the lanes' sorted short lists (a lane whose
// list runs dry refills it with its next best keys).
template <int MAXC>
__device__ __forceinline__ void wg_topm_epilogue(const float *Ls, int lstride, int ncols,
                                                 int col0, int nrow, int M, uint64_t *out,
                                                 size_t rstride) {
  constexpr int KPL = MAXC / 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6, hl = lane & 31;
  for (int rb = wave * 2; rb < nrow; rb += 2 * nw) {
    const int r = rb + (lane >> 5);
    const bool active = r < nrow;
    // every read in bounds (row r < 16, column clamped), the empty ones
    // zeroed afterwards: no branch around each read, all in flight at once
    uint32_t hv[KPL];
    const float *lrow = Ls + (active ? r : 0) * lstride;
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
      const int c = hl + 32 * i;
      const float x = lrow[c < ncols ? c : 0];
      hv[i] = (active && c < ncols) ? f32_ord(x) : 0u;
    }
    auto key_of = [&](int i) -> uint64_t {
      return ((uint64_t)hv[i] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)(col0 + hl + 32 * i));
    };
    uint64_t *outr = out + (size_t)r * rstride;
    bool done = false;
    if (M <= 64) {
      // S: every lane's NR best values (NR = 4 when M > 32, so that tau, the
      // M-th largest of 32 NR values, stays high enough for the keys that
      // reach it to fit a list)
      auto tau_of = [&](auto nr) -> uint32_t {
        constexpr int NR = decltype(nr)::value;
        uint32_t sv[NR];
#pragma unroll
        for (int t = 0; t < NR; ++t) sv[t] = 0u;
#pragma unroll
        for (int i = 0; i < KPL; ++i) {
          uint32_t x = hv[i];
#pragma unroll
          for (int t = 0; t < NR; ++t) {
            const uint32_t hi = max(x, sv[t]);
            x = min(x, sv[t]);
            sv[t] = hi;
          }
        }
        bitonic_sort32<NR, 2>(sv, hl);
        return bitonic_elem<NR>(sv, M - 1);
      };
      const uint32_t tau = M <= 32 ? tau_of(std::integral_constant<int, 2>())
                                   : tau_of(std::integral_constant<int, 4>());
      int cnt = 0;
#pragma unroll
      for (int i = 0; i < KPL; ++i) cnt += (hv[i] >= tau && hv[i] != 0u) ? 1 : 0;
      // inclusive prefix of the counts over the half-wave, and its total
      int incl = cnt, tot = cnt, y;
      y = (int)dpp_u32<0xB1>((uint32_t)tot); if (hl & 1) incl += y; tot += y;
      y = (int)dpp_u32<0x4E>((uint32_t)tot); if (hl & 2) incl += y; tot += y;
      y = __builtin_amdgcn_ds_swizzle(tot, 0x101F); if (hl & 4) incl += y; tot += y;
      y = __builtin_amdgcn_ds_swizzle(tot, 0x201F); if (hl & 8) incl += y; tot += y;
      y = __builtin_amdgcn_ds_swizzle(tot, 0x401F); if (hl & 16) incl += y; tot += y;
      if (tot <= K1_LCAP) {
        if (active) {
          int pos = incl - cnt;
          uint64_t best = 0;
#pragma unroll
          for (int i = 0; i < KPL; ++i)
            if (hv[i] >= tau && hv[i] != 0u) {
              const uint64_t k = key_of(i);
              outr[pos++] = k;
              best = k > best ? k : best;
            }
          const uint64_t head = group_max_u64<32>(best);
          if (hl == 0) {
            outr[K1_LCAP] = (uint64_t)tau << 32;
            outr[K1_LCAP + 1] = head;
            outr[K1_LCAP + 2] = (uint64_t)tot;
          }
        }
        done = true;
      }
    }
    if (!done) {
      uint64_t keys[KPL];
#pragma unroll
      for (int i = 0; i < KPL; ++i) keys[i] = hv[i] ? key_of(i) : 0ull;
      uint64_t loc[EPI_T];
      lane_best<KPL>(keys, ~0ull, loc);
      uint64_t first = 0, last = 0;
      int nz = 0;
      for (int m = 0; m < M; ++m) {
        const uint64_t top = group_max_u64<32>(loc[0]);
        if (active && hl == 0) outr[m] = top;
        if (m == 0) first = top;
        last = top;
        nz += top != 0 ? 1 : 0;
        if (loc[0] == top && top != 0) {
#pragma unroll
          for (int t = 0; t + 1 < EPI_T; ++t) loc[t] = loc[t + 1];
          loc[EPI_T - 1] = 0;
          if (loc[0] == 0) lane_best<KPL>(keys, top, loc);
        }
      }
      if (active && hl == 0) {
        outr[K1_LCAP] = nz == M ? last : 0ull;
        outr[K1_LCAP + 1] = first;
        outr[K1_LCAP + 2] = (uint64_t)nz;
      }
    }
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
// banks.  The ring runs across tile boundaries.  The compiler makes a wave
// wait for its copies in flight before it reads the ring; the eight waves of
// a CU cover each other's waits (copies issued out of the compiler's sight,
// with a wait for one buffer only, measured the same time).
// RING == 0 (hidden rows too large for a ring beside them): every lane loads
// its own row's A fragments straight into registers, K1_PF chunks ahead.
template <int RING>
__global__ __launch_bounds__(K1_WAVES * 64) void k1_lmhead_bf16(
    const float *__restrict__ H, int rows, int d, const uint16_t *__restrict__ W, int V,
    const float *__restrict__ bias, int M, uint64_t *__restrict__ part,
    const uint16_t *__restrict__ W1, int ldw1, int r, float *__restrict__ uH,
    const int32_t *__restrict__ root, int b, int Dp1, TreeBufs tb) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int P = gridDim.y, RB = gridDim.x;
  int y = blockIdx.y, bx = blockIdx.x;
  // Several 16-row blocks: workgroups are handed to the 8 XCDs in turn, so
  // task (row block, slice) is renumbered to give each XCD a contiguous run
  // of tasks in which all row blocks of one slice come one after another;
  // they run side by side and read the slice's W_lm tiles through that
  // XCD's L2 instead of each from HBM.
  if (RB > 1 && (RB * P) % 8 == 0) {
    const int id = bx + RB * y;
    const int task = (id & 7) * (RB * P / 8) + (id >> 3);
    y = task / RB;
    bx = task - y * RB;
  }
  const int row0 = bx * 16;
  const int nrow = min(16, rows - row0);
  const int cpr = d >> 3;   // 16-byte chunks per hidden row (a multiple of 16)
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
  // this lane's hidden row in LDS (B operand), 16-byte chunks, swizzled
  const uint4 *hrow = reinterpret_cast<const uint4 *>(smem) + lr * cpr;
  const int hsw = lr & 7;
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
  // The hidden rows and the bias are staged before the first W_lm copies
  // are issued: behind those copies (every CU's, in the same memory queues)
  // their loads took several microseconds.
  // bias of this slice's vocabulary columns (at most K1_MAXCOLS = 640 of
  // them, two per thread)
  const int bc0 = t0 * 16, bnc = min(min(t1, ntV) * 16, V) - bc0;
  const int bcA = threadIdx.x, bcB = threadIdx.x + K1_WAVES * 64;
  static_assert(K1_MAXCOLS <= 2 * K1_WAVES * 64, "two bias values per thread");
  // (a slice of W1 tiles only has bnc <= 0 and reads nothing)
  const bool hasb = bias && bnc > 0;
  const float bvA = hasb ? bias[bc0 + min(bcA, bnc - 1)] : 0.f;
  const float bvB = hasb ? bias[bc0 + min(bcB, bnc - 1)] : 0.f;
  // the 16 hidden rows of this block, rounded to bf16 (nearest-even) while
  // they are staged in LDS (rows past the last are zeros); 16-byte chunk j
  // of row q is stored at chunk j ^ (q & 7) of the row, so the B-fragment
  // reads (16 rows, same chunk) hit distinct banks
  {
    constexpr int HB = 5;   // chunks per thread in flight at a time
    for (int ci0 = threadIdx.x; ci0 < 16 * cpr; ci0 += HB * K1_WAVES * 64) {
      float4 v[HB][2];
#pragma unroll
      for (int h = 0; h < HB; ++h) {
        const int ci = ci0 + h * K1_WAVES * 64, rr = ci / cpr, j = ci - rr * cpr;
        v[h][0] = v[h][1] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (ci < 16 * cpr && row0 + rr < rows) {
          const float *src = H + (size_t)(row0 + rr) * d + 8 * (j ^ (rr & 7));
          v[h][0] = *reinterpret_cast<const float4 *>(src);
          v[h][1] = *reinterpret_cast<const float4 *>(src + 4);
        }
      }
#pragma unroll
      for (int h = 0; h < HB; ++h) {
        const int ci = ci0 + h * K1_WAVES * 64;
        if (ci < 16 * cpr) {
          auto pk = [](float lo, float hi) {
            return (uint32_t)f32_to_bf16_rne(lo) | ((uint32_t)f32_to_bf16_rne(hi) << 16);
          };
          *reinterpret_cast<uint4 *>(Hs + (size_t)ci * 8) =
              make_uint4(pk(v[h][0].x, v[h][0].y), pk(v[h][0].z, v[h][0].w),
                         pk(v[h][1].x, v[h][1].y), pk(v[h][1].z, v[h][1].w));
        }
      }
    }
  }
  float *bs = reinterpret_cast<float *>(smem + lmhead_smem_body(d) + (size_t)K1_WAVES * RING * K1_CHUNK);
  if (bcA < bnc) bs[bcA] = bvA;
  if (bcB < bnc) bs[bcB] = bvB;
  // the first W_lm loads are in flight while the tree buffers are started
  if (ntw > 0) {
    if constexpr (RING > 0) {
      ring_rows(0);
#pragma unroll
      for (int p0 = 0; p0 < RING; ++p0) ring_issue();
    } else {
      reg_start(0);
    }
  }
  // round start: the first workgroup of each slice starts the tree buffers
  // of its requests (read only by the kernels after this one)
  if (bx == 0 && root)
    for (int q = y; q < b; q += P) init_round_request(q, root, tb, Dp1, threadIdx.x, K1_WAVES * 64);
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
          uint4 av[4], hv[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            av[j] = buf[(4 * j + g) ^ lr];
            hv[j] = hrow[c * 16 + ((4 * j + g) ^ hsw)];
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
#pragma unroll
              for (int j = 0; j < 4; ++j)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    as_bf16x8(regs[pp][j]), as_bf16x8(hrow[c * 16 + ((4 * g + j) ^ hsw)]), acc, 0,
                    0, 0);
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
  // vocabulary tiles: the bias reads (in bounds: c < K1_MAXCOLS) all issued
  // before the logit stores, which are predicated, not branched around
  {
    float bv[K1_TPW][4];
#pragma unroll
    for (int i = 0; i < K1_TPW; ++i)
#pragma unroll
      for (int t = 0; t < 4; ++t) bv[i][t] = bs[(wave + K1_WAVES * i) * 16 + 4 * g + t];
#pragma unroll
    for (int i = 0; i < K1_TPW; ++i) {
      const int lt = wave + K1_WAVES * i, tt = t0 + lt;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int c = lt * 16 + 4 * g + t;
        if (lr < nrow && lt < nt && tt < ntV && t0 * 16 + c < V) Ls[lr * LSTR + c] = vals[i][t] + bv[i][t];
      }
    }
  }
  // tiles of W1 rows: uH
  if (lr < nrow && t1 > ntV) {
#pragma unroll
    for (int i = 0; i < K1_TPW; ++i) {
      const int lt = wave + K1_WAVES * i, tt = t0 + lt;
      if (lt < nt && tt >= ntV) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int uc = (tt - ntV) * 16 + 4 * g + t;
          if (uc < r) uH[(size_t)(row0 + lr) * r + uc] = vals[i][t];
        }
      }
    }
  }
  __syncthreads();
  const int vend = min(min(t1, ntV) * 16, V);
  const int ncols = vend > t0 * 16 ? vend - t0 * 16 : 0;
  wg_topm_epilogue<K1_MAXCOLS>(Ls, LSTR, ncols, t0 * 16, nrow, M,
                               part + ((size_t)row0 * P + y) * K1_LSTRIDE, (size_t)P * K1_LSTRIDE);
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
                                part + ((size_t)row0 * P + y) * K1_LSTRIDE, (size_t)P * K1_LSTRIDE);
}

// K1b: one workgroup per row selects the row's M best keys from its P lists.
//
// Each list guarantees that the row's M-th best key is >= its tau; M heads
// are M distinct keys, so the M-th largest value among 64 (M > 32: 256) of
// the heads (the best of the lists l = slot mod 64 or 256) is a bound as
// well; the larger sort costs more than it saves for small M.  tau, the largest of these bounds, can only be reached in lists
// whose head reaches it (at most M of them), and usually by only a few more
// than M keys: those are gathered in LDS and each one's rank among them is
// counted.  If more than K1B_FAST keys pass (heavy ties), the exact M-th
// best key is found first by bisection over counts (the largest x with at
// least M listed keys >= x, between tau and the best head; every key the
// row's M best could be is listed), leaving exactly M keys to rank.
constexpr int K1B_THREADS = 512;
constexpr int K1B_FAST = 2048;   // gathered keys
constexpr int K1B_UNROLL = 8;   // live lists per wave in flight
static_assert(K1_LCAP <= 128, "a list's keys are two per lane");

size_t topm_merge_smem(int P) {
  return (size_t)K1B_FAST * 8 + (size_t)P * 8 + (size_t)P * 4 * 2;
}

// The merge of one row by a workgroup of K1B_THREADS threads (dynamic LDS
// laid out as topm_merge_smem(P) says).  Once the keys to be ranked are
// gathered, every thread calls gathered(keys, n) (n of them, in LDS, in no
// particular order); then out(rank, key, i) is called once for every rank <
// M, i being the key's position among the gathered ones (key 0 and i = -1
// for the ranks past the listed keys).
template <class Gathered, class Out>
__device__ void topm_merge_row(const uint64_t *__restrict__ part, int P, int M, int row,
                               uint8_t *smem, Gathered gathered, Out out) {
  __shared__ uint64_t red[K1B_THREADS / 64];
  __shared__ int redi[K1B_THREADS / 64];
  __shared__ int ncand, nlive;
  uint64_t *cand = reinterpret_cast<uint64_t *>(smem);                 // [K1B_FAST]
  uint64_t *heads = cand + K1B_FAST;                                   // [P]
  int *cnt = reinterpret_cast<int *>(heads + P);                       // [P]
  int *live = cnt + P;                                                 // [P]
  const int tid = threadIdx.x, nt = K1B_THREADS;
  const int lane = tid & 63, wave = tid >> 6, nwv = nt >> 6;
  const uint64_t *base = part + (size_t)row * P * K1_LSTRIDE;
  auto block_max = [&](uint64_t v) -> uint64_t {
    v = group_max_u64<64>(v);
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    uint64_t m = 0;
    for (int w = 0; w < nwv; ++w) m = red[w] > m ? red[w] : m;
    return m;
  };
  auto block_sum = [&](int c) -> int {
    c += (int)xchg_u32<1>((uint32_t)c);
    c += (int)xchg_u32<2>((uint32_t)c);
    c += (int)xchg_u32<4>((uint32_t)c);
    c += (int)xchg_u32<8>((uint32_t)c);
    c += (int)xchg_u32<16>((uint32_t)c);
    c += (int)xchg_u32<32>((uint32_t)c);
    __syncthreads();
    if (lane == 0) redi[wave] = c;
    __syncthreads();
    int tot = 0;
    for (int w = 0; w < nwv; ++w) tot += redi[w];
    return tot;
  };

  uint64_t t = 0;
  for (int l = tid; l < P; l += nt) {
    const uint64_t *m = base + (size_t)l * K1_LSTRIDE + K1_LCAP;
    const uint64_t tl = m[0];
    heads[l] = m[1];
    cnt[l] = (int)min(m[2], (uint64_t)K1_LCAP);
    t = tl > t ? tl : t;
  }
  if (tid == 0) { ncand = 0; nlive = 0; }
  __syncthreads();
  if (wave == 0 && M <= P) {
    // 32 NR distinct heads (the best of the lists l = slot mod 32 NR), sorted
    // by value: at least M keys reach the M-th largest value among them
    const int hl = lane & 31;
    auto bound = [&](auto nr) -> uint64_t {
      constexpr int NR = decltype(nr)::value;
      uint32_t v[NR];
#pragma unroll
      for (int h = 0; h < NR; ++h) {
        uint64_t b = 0;
        for (int l = NR * hl + h; l < P; l += 32 * NR) b = heads[l] > b ? heads[l] : b;
        v[h] = (uint32_t)(b >> 32);
      }
      bitonic_sort32<NR, 2>(v, hl);
      return (uint64_t)bitonic_elem<NR>(v, M - 1) << 32;
    };
    const uint64_t th = M <= 32 ? bound(std::integral_constant<int, 2>())
                                : bound(std::integral_constant<int, 8>());
    t = th > t ? th : t;
  }
  const uint64_t tau = block_max(t);
  uint64_t hmax = 0;
  for (int l = tid; l < P; l += nt) {
    const uint64_t h = heads[l];
    if (h >= tau && h != 0ull && cnt[l] > 0) live[atomicAdd(&nlive, 1)] = l;
    hmax = h > hmax ? h : hmax;
  }
  hmax = block_max(hmax);   // (its barriers also publish live / nlive)

  // f(key) for every key of the live lists
  // f(key) for every key of the live lists: wave w takes lists w, w + 8, ...
  // (K1B_UNROLL of them at once), lane l their keys l and l + 64
  auto sweep = [&](auto &&fn) {
    for (int l0 = wave; l0 < nlive; l0 += nwv * K1B_UNROLL) {
      uint64_t v[K1B_UNROLL][2];
#pragma unroll
      for (int u = 0; u < K1B_UNROLL; ++u) {
        const int li = l0 + u * nwv;
        const int l = li < nlive ? live[li] : 0, c = li < nlive ? cnt[l] : 0;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int k = lane + 64 * h;
          v[u][h] = k < c ? base[(size_t)l * K1_LSTRIDE + k] : 0ull;
        }
      }
#pragma unroll
      for (int u = 0; u < K1B_UNROLL; ++u) {
        fn(v[u][0]);
        fn(v[u][1]);
      }
    }
  };
  auto gather = [&](uint64_t thr) {
    sweep([&](uint64_t v) {
      if (v >= thr && v != 0ull) {
        const int at = atomicAdd(&ncand, 1);
        if (at < K1B_FAST) cand[at] = v;
      }
    });
    __syncthreads();
  };
  gather(tau);
  int n = ncand;
  if (n > K1B_FAST) {
    // count(>= lo) >= M > count(>= hi)
    uint64_t lo = tau, hi = hmax + 1;
    while (hi - lo > 1) {
      const uint64_t mid = lo + (hi - lo) / 2;
      int c = 0;
      sweep([&](uint64_t v) { c += (v >= mid && v != 0ull) ? 1 : 0; });
      if (block_sum(c) >= M) lo = mid; else hi = mid;
    }
    __syncthreads();
    if (tid == 0) ncand = 0;
    __syncthreads();
    gather(lo);
    n = min(ncand, K1B_FAST);
  }
  gathered(cand, n);
  // rank of each gathered key among them (keys are distinct)
  const int tpn = split_width(n, nt), sub = tid & (tpn - 1);
  for (int b0 = 0; b0 < n; b0 += nt / tpn) {
    const int i = b0 + tid / tpn;
    const uint64_t k = i < n ? cand[i] : 0ull;
    int rk = i < n ? count_split<true>(cand, n, k, sub, tpn) : 0;
    rk = sum_adjacent(rk, tpn);
    if (i < n && sub == 0 && rk < M) out(rk, k, i);
  }
  for (int m = n + tid; m < M; m += nt) out(m, 0ull, -1);
}

__global__ __launch_bounds__(K1B_THREADS) void k1b_topm_merge(
    const uint64_t *__restrict__ part, int P, int M, int32_t *__restrict__ C,
    float *__restrict__ Cl) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int row = blockIdx.x;
  // (key 0: token -1, the value of an empty slot)
  topm_merge_row(part, P, M, row, smem, [](const uint64_t *, int) {},
                 [&](int rk, uint64_t k, int) {
                   C[(size_t)row * M + rk] = (int32_t)key_tie(k);
                   Cl[(size_t)row * M + rk] = key_val(k);
                 });
}

// The merge fused with the correction tables of the persistent depth loop
// (bf16, M <= 64, r <= 256, s a multiple of TT_NB): workgroup (x, row) merges
// row = request * D + depth and forms
//   G[row][n][j] = W2[C[j]] . W1t[n]   for its TT_NB state units n
// on the matrix cores (fp32 sums over the rank).  The W1t fragments are
// loaded before the merge (they do not depend on it), and the W2 rows of the
// gathered keys are copied into LDS while they are ranked.  Workgroup 0 of
// the row writes C and Cl, and forms g[row][j] = Cl[j] + W2[C[j]] . uH[row]
// on the matrix cores too, against uH split exactly into three bf16 terms
// (every product exact in fp32; the terms' sums are added hi + mid + lo).
constexpr int TT_NB = 128;
constexpr int TT_KS = 8;    // k steps of 32 (rank <= 256)
constexpr int TT_PF = 96;   // most gathered keys whose W2 rows are copied into LDS (>= 64)
size_t topm_tables_smem(int P, int r) {
  return topm_merge_smem(P) + ((size_t)TT_PF * (r / 8) + 64) * 16;
}
__global__ __launch_bounds__(K1B_THREADS) void k_topm_tables(
    const uint64_t *__restrict__ part, int P, int M, int r, int s,
    const uint16_t *__restrict__ W2, const uint16_t *__restrict__ W1t,
    const float *__restrict__ uH, int32_t *__restrict__ C, float *__restrict__ Cl,
    float *__restrict__ G, float *__restrict__ g) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ int32_t tok_s[64];
  __shared__ float cl_s[64];
  __shared__ int16_t gi_s[64];   // gathered position of each rank (-1: none)
  __shared__ int pf_s;           // the gathered keys' W2 rows are in LDS
  __shared__ __align__(16) float uh_s[256];
  // (past the merge's LDS: K1B_FAST keys, P heads, P counts and P list ids)
  uint16_t *w2s = reinterpret_cast<uint16_t *>(smem + (size_t)K1B_FAST * 8 + (size_t)P * 16);
  const int row = blockIdx.y, n0 = blockIdx.x * TT_NB, tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, lr = lane & 15, gq = lane >> 4;
  const int rp = (r + 31) & ~31, nks = rp >> 5, r16 = r >> 3;
  const bool sw = (r16 & 15) == 0;
  const int n = n0 + wave * 16 + lr;   // < s (s % TT_NB == 0)
  uint4 bv[TT_KS];
#pragma unroll
  for (int ks = 0; ks < TT_KS; ++ks)
    if (ks < nks) bv[ks] = *reinterpret_cast<const uint4 *>(W1t + (size_t)n * rp + ks * 32 + gq * 8);
  const bool gw = blockIdx.x == 0 && wave == 0;
  if (gw)   // uH[row] into LDS (r / 4 pieces of 16 bytes; r % 8 == 0)
    lds_copy16(uH + (size_t)row * r + 4 * min(lane, r / 4 - 1), lds_addr(uh_s));
  // 16-byte piece c of W2 row i (gathered position, or rank) goes to LDS
  // position i r / 8 + p, p = c (with r a multiple of 128: c ^ (i & 15), so
  // the A-fragment reads of 16 rows spread over the banks); one copy
  // instruction per 64 pieces, lanes past the end copying the last piece again
  auto copy_rows = [&](int nr, auto tok_of) {
    const int tot = nr * r16;
    for (int base = wave * 64; base < tot; base += K1B_THREADS) {
      const int i = min(base + lane, tot - 1), gk = i / r16, pp = i - gk * r16;
      const int c = sw ? (pp ^ (gk & 15)) : pp;
      const int tk = tok_of(gk);
      lds_copy16(W2 + (size_t)(tk < 0 ? 0 : tk) * r + 8 * c, lds_addr(w2s + (size_t)base * 8));
    }
  };
  topm_merge_row(
      part, P, M, row, smem,
      [&](const uint64_t *cand, int ng) {
        // the gathered keys' W2 rows, copied while they are ranked
        const int pf = ng <= TT_PF;
        if (tid == 0) pf_s = pf;
        if (pf) copy_rows(ng, [&](int gk) { return (int)key_tie(cand[gk]); });
      },
      [&](int rk, uint64_t k, int i) {
        tok_s[rk] = (int32_t)key_tie(k);
        cl_s[rk] = key_val(k);
        gi_s[rk] = (int16_t)i;
        if (blockIdx.x == 0) {
          C[(size_t)row * M + rk] = (int32_t)key_tie(k);
          Cl[(size_t)row * M + rk] = key_val(k);
        }
      });
  __syncthreads();
  const bool pf = pf_s != 0;
  if (!pf) copy_rows(M, [&](int j) { return tok_s[j]; });   // (many gathered keys: the M rows by rank)
  wait_vm<0>();   // this wave's copies have landed; the barrier covers the other waves'
  __syncthreads();
  // g's B fragments: column lr < 3 holds term lr of uH[row], the rest zeros
  uint4 ub[TT_KS];
  if (gw) {
#pragma unroll
    for (int ks = 0; ks < TT_KS; ++ks)
      if (ks < nks) {
        const int k = min(ks * 32 + gq * 8, r - 8);
        const float4 x0 = *reinterpret_cast<const float4 *>(uh_s + k);
        const float4 x1 = *reinterpret_cast<const float4 *>(uh_s + k + 4);
        const bool in = ks * 32 + gq * 8 < r;
        float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = in ? x[e] : 0.f;
        uint4 t3[3];
        split3_bf16(x, t3);
        ub[ks] = lr == 0 ? t3[0] : lr == 1 ? t3[1] : lr == 2 ? t3[2] : make_uint4(0u, 0u, 0u, 0u);
      }
  }
  // A fragments: the candidates' W2 rows from LDS (up to four 16-row tiles;
  // W1t is zero-padded past r, so any finite weight may meet the padding;
  // empty candidate slots are masked at the store)
  const int nmt = (M + 15) >> 4;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
    if (mt < nmt) {
      const int j = min(mt * 16 + lr, M - 1);
      const int ri = pf ? max((int)gi_s[j], 0) : j;
      const uint16_t *wr = w2s + (size_t)ri * r;
      uint4 a[TT_KS];
#pragma unroll
      for (int ks = 0; ks < TT_KS; ++ks)
        if (ks < nks) {
          const int c = min(ks * 4 + gq, r16 - 1);
          a[ks] = *reinterpret_cast<const uint4 *>(wr + 8 * (sw ? c ^ (ri & 15) : c));
        }
      f32x4 acc = {0.f, 0.f, 0.f, 0.f}, ag = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < TT_KS; ++ks)
        if (ks < nks) {
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[ks]), as_bf16x8(bv[ks]), acc,
                                                        0, 0, 0);
          if (gw)
            ag = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[ks]), as_bf16x8(ub[ks]), ag,
                                                         0, 0, 0);
        }
      // lane holds D[candidate mt 16 + 4 gq + t][unit n] (and, for g, the
      // candidate's sum against term lr of uH)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int jj = mt * 16 + 4 * gq + t;
        if (jj < M) G[((size_t)row * s + n) * M + jj] = tok_s[jj] < 0 ? 0.f : acc[t];
      }
      if (gw) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float hi = __shfl(ag[t], gq * 16), mid = __shfl(ag[t], gq * 16 + 1),
                      lo = __shfl(ag[t], gq * 16 + 2);
          const int jj = mt * 16 + 4 * gq + t;
          if (lr == 0 && jj < M) g[(size_t)row * M + jj] = cl_s[jj] + ((hi + mid) + lo);
        }
      }
    }
}

// Round start ahead of the tiled bf16 product: Hb = bf16_rne(H) with rows
// padded to a multiple of 16 by zeros (the tiled products read it), and
// init_round_request for every request.
__global__ __launch_bounds__(256) void k1_stage_hidden(const float *__restrict__ H, int rows,
                                                       int rows_pad, int d,
                                                       uint16_t *__restrict__ Hb,
                                                       const int32_t *__restrict__ root, int b,
                                                       int Dp1, TreeBufs tb) {
  const int q4 = d >> 2;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;   // one float4 each
  if (i < rows_pad * q4) {
    const int rr = i / q4, k = (i - rr * q4) * 4;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (rr < rows) v = *reinterpret_cast<const float4 *>(H + (size_t)rr * d + k);
    const uint32_t lo = (uint32_t)f32_to_bf16_rne(v.x) | ((uint32_t)f32_to_bf16_rne(v.y) << 16);
    const uint32_t hi = (uint32_t)f32_to_bf16_rne(v.z) | ((uint32_t)f32_to_bf16_rne(v.w) << 16);
    *reinterpret_cast<uint2 *>(Hb + (size_t)rr * d + k) = make_uint2(lo, hi);
  }
  if (root)
    for (int q = blockIdx.x; q < b; q += gridDim.x)
      init_round_request(q, root, tb, Dp1, threadIdx.x, blockDim.x);
}

// ---- many hidden rows (32 or more): the base logits as a tiled MFMA
// product written to memory, then the same per-slice candidate lists.
// Exact candidate list for M > 64 (logits in LDS, one row per half-wave):
// the M-th largest key K of the slice is found by bisection, first over the
// 32 bits of the ordered value (the M-th largest value v), then, where more
// than M keys reach v, over the 32-bit tie field among the keys whose value
// is v (keys are distinct, so count(keys >= T) >= M holds exactly for
// T <= K; each step is one comparison per held key and a half-wave sum);
// where exactly M keys reach v, K is the one of value v with the smallest
// tie field.  The value search stops early once a step's count is exactly M
// (for every row of the wave): that value, with tie field 0, bounds exactly
// the M best keys, and it is the list's bound instead of K.
// The keys >= K, exactly M of them, are written unsorted with K as the
// list's bound, the best key and the count (the layout of the fast path).
// A slice with fewer than M keys writes all of them with a zero bound.
template <int MAXC>
__device__ __forceinline__ void wg_topm_bisect(const float *Ls, int lstride, int ncols, int col0,
                                               int nrow, int M, uint64_t *out, size_t rstride) {
  constexpr int KPL = MAXC / 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6, hl = lane & 31;
  // inclusive prefix (over the half-wave, by lane) of c, and its total
  auto scan = [&](int c, int &incl, int &tot) {
    int y;
    incl = c; tot = c;
    y = (int)dpp_u32<0xB1>((uint32_t)tot); if (hl & 1) incl += y; tot += y;
    y = (int)dpp_u32<0x4E>((uint32_t)tot); if (hl & 2) incl += y; tot += y;
    y = __builtin_amdgcn_ds_swizzle(tot, 0x101F); if (hl & 4) incl += y; tot += y;
    y = __builtin_amdgcn_ds_swizzle(tot, 0x201F); if (hl & 8) incl += y; tot += y;
    y = __builtin_amdgcn_ds_swizzle(tot, 0x401F); if (hl & 16) incl += y; tot += y;
  };
  auto total = [&](int c) { int incl, tot; scan(c, incl, tot); return tot; };
  for (int rb = wave * 2; rb < nrow; rb += 2 * nw) {
    const int r = rb + (lane >> 5);
    const bool active = r < nrow;
    uint32_t hv[KPL];   // ordered values, 0 = empty column
    const float *lrow = Ls + (active ? r : 0) * lstride;   // reads in bounds, no branches
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
      const int c = hl + 32 * i;
      const float x = lrow[c < ncols ? c : 0];
      hv[i] = (active && c < ncols) ? f32_ord(x) : 0u;
    }
    auto tie_of = [&](int i) { return 0xFFFFFFFFu - (uint32_t)(col0 + hl + 32 * i); };
    uint64_t T = 0;   // the M-th largest key (0: fewer than M keys)
    if (ncols > M) {
      // (a step whose count is exactly M has found a value bound with
      // exactly M keys at or above it: once every row of the wave has one,
      // the search stops and that bound is the list's)
      uint32_t tv = 0;
      bool sep = false;
      for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = tv | (1u << bit);
        int c = 0;
#pragma unroll
        for (int i = 0; i < KPL; ++i) c += hv[i] >= cand ? 1 : 0;
        const int tc = total(c);
        if (tc >= M) tv = cand;
        sep = sep || tc == M;
        if (__all(!active || sep)) break;
      }
      int cgt = 0, cge = 0;
      uint64_t ntie = 0;   // largest complemented tie among the keys of value tv
#pragma unroll
      for (int i = 0; i < KPL; ++i) {
        cgt += hv[i] > tv ? 1 : 0;
        cge += hv[i] >= tv ? 1 : 0;
        if (hv[i] == tv) ntie = max(ntie, (uint64_t)(0xFFFFFFFFu - tie_of(i)));
      }
      const int need = M - total(cgt);   // keys of value tv that belong in the list
      const int nge = total(cge);
      uint32_t tt;
      if (__all(!active || nge == M)) {
        // (every row of the wave) all keys of value tv belong: K has the smallest tie
        tt = 0xFFFFFFFFu - (uint32_t)group_max_u64<32>(ntie);
      } else {
        tt = 0;
        for (int bit = 31; bit >= 0; --bit) {
          const uint32_t cand = tt | (1u << bit);
          int c = 0;
#pragma unroll
          for (int i = 0; i < KPL; ++i) c += (hv[i] == tv && tie_of(i) >= cand) ? 1 : 0;
          if (total(c) >= need) tt = cand;
        }
      }
      T = sep ? (uint64_t)tv << 32 : ((uint64_t)tv << 32) | tt;
    }
    const uint64_t lo = T ? T : 1ull;   // key 0 marks an empty column
    int c = 0;
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
      const uint64_t k = hv[i] ? ((uint64_t)hv[i] << 32) | tie_of(i) : 0ull;
      if (k >= lo) { ++c; best = k > best ? k : best; }
    }
    int incl, tot;
    scan(c, incl, tot);
    const uint64_t head = group_max_u64<32>(best);
    if (active) {
      uint64_t *outr = out + (size_t)r * rstride;
      int pos = incl - c;
#pragma unroll
      for (int i = 0; i < KPL; ++i) {
        const uint64_t k = hv[i] ? ((uint64_t)hv[i] << 32) | tie_of(i) : 0ull;
        if (k >= lo) outr[pos++] = k;
      }
      if (hl == 0) {
        outr[K1_LCAP] = T;
        outr[K1_LCAP + 1] = head;
        outr[K1_LCAP + 2] = (uint64_t)tot;
      }
    }
  }
}

// The candidate list of (16-row block, vocabulary slice y) from logits in
// memory: the slice's logits go to LDS and the LM-head kernel's epilogue
// runs on them unchanged (slices cover the vocabulary tiles only).
// 8 rows (4 waves) per workgroup: two or more workgroups per CU, so that one
// workgroup's loads overlap another's selection
constexpr int LS_ROWS = 8;
// With ovf given, only the workgroups whose flag k1_lists_bounded raised
// run (exact lists, BISECT); the others leave at once.
template <bool BISECT>
__global__ __launch_bounds__(LS_ROWS / 2 * 64) void k1_lists_from_logits(
    const float *__restrict__ L, int rows, int V, int M, uint64_t *__restrict__ part,
    const int32_t *__restrict__ ovf) {
  extern __shared__ __align__(16) uint8_t smem[];
  float *Ls = reinterpret_cast<float *>(smem);
  const int P = gridDim.y, y = blockIdx.y, row0 = blockIdx.x * LS_ROWS;
  if (ovf && ovf[(size_t)blockIdx.x * P + y] == 0) return;
  const int nrow = min(LS_ROWS, rows - row0);
  const int ntV = (V + 15) >> 4;
  const int t0 = (int)((long long)ntV * y / P), t1 = (int)((long long)ntV * (y + 1) / P);
  const int c0 = t0 * 16, ncols = max(0, min(t1 * 16, V) - c0);
  // the slice's logits into LDS, up to LU loads per thread in flight (16-byte
  // ones when every row segment starts 16-byte aligned: V % 4 == 0, c0 and
  // ncols multiples of 4)
  constexpr int LU = 8;
  const int nt = blockDim.x;
  if ((V & 3) == 0) {
    const int nq = ncols >> 2, n4 = nrow * nq;
    for (int i0 = threadIdx.x; i0 < n4; i0 += nt * LU) {
      f32x4 v[LU];
#pragma unroll
      for (int u = 0; u < LU; ++u) {
        const int i = min(i0 + u * nt, n4 - 1);   // (a repeated load past the end)
        const int rr = i / nq, c = (i - rr * nq) * 4;
        v[u] = *reinterpret_cast<const f32x4 *>(L + (size_t)(row0 + rr) * V + c0 + c);
      }
#pragma unroll
      for (int u = 0; u < LU; ++u) {
        const int i = i0 + u * nt;
        if (i < n4) {
          const int rr = i / nq, c = (i - rr * nq) * 4;
          *reinterpret_cast<f32x4 *>(Ls + rr * K1_MAXCOLS + c) = v[u];
        }
      }
    }
  } else {
    const int n1 = nrow * ncols;
    for (int i0 = threadIdx.x; i0 < n1; i0 += nt * LU) {
      float v[LU];
#pragma unroll
      for (int u = 0; u < LU; ++u) {
        const int i = min(i0 + u * nt, n1 - 1);
        const int rr = i / ncols, c = i - rr * ncols;
        v[u] = L[(size_t)(row0 + rr) * V + c0 + c];
      }
#pragma unroll
      for (int u = 0; u < LU; ++u) {
        const int i = i0 + u * nt;
        if (i < n1) {
          const int rr = i / ncols, c = i - rr * ncols;
          Ls[rr * K1_MAXCOLS + c] = v[u];
        }
      }
    }
  }
  __syncthreads();
  uint64_t *out = part + ((size_t)row0 * P + y) * K1_LSTRIDE;
  if constexpr (BISECT)
    wg_topm_bisect<K1_MAXCOLS>(Ls, K1_MAXCOLS, ncols, c0, nrow, M, out, (size_t)P * K1_LSTRIDE);
  else
    wg_topm_epilogue<K1_MAXCOLS>(Ls, K1_MAXCOLS, ncols, c0, nrow, M, out, (size_t)P * K1_LSTRIDE);
}

// Lists under the row-wide bound (rbound[row], from k1_row_bound: an ordered
// value that at least M keys of the row reach): every slice key of value >=
// the bound, written unsorted with the bound as the list's tau, the slice's
// best key and the count — usually a few keys per slice.  Such a list holds
// every slice key at or above its tau, and M keys of the row reach it, which
// is all the merge relies on.  One row per half-wave, LS_ROWS rows per
// workgroup (the grid of k1_lists_from_logits); lane l reads columns l + 32 i
// straight from the logits (128 contiguous bytes per half-wave and step).
// Where a row's keys would overflow a list (ties) its wave writes nothing and
// the workgroup's flag ovf[block] is set (else cleared); the exact kernel
// then rewrites the lists of the flagged workgroups.
__global__ __launch_bounds__(LS_ROWS / 2 * 64) void k1_lists_bounded(
    const float *__restrict__ L, int rows, int V, const uint32_t *__restrict__ rbound,
    uint64_t *__restrict__ part, int32_t *__restrict__ ovf) {
  constexpr int KPL = K1_MAXCOLS / 32;
  __shared__ int any_over;
  const int P = gridDim.y, y = blockIdx.y, row0 = blockIdx.x * LS_ROWS;
  const int ntV = (V + 15) >> 4;
  const int t0 = (int)((long long)ntV * y / P), t1 = (int)((long long)ntV * (y + 1) / P);
  const int c0 = t0 * 16, ncols = max(0, min(t1 * 16, V) - c0);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, hl = lane & 31;
  const int rr = 2 * wave + (lane >> 5), r = row0 + rr;
  const bool active = r < rows;
  if (threadIdx.x == 0) any_over = 0;
  const float *lr = L + (size_t)(active ? r : row0) * V + c0;   // in bounds for every lane
  uint32_t hv[KPL];
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const int c = hl + 32 * i;
    const float x = lr[c < ncols ? c : 0];
    hv[i] = (active && c < ncols) ? f32_ord(x) : 0u;
  }
  const uint32_t tb = active ? rbound[r] : 0xFFFFFFFFu;
  int cnt = 0;
  uint64_t best = 0;
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const bool in = hv[i] >= tb && hv[i] != 0u;
    cnt += in ? 1 : 0;
    const uint64_t k = ((uint64_t)hv[i] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)(c0 + hl + 32 * i));
    best = (in && k > best) ? k : best;
  }
  // inclusive prefix of the counts over the half-wave, and its total
  int incl = cnt, tot = cnt, yv;
  yv = (int)dpp_u32<0xB1>((uint32_t)tot); if (hl & 1) incl += yv; tot += yv;
  yv = (int)dpp_u32<0x4E>((uint32_t)tot); if (hl & 2) incl += yv; tot += yv;
  yv = __builtin_amdgcn_ds_swizzle(tot, 0x101F); if (hl & 4) incl += yv; tot += yv;
  yv = __builtin_amdgcn_ds_swizzle(tot, 0x201F); if (hl & 8) incl += yv; tot += yv;
  yv = __builtin_amdgcn_ds_swizzle(tot, 0x401F); if (hl & 16) incl += yv; tot += yv;
  const uint64_t head = group_max_u64<32>(best);
  const bool over = __any(active && (tb == 0u || tot > K1_LCAP));
  __syncthreads();   // (any_over cleared)
  if (over) {
    if (lane == 0) any_over = 1;
  } else if (active) {
    uint64_t *outr = part + ((size_t)r * P + y) * K1_LSTRIDE;
    int pos = incl - cnt;
#pragma unroll
    for (int i = 0; i < KPL; ++i)
      if (hv[i] >= tb && hv[i] != 0u)
        outr[pos++] = ((uint64_t)hv[i] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)(c0 + hl + 32 * i));
    if (hl == 0) {
      outr[K1_LCAP] = (uint64_t)tb << 32;
      outr[K1_LCAP + 1] = head;
      outr[K1_LCAP + 2] = (uint64_t)tot;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) ovf[(size_t)blockIdx.x * P + y] = any_over;
}

// Row-wide list bound: the M-th largest of the row's ng column-group maxima
// (ordered values; ng >= M).  Each maximum is the value of a distinct key
// of the row, so at least M keys reach the bound, and with many narrow
// groups it lies close below the row's M-th largest value.  One workgroup
// per row, radix passes of 8 bits from the top: each pass counts the
// maxima that match the digits found so far by their next digit and keeps
// the digit where the count from the top reaches the number still wanted.
constexpr int RB_THREADS = 256;
__global__ __launch_bounds__(RB_THREADS) void k1_row_bound(const uint32_t *__restrict__ gmax,
                                                          int ng, int ldg, int M,
                                                          uint32_t *__restrict__ bound) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t pick[2];
  const int tid = threadIdx.x, lane = tid & 63;
  const uint32_t *gm = gmax + (size_t)blockIdx.x * ldg;
  uint32_t prefix = 0, pmask = 0, need = (uint32_t)M;
  for (int shift = 24; shift >= 0; shift -= 8) {
    hist[tid] = 0u;
    __syncthreads();
    for (int i = tid; i < ng; i += RB_THREADS) {
      const uint32_t k = gm[i];
      if ((k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      // lane l: digits 255 - 4 l .. 252 - 4 l; counts of the higher digits first
      uint32_t c[4], sum = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) { c[j] = hist[255 - 4 * lane - j]; sum += c[j]; }
      uint32_t before = (uint32_t)wave_scan_add((int)sum) - sum;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (before < need && before + c[j] >= need) { pick[0] = 255u - 4u * lane - j; pick[1] = before; }
        before += c[j];
      }
    }
    __syncthreads();
    prefix |= pick[0] << shift;
    pmask |= 255u << shift;
    need -= pick[1];
  }
  if (tid == 0) bound[blockIdx.x] = prefix;
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

hipError_t lmhead_prepare(int wtype, int ring, size_t lds_bytes) {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k1b_topm_merge),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, 131072);
  if (e == hipSuccess)
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_topm_tables),
                            hipFuncAttributeMaxDynamicSharedMemorySize, 131072);
  if (e != hipSuccess || wtype != WT_BF16) return e;
  const void *fn = ring == 2 ? k1_fn<2>() : ring == 1 ? k1_fn<1>() : k1_fn<0>();
  return set_lds_limit(fn, lds_bytes);
}

hipError_t launch_lmhead(const LMHeadArgs &a, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  dim3 grid((a.rows + 15) / 16, a.P);
  if (a.wtype == WT_BF16) {
    const size_t sm = lmhead_smem(a.d, a.wtype, a.ring);
#define K1_LAUNCH(RING)                                                                           \
  hipExtLaunchKernelGGL((k1_lmhead_bf16<RING>), grid, dim3(K1_WAVES * 64), (uint32_t)sm, st, ev0,  \
                        ev1, 0u, a.H, a.rows, a.d,                                                 \
                        static_cast<const uint16_t *>(a.W), a.V, a.bias, a.M, a.part,              \
                        static_cast<const uint16_t *>(a.W1), a.ldw1, a.r, a.uH, a.root, a.b,       \
                        a.Dp1, a.t)
    if (a.ring == 2) K1_LAUNCH(2);
    else if (a.ring == 1) K1_LAUNCH(1);
    else K1_LAUNCH(0);
#undef K1_LAUNCH
  } else {
    hipExtLaunchKernelGGL(k1_lmhead_f32, grid, dim3(K1F_THREADS), 0u, st, ev0, ev1, 0u, a.H,
                          a.rows, a.d, static_cast<const float *>(a.W), a.V, a.bias, a.M, a.part,
                          a.root, a.b, a.Dp1, a.t);
  }
  return hipGetLastError();
}

bool lmhead_tiled_ok(int rows, int d, int wtype) {
  return wtype == WT_BF16 && rows >= 32 && d % 64 == 0;
}

hipError_t launch_lmhead_tiled(const LMHeadArgs &a, float *logits, hipStream_t st, hipEvent_t ev0,
                               hipEvent_t ev1) {
  // the kernel's own start and end events time the product alone (the list
  // kernel falls into the next stage)
  hipError_t e;
  GemmArgs g{a.rows, a.V, a.d, a.Hb, WT_BF16, a.d, nullptr, 0, a.W, WT_BF16, a.d, a.bias,
             nullptr, 0, 1, 0, 0, logits, a.V};
  // one row tile: 320-token tiles make 1.9 rounds of workgroups over the
  // vocabulary (475 tiles at V = 151936) instead of 2.3 rounds of 256
  const int bn = a.rows <= 128 ? 320 : 256;
  const int bm = a.rows >= 256 ? 256 : 128;
  const int gw = bn / 4;   // columns per wave of the tile: the maxima's groups
  const int ng = (a.V + gw - 1) / gw;
  // the row-wide list bound needs M groups (lmhead_groups sizes gmax for
  // the narrowest groups)
  const bool rowb = a.gmax && a.rbound && a.ovf && ng >= a.M;
  if (rowb) { g.gmax = a.gmax; g.ldg = lmhead_groups(a.V); }
  if (!mm_ok(g)) return hipErrorInvalidValue;   // lmhead_tiled_ok admits bf16 rows with d % 64 == 0 only
  e = launch_mm_lm(g, bm, bn, st, ev0, ev1);
  if (e != hipSuccess) return e;
  if (rowb) {
    hipLaunchKernelGGL(k1_row_bound, dim3(a.rows), dim3(RB_THREADS), 0, st, a.gmax, ng,
                       lmhead_groups(a.V), a.M, a.rbound);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // lists under the row bound, exact lists (bisection) for the workgroups
  // whose keys overflowed them; without the bound, exact lists for M > 64,
  // else the fast per-slice lists (each a kernel of its own: fewer registers)
  const dim3 lgrid((a.rows + LS_ROWS - 1) / LS_ROWS, a.P);
  if (rowb)
    hipLaunchKernelGGL(k1_lists_bounded, lgrid, dim3(LS_ROWS / 2 * 64), 0, st, (const float *)logits,
                       a.rows, a.V, (const uint32_t *)a.rbound, a.part, a.ovf);
  if (rowb || a.M > 64)
    hipExtLaunchKernelGGL(k1_lists_from_logits<true>, lgrid,
                          dim3(LS_ROWS / 2 * 64), (uint32_t)(LS_ROWS * K1_MAXCOLS * 4), st, nullptr, nullptr,
                          0u, (const float *)logits, a.rows, a.V, a.M, a.part,
                          rowb ? (const int32_t *)a.ovf : nullptr);
  else
    hipExtLaunchKernelGGL(k1_lists_from_logits<false>, dim3((a.rows + LS_ROWS - 1) / LS_ROWS, a.P),
                          dim3(LS_ROWS / 2 * 64), (uint32_t)(LS_ROWS * K1_MAXCOLS * 4), st, nullptr, nullptr,
                          0u, (const float *)logits, a.rows, a.V, a.M, a.part, nullptr);
  return hipGetLastError();
}

hipError_t launch_stage_hidden(const LMHeadArgs &a, hipStream_t st) {
  if (a.wtype != WT_BF16) return hipSuccess;   // the fp32 kernel starts the round itself
  const int rows_pad = (a.rows + 15) & ~15, n4 = rows_pad * (a.d >> 2);
  hipLaunchKernelGGL(k1_stage_hidden, dim3((n4 + 255) / 256), dim3(256), 0, st, a.H, a.rows,
                     rows_pad, a.d, a.Hb, a.root, a.b, a.Dp1, a.t);
  return hipGetLastError();
}

bool topm_tables_ok(int M, int r, int s, const void *W2, const void *W1t) {
  return M <= 64 && r % 8 == 0 && r <= 32 * TT_KS && s % TT_NB == 0 &&
         reinterpret_cast<uintptr_t>(W2) % 16 == 0 && reinterpret_cast<uintptr_t>(W1t) % 16 == 0;
}

hipError_t launch_topm_tables(const uint64_t *part, int P, int M, int rows, int r, int s,
                              const void *W2, const void *W1t, const float *uH, int32_t *C,
                              float *Cl, float *G, float *g, hipStream_t st) {
  if (!topm_tables_ok(M, r, s, W2, W1t)) return hipErrorInvalidValue;
  const size_t sm = topm_tables_smem(P, r);
  hipLaunchKernelGGL(k_topm_tables, dim3(s / TT_NB, rows), dim3(K1B_THREADS), sm, st, part, P, M,
                     r, s, static_cast<const uint16_t *>(W2), static_cast<const uint16_t *>(W1t),
                     uH, C, Cl, G, g);
  return hipGetLastError();
}

hipError_t launch_topm_merge(const uint64_t *part, int P, int M, int rows, int32_t *C,
                             float *Cl, hipStream_t st) {
  const size_t sm = topm_merge_smem(P);
  hipLaunchKernelGGL(k1b_topm_merge, dim3(rows), dim3(K1B_THREADS), sm, st, part, P, M, C, Cl);
  return hipGetLastError();
}

}  // namespace dtree
