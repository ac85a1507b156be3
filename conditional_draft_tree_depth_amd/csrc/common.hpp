// Device helpers shared by the draft-tree kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dtree {

constexpr int kWave = 64;

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}
// Round a finite fp32 to bf16, nearest-even.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Weight element loads: bf16 weights arrive as raw uint16 patterns.
__device__ __forceinline__ float wload(const uint16_t *p, size_t i) {
  return bf16_bits_to_f32(p[i]);
}
__device__ __forceinline__ float wload(const float *p, size_t i) { return p[i]; }

// ---------------------------------------------------------------- keys
// Monotone map of fp32 to uint32 (larger float -> larger integer); -0 is
// folded onto +0 so the two compare equal, as they do as floats.
__device__ __forceinline__ uint32_t f32_ord(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float ord_f32(uint32_t o) {
  uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
  return __uint_as_float(u);
}
// 64-bit selection key, larger is better: value descending, then the tie
// field ascending.  Valid keys are never 0, which marks an empty slot.
__device__ __forceinline__ uint64_t make_key(float v, uint32_t tie) {
  return ((uint64_t)f32_ord(v) << 32) | (uint64_t)(0xFFFFFFFFu - tie);
}
__device__ __forceinline__ uint32_t key_tie(uint64_t k) {
  return 0xFFFFFFFFu - (uint32_t)(k & 0xFFFFFFFFull);
}
__device__ __forceinline__ float key_val(uint64_t k) { return ord_f32((uint32_t)(k >> 32)); }

// ---------------------------------------------------------------- wave ops
// Lane exchanges inside rows of 16 lanes go through DPP (no LDS round trip):
// 0xB1 = lane ^ 1, 0x4E = lane ^ 2, 0x141 = 7 - lane within 8, 0x140 =
// 15 - lane within 16; across rows, ds_swizzle 0x401F = lane ^ 16 within 32.
// For an all-reduce any partner in the other half of a group will do.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}
template <int STEP>
__device__ __forceinline__ uint32_t xchg_u32(uint32_t v) {   // partner for group size 2 STEP
  if constexpr (STEP == 1) return dpp_u32<0xB1>(v);
  else if constexpr (STEP == 2) return dpp_u32<0x4E>(v);
  else if constexpr (STEP == 4) return dpp_u32<0x141>(v);
  else if constexpr (STEP == 8) return dpp_u32<0x140>(v);
  else if constexpr (STEP == 16) return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F);
  else return (uint32_t)__shfl_xor((int)v, 32);
}
template <int STEP>
__device__ __forceinline__ float xchg_f32(float v) {
  return __uint_as_float(xchg_u32<STEP>(__float_as_uint(v)));
}
template <int STEP>
__device__ __forceinline__ uint64_t xchg_u64(uint64_t v) {
  return ((uint64_t)xchg_u32<STEP>((uint32_t)(v >> 32)) << 32) | xchg_u32<STEP>((uint32_t)v);
}
// inclusive prefix sum over the 64 lanes of a wave (DPP: shifts within rows
// of 16 lanes, then the row ends broadcast into the later rows)
__device__ __forceinline__ int wave_scan_add(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);   // row_bcast:15, rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);   // row_bcast:31, rows 2, 3
  return v;
}
__device__ __forceinline__ float wave_max_f32(float v) {
  v = fmaxf(v, xchg_f32<1>(v));
  v = fmaxf(v, xchg_f32<2>(v));
  v = fmaxf(v, xchg_f32<4>(v));
  v = fmaxf(v, xchg_f32<8>(v));
  v = fmaxf(v, xchg_f32<16>(v));
  return fmaxf(v, xchg_f32<32>(v));
}
__device__ __forceinline__ float wave_sum_f32(float v) {
  v += xchg_f32<1>(v);
  v += xchg_f32<2>(v);
  v += xchg_f32<4>(v);
  v += xchg_f32<8>(v);
  v += xchg_f32<16>(v);
  return v + xchg_f32<32>(v);
}
// The same maximum and sum with the exchanges across rows and across halves
// done by the lane-pair swaps (vector ALU only, no LDS round trip); every
// lane of the wave must be active.  Each swap leaves a lane its own value
// and its partner's, one in each slot, and the operations are symmetric, so
// the results are those of wave_max_f32 / wave_sum_f32 bit for bit.
__device__ __forceinline__ float pair_max_f32(float v, bool x32) {
  const uint32_t u = __float_as_uint(v);
  const auto r = x32 ? __builtin_amdgcn_permlane32_swap(u, u, false, false)
                     : __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum_f32(float v, bool x32) {
  const uint32_t u = __float_as_uint(v);
  const auto r = x32 ? __builtin_amdgcn_permlane32_swap(u, u, false, false)
                     : __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float wave_max_f32_full(float v) {
  v = fmaxf(v, xchg_f32<1>(v));
  v = fmaxf(v, xchg_f32<2>(v));
  v = fmaxf(v, xchg_f32<4>(v));
  v = fmaxf(v, xchg_f32<8>(v));
  return pair_max_f32(pair_max_f32(v, false), true);
}
__device__ __forceinline__ float wave_sum_f32_full(float v) {
  v += xchg_f32<1>(v);
  v += xchg_f32<2>(v);
  v += xchg_f32<4>(v);
  v += xchg_f32<8>(v);
  return pair_sum_f32(pair_sum_f32(v, false), true);
}
// max over aligned groups of WIDTH lanes (a power of two <= 64)
template <int WIDTH>
__device__ __forceinline__ uint64_t group_max_u64(uint64_t v) {
  uint64_t w;
  if constexpr (WIDTH >= 2) { w = xchg_u64<1>(v); v = w > v ? w : v; }
  if constexpr (WIDTH >= 4) { w = xchg_u64<2>(v); v = w > v ? w : v; }
  if constexpr (WIDTH >= 8) { w = xchg_u64<4>(v); v = w > v ? w : v; }
  if constexpr (WIDTH >= 16) { w = xchg_u64<8>(v); v = w > v ? w : v; }
  if constexpr (WIDTH >= 32) { w = xchg_u64<16>(v); v = w > v ? w : v; }
  if constexpr (WIDTH >= 64) { w = xchg_u64<32>(v); v = w > v ? w : v; }
  return v;
}

// Block-wide bitonic sort of n (power of two) keys with an int payload,
// descending.  All threads of the block must call it.
__device__ inline void block_bitonic_desc(uint64_t *keys, int32_t *vals, int n) {
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n; i += blockDim.x) {
        int ixj = i ^ j;
        if (ixj > i) {
          uint64_t a = keys[i], b = keys[ixj];
          bool desc = (i & k) == 0;
          if (desc ? (a < b) : (a > b)) {
            keys[i] = b;
            keys[ixj] = a;
            int32_t t = vals[i];
            vals[i] = vals[ixj];
            vals[ixj] = t;
          }
        }
      }
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------- rank counts
// threads per element when nt threads count ranks of n elements: a power of
// two up to 16, all elements in one pass when they fit
__device__ __forceinline__ int split_width(int n, int nt) {
  int tpn = 1;
  while (tpn * 2 * n <= nt && tpn < 16) tpn *= 2;
  return tpn;
}

// part `part` of tpn of the count of a[0..n) ordered before x (greater if
// GREATER, else smaller).  a is 16-byte aligned and the parts start at
// multiples of 8 elements, so groups of 8 come in as 16-byte LDS reads.
template <bool GREATER, typename T>
__device__ __forceinline__ int count_split(const T *a, int n, T x, int part, int tpn) {
  static_assert(sizeof(T) == 4 || sizeof(T) == 8, "32- or 64-bit keys");
  const int per = ((n + tpn - 1) / tpn + 7) & ~7, j0 = part * per, j1 = min(n, j0 + per);
  int cnt = 0, j = j0;
  for (; j + 8 <= j1; j += 8) {
    constexpr int NV = 8 * (int)sizeof(T) / 16;
    uint4 raw[NV];
#pragma unroll
    for (int u = 0; u < NV; ++u) raw[u] = reinterpret_cast<const uint4 *>(a + j)[u];
    uint32_t w[4 * NV];
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      w[4 * u] = raw[u].x; w[4 * u + 1] = raw[u].y; w[4 * u + 2] = raw[u].z; w[4 * u + 3] = raw[u].w;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      T v;
      if constexpr (sizeof(T) == 8) v = ((uint64_t)w[2 * u + 1] << 32) | w[2 * u];
      else v = w[u];
      cnt += GREATER ? (v > x) : (v < x);
    }
  }
  for (; j < j1; ++j) cnt += GREATER ? (a[j] > x) : (a[j] < x);
  return cnt;
}

// sum over the tpn adjacent lanes of an element (every lane of the wave
// takes part)
__device__ __forceinline__ int sum_adjacent(int cnt, int tpn) {
  if (tpn >= 2) cnt += (int)xchg_u32<1>((uint32_t)cnt);
  if (tpn >= 4) cnt += (int)xchg_u32<2>((uint32_t)cnt);
  if (tpn >= 8) cnt += (int)xchg_u32<4>((uint32_t)cnt);
  if (tpn >= 16) cnt += (int)xchg_u32<8>((uint32_t)cnt);
  return cnt;
}

__device__ __forceinline__ int next_pow2(int n) {
  int p = 1;
  while (p < n) p <<= 1;
  return p;
}

// Exact three-term bf16 split of 8 fp32 values, each term packed as one
// 16-byte MFMA fragment: hi = bf16(x), mid = bf16(x - hi), lo = bf16(x - hi
// - mid), so x - hi - mid - lo is below 2^-24 |x|; a bf16 weight times each
// term is exact in fp32.
__device__ __forceinline__ void split3_bf16(const float (&x)[8], uint4 (&t)[3]) {
  uint32_t w[3][4];
#pragma unroll
  for (int k = 0; k < 8; k += 2) {
    uint32_t h[3][2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const uint16_t b0 = f32_to_bf16_rne(x[k + e]);
      const float r1 = x[k + e] - bf16_bits_to_f32(b0);
      const uint16_t b1 = f32_to_bf16_rne(r1);
      const uint16_t b2 = f32_to_bf16_rne(r1 - bf16_bits_to_f32(b1));
      h[0][e] = b0; h[1][e] = b1; h[2][e] = b2;
    }
#pragma unroll
    for (int q = 0; q < 3; ++q) w[q][k / 2] = h[q][0] | (h[q][1] << 16);
  }
#pragma unroll
  for (int q = 0; q < 3; ++q) t[q] = make_uint4(w[q][0], w[q][1], w[q][2], w[q][3]);
}

// ---- staged tiles: direct global-to-LDS copies with waits of our own ----
// The compiler, seeing a copy into LDS in flight, waits for every such copy
// before any LDS read it cannot prove unrelated (and a workgroup fence
// waits for all of them), which serialises a multi-stage ring.  The copies
// below are issued where the compiler does not track them; the kernel
// waits for its own copies with wait_vm before a bare barrier.

// 16 bytes per lane from g into LDS at byte address lds + 16 * lane (lds
// is uniform over the wave)
__device__ __forceinline__ void lds_copy16(const void *g, uint32_t lds) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(g) : "memory", "m0");
#pragma clang diagnostic pop
}
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void *)p;
}
// this wave's vector memory operations: at most N still in flight (gfx9
// encoding, lgkmcnt and expcnt left free)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
// workgroup barrier without a memory fence (the compiler keeps memory
// accesses on their side of it)
__device__ __forceinline__ void bare_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace dtree
