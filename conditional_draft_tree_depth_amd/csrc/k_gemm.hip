// Row-gathered products of activations and stored (bf16/fp32) weights, and
// the GRU cell.
//
// Used for the path-independent projection uH = W1[:, :d] Hq, the per-branch
// part W1[:, d:] S of the low-rank head ("Resumen Técnico: Domino",
// Metodología 2: [H_i ; S_{i-1}] is projected to rank r), and the GRU input
// and state projections.  fp32 activations are never rounded to bf16 (the
// GRU state enters the matrix cores as an exact three-term bf16 split);
// accumulation is fp32.  Three kernels: bf16 weights with fewer than 256
// rows, a contraction split over 8 waves (k_skinny_bf16); bf16 operands
// with many rows, 256 x 128 or 128 x 128 tiles (k_mm); anything else, a plain
// tiled VALU product (k_gemm_xwT: 64 x 64 outputs per 256-thread
// workgroup, 16-wide k chunks staged in LDS).
#include <algorithm>
#include <hip/hip_ext.h>

#include "common.hpp"
#include "kernels.hpp"

namespace dtree {

constexpr int GT = 64, GK = 16;

template <typename XT>
__device__ __forceinline__ float xload(const XT *p, size_t i, int xround);
template <>
__device__ __forceinline__ float xload<float>(const float *p, size_t i, int xround) {
  const float v = p[i];
  return xround ? bf16_bits_to_f32(f32_to_bf16_rne(v)) : v;
}
template <>
__device__ __forceinline__ float xload<uint16_t>(const uint16_t *p, size_t i, int) {
  return bf16_bits_to_f32(p[i]);
}

template <typename XT, typename WT>
__global__ __launch_bounds__(256) void k_gemm_xwT(GemmArgs a) {
  __shared__ float Xs[GK][GT + 4];
  __shared__ float Ws[GK][GT + 4];
  const XT *X = static_cast<const XT *>(a.X);
  const WT *Wt = static_cast<const WT *>(a.W);
  const int tid = threadIdx.x;
  const int r0 = blockIdx.y * GT, n0 = blockIdx.x * GT;
  const int tx = tid & 15, ty = tid >> 4;
  // loader coordinates: 64 rows x 16 k, 4 consecutive k per thread
  const int lrow = tid >> 2, lk = (tid & 3) * 4;
  const int xr = r0 + lrow;
  const bool xok = xr < a.R;
  const size_t xbase = xok ? (size_t)(a.xidx ? a.xidx[xr] : xr) * a.ldx : 0;
  const int wn = n0 + lrow;
  const bool wok = wn < a.N;
  const size_t wbase = (size_t)wn * a.ldw;

  float acc[4][4] = {};
  for (int k0 = 0; k0 < a.Kd; k0 += GK) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int k = k0 + lk + q;
      Xs[lk + q][lrow] = (xok && k < a.Kd) ? xload<XT>(X, xbase + k, a.xround) : 0.f;
      Ws[lk + q][lrow] = (wok && k < a.Kd) ? wload(Wt, wbase + k) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < GK; ++k) {
      float xv[4], wv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) xv[i] = Xs[k][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) wv[j] = Ws[k][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] += xv[i] * wv[j];
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = r0 + ty * 4 + i;
    if (row >= a.R) continue;
    const float *add = a.addend ? a.addend + (size_t)((row / a.adiv) * a.amul + a.aoff) * a.lda : nullptr;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n >= a.N) continue;
      float v = acc[i][j];
      if (a.bias && n >= a.bias_n0) v += a.bias[n - a.bias_n0];
      if (add && n < a.add_n) v += add[n];
      a.Y[(size_t)row * a.ldy + n] = v;
    }
  }
}

// Row-gathered product on MFMA for bf16 weights: Y = X W^T (+ bias, +
// addend), any number of activation rows.  One workgroup takes 16 weight
// rows (the A operand, loaded once into registers) and up to 128 activation
// rows; its 8 waves split the contraction (wave w takes the 32-wide k-steps
// w, w + 8, ...), so a 3072 x 2560 weight is streamed by 192 x 8 waves with
// all of a wave's weight loads in flight at once.  Activation fragments (the
// B operand) come straight from global memory (they are small and shared
// by every workgroup, so they stay in L2); the fragments of the next 16-row
// block are loaded while the current one feeds the matrix cores.  The 8
// partial sums of every output are added in a fixed order through LDS.
// fp32 activations that must not be rounded (the GRU state) are split
// exactly into three bf16 terms x = hi + mid + lo (each term is the bf16
// rounding of what the previous ones left, so the remainder is below
// 2^-24 |x|); every term is multiplied by the same weight fragment.
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
constexpr int SK_WAVES = 8;       // waves per workgroup (contraction split)
constexpr int SK_RB = 8;          // 16-row activation blocks per workgroup
constexpr int SK_KSW_B = 16;      // k-steps per wave, bf16 activations: K <= 4096
constexpr int SK_KSW_F = 8;       // k-steps per wave, fp32 activations: K <= 2048

__device__ __forceinline__ bf16x8 sk_bf(uint4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ f32x4 sk_mfma(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(sk_bf(a), sk_bf(b), c, 0, 0, 0);
}
__device__ __forceinline__ uint32_t sk_pack(uint16_t lo, uint16_t hi) {
  return (uint32_t)lo | ((uint32_t)hi << 16);
}

// Term t (0: hi, 1: mid, 2: lo; TERMS == 1: the bf16 rounding) of 8 fp32
// activations, packed as one B fragment.
template <int TERMS>
__device__ __forceinline__ void sk_split(const float4 &x0, const float4 &x1, uint4 (&t)[TERMS]) {
  const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
  uint16_t h[TERMS][8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    h[0][k] = f32_to_bf16_rne(x[k]);
    if constexpr (TERMS == 3) {
      const float r1 = x[k] - bf16_bits_to_f32(h[0][k]);
      h[1][k] = f32_to_bf16_rne(r1);
      h[2][k] = f32_to_bf16_rne(r1 - bf16_bits_to_f32(h[1][k]));
    }
  }
#pragma unroll
  for (int q = 0; q < TERMS; ++q)
    t[q] = make_uint4(sk_pack(h[q][0], h[q][1]), sk_pack(h[q][2], h[q][3]),
                      sk_pack(h[q][4], h[q][5]), sk_pack(h[q][6], h[q][7]));
}

// CT column tiles of 16 per workgroup: each activation fragment (and its
// split) is loaded once and multiplied by CT weight fragments, so that
// CT-fold fewer workgroups re-read the activation rows (RBM row blocks at
// most, the partial sums of all of them in LDS).
template <int TERMS, typename XT, int KSW, int CT = 1, int RBM = SK_RB>
__global__ __launch_bounds__(SK_WAVES * 64) void k_skinny_bf16(GemmArgs a, int RB) {
  constexpr bool XB = sizeof(XT) == 2;
  constexpr int NC = 16 * CT;   // output columns per workgroup
  __shared__ __align__(16) float red[SK_WAVES * RBM * 16 * NC];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * NC, r0 = blockIdx.y * (16 * RB);
  const int R = a.Rdev ? min(*a.Rdev, a.R) : a.R;   // rows past the device count: no work
  if (r0 >= R) return;
  const int nrb = min(RB, (R - r0 + 15) >> 4);
  const int nks = a.Kd >> 5;
  // the bias and addend terms of the outputs this thread writes at the end
  // (at most OPT of them): with several column tiles they are loaded first
  // (they depend on nothing computed here), else at the end (measured: the
  // four-tile form's 8B x8 depth loop 419 -> 412 us, the one-tile form's
  // wide depth loop 365 -> 380 us with its registers grown)
  constexpr int OPT = (RBM * 16 * NC + SK_WAVES * 64 - 1) / (SK_WAVES * 64);
  constexpr bool PRE = CT > 1;
  float pb[OPT], pa[OPT];
  auto terms = [&](int k) {
    const int o = tid + k * SK_WAVES * 64;
    const int rb = o / (16 * NC), rr = (o / NC) & 15, nn = o % NC;
    const int row = r0 + rb * 16 + rr, n = n0 + nn;
    pb[k] = 0.f;
    pa[k] = 0.f;
    if (o < nrb * 16 * NC && row < R && n < a.N) {
      if (a.bias && n >= a.bias_n0) pb[k] = a.bias[n - a.bias_n0];
      if (a.addend && n < a.add_n) pa[k] = a.addend[(size_t)((row / a.adiv) * a.amul + a.aoff) * a.lda + n];
    }
  };
  if constexpr (PRE) {
#pragma unroll
    for (int k = 0; k < OPT; ++k) terms(k);
  }
  // k-steps past the contraction load the last one again (every load is
  // unconditional and in bounds) and are skipped at the products
  uint4 wa[CT][KSW];
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    const uint16_t *wrow =
        static_cast<const uint16_t *>(a.W) + (size_t)min(n0 + 16 * c + lr, a.N - 1) * a.ldw + g * 8;
#pragma unroll
    for (int i = 0; i < KSW; ++i)
      wa[c][i] = *reinterpret_cast<const uint4 *>(wrow + min(wave + SK_WAVES * i, nks - 1) * 32);
  }
  // activation row of lane lr in row block rb (rows past R repeat the last
  // row; their sums are never stored)
  auto xrow = [&](int rb) -> size_t {
    const int row = min(r0 + rb * 16 + lr, R - 1);
    return (size_t)(a.xidx ? a.xidx[row] : row) * a.ldx + g * 8;
  };
  // lane holds Y[row lr][weight row 4 g + t] of column tile c
  auto put = [&](int rb, int c, const f32x4 &acc) {
    *reinterpret_cast<f32x4 *>(red + ((wave * RBM + rb) * 16 + lr) * NC + 16 * c + 4 * g) = acc;
  };
  if constexpr (XB) {
    const uint16_t *X = static_cast<const uint16_t *>(a.X);
    uint4 xc[KSW], xn[KSW];
    auto load = [&](int rb, uint4 (&xv)[KSW]) {
      const uint16_t *xp = X + xrow(rb);
#pragma unroll
      for (int i = 0; i < KSW; ++i)
        xv[i] = *reinterpret_cast<const uint4 *>(xp + min(wave + SK_WAVES * i, nks - 1) * 32);
    };
    load(0, xc);
    for (int rb = 0; rb < nrb; ++rb) {
      if (rb + 1 < nrb) load(rb + 1, xn);
      f32x4 acc[CT];
#pragma unroll
      for (int c = 0; c < CT; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < KSW; ++i)
        if (wave + SK_WAVES * i < nks) {
#pragma unroll
          for (int c = 0; c < CT; ++c) acc[c] = sk_mfma(wa[c][i], xc[i], acc[c]);
        }
#pragma unroll
      for (int c = 0; c < CT; ++c) put(rb, c, acc[c]);
#pragma unroll
      for (int i = 0; i < KSW; ++i) xc[i] = xn[i];
    }
  } else {
    const float *X = static_cast<const float *>(a.X);
    float4 xc[KSW][2], xn[KSW][2];
    auto load = [&](int rb, float4 (&xv)[KSW][2]) {
      const float *xp = X + xrow(rb);
#pragma unroll
      for (int i = 0; i < KSW; ++i) {
        const float *pk = xp + min(wave + SK_WAVES * i, nks - 1) * 32;
        xv[i][0] = *reinterpret_cast<const float4 *>(pk);
        xv[i][1] = *reinterpret_cast<const float4 *>(pk + 4);
      }
    };
    load(0, xc);
    for (int rb = 0; rb < nrb; ++rb) {
      if (rb + 1 < nrb) load(rb + 1, xn);
      f32x4 acc[CT];
#pragma unroll
      for (int c = 0; c < CT; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < KSW; ++i)
        if (wave + SK_WAVES * i < nks) {
          uint4 t[TERMS];
          sk_split<TERMS>(xc[i][0], xc[i][1], t);
#pragma unroll
          for (int c = 0; c < CT; ++c)
#pragma unroll
            for (int q = 0; q < TERMS; ++q) acc[c] = sk_mfma(wa[c][i], t[q], acc[c]);
        }
#pragma unroll
      for (int c = 0; c < CT; ++c) put(rb, c, acc[c]);
#pragma unroll
      for (int i = 0; i < KSW; ++i) { xc[i][0] = xn[i][0]; xc[i][1] = xn[i][1]; }
    }
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < OPT; ++k) {
    const int o = tid + k * SK_WAVES * 64;
    if (o >= nrb * 16 * NC) break;
    const int rb = o / (16 * NC), rr = (o / NC) & 15, nn = o % NC;
    const int row = r0 + rb * 16 + rr, n = n0 + nn;
    if constexpr (!PRE) terms(k);
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < SK_WAVES; ++w) v += red[((w * RBM + rb) * 16 + rr) * NC + nn];
    if (row < R && n < a.N) {
      if (a.bias && n >= a.bias_n0) v += pb[k];
      if (a.addend && n < a.add_n) v += pa[k];
      a.Y[(size_t)row * a.ldy + n] = v;
    }
  }
}

// Many activation rows (256 or more), bf16 x bf16: WM x WN waves per
// workgroup, each a (BM/WM) x (BN/WN) block of 16 x 16 MFMA tiles (two waves
// per SIMD, or two workgroups per CU, so that one wave's fragment reads
// overlap another's MFMAs).  k chunks of 64: a row's chunk is one 128-byte
// line, eight 16-byte pieces, piece c of row q stored at position c ^ (q & 7)
// so that the fragment reads of 16 rows hit distinct banks (32-wide chunks,
// half lines, measured slower: more LDS bank conflicts and, for a streamed
// operand, the other half of each line fetched again).  A ring of STAGES
// chunks, STAGES - 1 of them in flight while one is read; the copies are
// tracked by the kernel's own waits.  Activation rows are gathered through
// xidx; the weights' k index runs modulo kw (a state split into bf16 planes
// meets the same weights once per plane); rows past the device count *Rdev
// do no work.  Tasks run in XCD-contiguous runs, so the row tiles of one
// weight tile share an L2.
template <int BM, int BN, int WM, int WN, int STAGES>
__global__ __launch_bounds__(WM * WN * 64) void k_mm(GemmArgs a) {
  constexpr int NW = WM * WN;
  constexpr int TM = BM / WM / 16, TN = BN / WN / 16;   // 16 x 16 tiles per wave
  constexpr int BK = 64;
  constexpr int CPR = BK / 8;                 // 16-byte pieces per row and chunk
  constexpr int RPI = 64 / CPR;               // rows per copy instruction
  constexpr int SROWS = BM + BN;
  constexpr int SBYTES = SROWS * BK * 2;
  constexpr int NI = SROWS / RPI / NW;        // copy instructions per wave per stage
  static_assert(SROWS % (RPI * NW) == 0 && BM % (RPI * NW) == 0, "copy split");
  constexpr int NIA = BM / RPI / NW;          // ... of which activation rows
  extern __shared__ __align__(16) uint8_t smem[];
  const uint4 *ring = reinterpret_cast<const uint4 *>(smem);
  const uint32_t ring_lds = lds_addr(smem);
  const int ntm = (a.R + BM - 1) / BM, ntn = (a.N + BN - 1) / BN;
  const int total = ntm * ntn;
  // tasks in XCD-contiguous runs (workgroup i runs on XCD i mod 8): the row
  // tiles of one weight tile run side by side on one XCD and share its L2
  const int per = (total + 7) / 8;
  const int task = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (task >= total) return;
  const int m0 = (task % ntm) * BM, n0 = (task / ntm) * BN;
  const int R = a.Rdev ? min(*a.Rdev, a.R) : a.R;   // rows past the device count: no work
  if (m0 >= R) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 15, g = lane >> 4;
  const int wm = (wave % WM) * (BM / WM), wn = (wave / WM) * (BN / WN);
  const uint16_t *X = static_cast<const uint16_t *>(a.X);
  const uint16_t *W = static_cast<const uint16_t *>(a.W);
  const int nk = a.Kd / BK, nkw = (a.kw ? a.kw : a.Kd) / BK;
  auto sw = [](int q) { return q & 7; };
  // copy instruction j = wave + NW i of a stage fills stage rows RPI j ..
  // RPI j + RPI - 1 (activation rows first): lane l -> row RPI j + l / CPR,
  // position l % CPR
  const uint16_t *src[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int srow = RPI * (wave + NW * i) + lane / CPR, pc = (lane % CPR) ^ sw(srow);
    if (i < NIA) {
      const int xr = min(m0 + srow, R - 1);
      src[i] = X + (size_t)(a.xidx ? a.xidx[xr] : xr) * a.ldx + 8 * pc;
    } else {
      src[i] = W + (size_t)min(n0 + srow - BM, a.N - 1) * a.ldw + 8 * pc;
    }
  }
  // chunk kc goes to stage kc % STAGES; past the last chunk a step re-issues
  // the last one (read by nobody), so every wait has the same count
  auto issue = [&](int kc) {
    const uint32_t dst = ring_lds + (uint32_t)((kc % STAGES) * SBYTES);
    const int kk = min(kc, nk - 1), kkw = kk % nkw;
#pragma unroll
    for (int i = 0; i < NI; ++i)
      lds_copy16(src[i] + BK * (i < NIA ? kk : kkw), dst + (uint32_t)((wave + NW * i) * 1024));
  };
  const int hl = sw(lr);   // rows of a fragment read are 16-aligned: sw(row) = sw(lr)
  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto epilogue = [&]() {
    // lane holds Y[activation row 4 g + t][output lr] of tile (i, j)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int n = n0 + wn + j * 16 + lr;
      if (n >= a.N) continue;
      const float bv = (a.bias && n >= a.bias_n0) ? a.bias[n - a.bias_n0] : 0.f;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int row = m0 + wm + i * 16 + 4 * g + t;
          if (row >= R) continue;
          float v = acc[i][j][t] + bv;
          if (a.addend && n < a.add_n)
            v += a.addend[(size_t)((row / a.adiv) * a.amul + a.aoff) * a.lda + n];
          a.Y[(size_t)row * a.ldy + n] = v;
        }
    }
  };
#pragma unroll
  for (int kc = 0; kc < STAGES - 1; ++kc) issue(kc);
  for (int kc = 0; kc < nk; ++kc) {
    // chunk kc has landed (this wave's copies; the next STAGES - 2 may
    // fly); after the barrier every wave's copies are visible and the
    // stage of chunk kc - 1 is free
    wait_vm<(STAGES - 2) * NI>();
    bare_barrier();
    issue(kc + STAGES - 1);
    // (fragments of the next chunk double-buffered and read while this
    // chunk's MFMAs run measured slower for the stress state product, 58
    // against 55 us)
    const uint4 *st = ring + (kc % STAGES) * (SBYTES / 16);
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      const int pc = (4 * ks + g) ^ hl;
      uint4 fa[TM], fb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) fa[i] = st[(wm + 16 * i + lr) * CPR + pc];
#pragma unroll
      for (int j = 0; j < TN; ++j) fb[j] = st[(BM + wn + 16 * j + lr) * CPR + pc];
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = sk_mfma(fa[i], fb[j], acc[i][j]);
    }
  }
  wait_vm<0>();   // no copy outlives the workgroup
  epilogue();
}

// The LM-head product (rows of H against the vocabulary rows of W_lm, no
// gather, no planes): the same tiles with a ring of its own per operand,
// 2 stages for the hidden rows (L2 hits) and SB for the weight rows, which
// stream from HBM, so SB - 1 chunks of them are in flight (the shared ring
// held 2, and the streamed chunks' latency set the pace).  At step kc the
// copies of hidden-row chunk kc + 1 and weight chunk kc + SB - 1 are issued;
// the wait before it leaves only the previous step's weight copies in
// flight, which makes both of chunk kc's copies land.
template <int BM, int BN, int WM, int WN, int SB>
__global__ __launch_bounds__(WM * WN * 64) void k_mm_lm(GemmArgs a) {
  constexpr int SA = 2;
  constexpr int NW = WM * WN;
  constexpr int TM = BM / WM / 16, TN = BN / WN / 16;
  constexpr int BK = 64, CPR = 8, RPI = 8;
  constexpr int ABYTES = BM * BK * 2, BBYTES = BN * BK * 2;
  constexpr int NA = BM / RPI / NW, NB = BN / RPI / NW;   // copy instructions per wave and chunk
  static_assert(BM % (RPI * NW) == 0 && BN % (RPI * NW) == 0 && SB >= 3, "copy split");
  extern __shared__ __align__(16) uint8_t smem[];
  const uint4 *ringA = reinterpret_cast<const uint4 *>(smem);
  const uint4 *ringB = reinterpret_cast<const uint4 *>(smem + SA * ABYTES);
  const uint32_t ldsA = lds_addr(smem), ldsB = ldsA + SA * ABYTES;
  const int ntm = (a.R + BM - 1) / BM, ntn = (a.N + BN - 1) / BN;
  const int total = ntm * ntn;
  const int per = (total + 7) / 8;
  const int task = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (task >= total) return;
  const int m0 = (task % ntm) * BM, n0 = (task / ntm) * BN;
  const int R = a.R;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 15, g = lane >> 4;
  const int wm = (wave % WM) * (BM / WM), wn = (wave / WM) * (BN / WN);
  const uint16_t *X = static_cast<const uint16_t *>(a.X);
  const uint16_t *W = static_cast<const uint16_t *>(a.W);
  const int nk = a.Kd / BK;
  // copy instruction i of an operand's chunk fills its rows RPI (wave + NW i)
  // .. + RPI - 1: lane l -> row + l / 8, position l % 8 (chunk c of row q
  // at position c ^ (q & 7))
  const uint16_t *srcA[NA], *srcB[NB];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int row = RPI * (wave + NW * i) + lane / CPR, pc = (lane % CPR) ^ (row & 7);
    srcA[i] = X + (size_t)min(m0 + row, R - 1) * a.ldx + 8 * pc;
  }
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int row = RPI * (wave + NW * i) + lane / CPR, pc = (lane % CPR) ^ (row & 7);
    srcB[i] = W + (size_t)min(n0 + row, a.N - 1) * a.ldw + 8 * pc;
  }
  // past the last chunk a step re-issues the last one (read by nobody), so
  // every wait has the same count
  auto issueA = [&](int kc) {
    const uint32_t dst = ldsA + (uint32_t)((kc % SA) * ABYTES);
    const int kk = min(kc, nk - 1);
#pragma unroll
    for (int i = 0; i < NA; ++i) lds_copy16(srcA[i] + BK * kk, dst + (uint32_t)((wave + NW * i) * 1024));
  };
  auto issueB = [&](int kc) {
    const uint32_t dst = ldsB + (uint32_t)((kc % SB) * BBYTES);
    const int kk = min(kc, nk - 1);
#pragma unroll
    for (int i = 0; i < NB; ++i) lds_copy16(srcB[i] + BK * kk, dst + (uint32_t)((wave + NW * i) * 1024));
  };
  const int hl = lr & 7;
  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  issueA(0);
#pragma unroll
  for (int kc = 0; kc < SB - 1; ++kc) issueB(kc);
  for (int kc = 0; kc < nk; ++kc) {
    // chunk kc of both operands has landed (this wave's copies): at step 0
    // the weight chunks 1 .. SB - 2 may fly, later the previous step's
    // weight chunk only
    if (kc == 0) wait_vm<(SB - 2) * NB>();
    else wait_vm<NB>();
    bare_barrier();
    issueA(kc + 1);
    issueB(kc + SB - 1);
    const uint4 *sa = ringA + (kc % SA) * (ABYTES / 16), *sb = ringB + (kc % SB) * (BBYTES / 16);
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      const int pc = (4 * ks + g) ^ hl;
      uint4 fa[TM], fb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) fa[i] = sa[(wm + 16 * i + lr) * CPR + pc];
#pragma unroll
      for (int j = 0; j < TN; ++j) fb[j] = sb[(wn + 16 * j + lr) * CPR + pc];
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = sk_mfma(fa[i], fb[j], acc[i][j]);
    }
  }
  wait_vm<0>();   // no copy outlives the workgroup
  // lane holds Y[row 4 g + t][output lr] of tile (i, j)
  uint32_t gm[TM][4];   // the lane's largest ordered output per row
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int t = 0; t < 4; ++t) gm[i][t] = 0u;
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int n = n0 + wn + j * 16 + lr;
    if (n >= a.N) continue;
    const float bv = a.bias ? a.bias[n] : 0.f;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int row = m0 + wm + i * 16 + 4 * g + t;
        const float y = acc[i][j][t] + bv;
        gm[i][t] = max(gm[i][t], f32_ord(y));
        if (row < R) a.Y[(size_t)row * a.ldy + n] = y;
      }
  }
  // group maxima: the wave's BN / WN columns, over the 16 lanes of a row
  // (lanes past the last column hold 0, below every ordered value)
  if (a.gmax && n0 + wn < a.N) {
    const int gi = (n0 + wn) / (BN / WN);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        uint32_t v = gm[i][t];
        v = max(v, xchg_u32<1>(v));
        v = max(v, xchg_u32<2>(v));
        v = max(v, xchg_u32<4>(v));
        v = max(v, xchg_u32<8>(v));
        const int row = m0 + wm + i * 16 + 4 * g + t;
        if (lr == 0 && row < R) a.gmax[(size_t)row * a.ldg + gi] = v;
      }
  }
}
template <int BM, int BN, int SB>
static constexpr size_t mm_lm_smem() { return (size_t)2 * BM * 128 + (size_t)SB * BN * 128; }
#define MM_LM_CONFIGS(X) X(128, 256, 2, 4, 4) X(128, 320, 2, 4, 3) X(256, 256, 2, 4, 3)

hipError_t launch_mm_lm(const GemmArgs &a, int bm, int bn, hipStream_t st, hipEvent_t ev0,
                        hipEvent_t ev1) {
  const int total = ((a.R + bm - 1) / bm) * ((a.N + bn - 1) / bn);
  const dim3 grid(8 * ((total + 7) / 8));
#define MM_LM_LAUNCH(BM_, BN_, WM_, WN_, SB_)                                                   \
  if (bm == BM_ && bn == BN_) {                                                                 \
    hipExtLaunchKernelGGL((k_mm_lm<BM_, BN_, WM_, WN_, SB_>), grid, dim3(WM_ * WN_ * 64),       \
                          (uint32_t)mm_lm_smem<BM_, BN_, SB_>(), st, ev0, ev1, 0u, a);          \
    return hipGetLastError();                                                                   \
  }
  MM_LM_CONFIGS(MM_LM_LAUNCH)
#undef MM_LM_LAUNCH
  return hipErrorInvalidValue;
}

template <int BM, int BN, int STAGES>
static constexpr size_t mm_smem() { return (size_t)STAGES * (BM + BN) * 128; }

// 256 x 128 tiles (sixteen waves of 32 x 64, one workgroup per CU) when they
// still make 256 or more tiles, else 128 x 128 (eight waves of 32 x 64, two
// workgroups per CU).  Four waves per SIMD cover each other's waits: the
// stress state product, 416 tiles of 128 x 128, took 53 us with four waves of
// 64 x 64 and 40 us with eight of 32 x 64; the stress distinct tokens'
// projections (256 x 128) 82 us with eight waves of 64 x 64, 75 with sixteen.
void mm_tile(int R, int N, int *bm, int *bn) {
  const long long big = (long long)((R + 255) / 256) * ((N + 127) / 128);
  *bm = big >= 256 ? 256 : 128;
  *bn = 128;
}

bool mm_ok(const GemmArgs &a) {
  const int kw = a.kw ? a.kw : a.Kd;
  auto al16 = [](const void *p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; };
  return a.wtype == WT_BF16 && a.xtype == WT_BF16 && a.Kd % 64 == 0 && kw % 64 == 0 &&
         a.Kd % kw == 0 && a.ldx % 8 == 0 && a.ldw % 8 == 0 && al16(a.X) && al16(a.W);
}

// configurations: (BM, BN, WM, WN)
// 128 x 128 tiles: a three-stage ring (96 KiB, one workgroup per CU) when
// the tiles fit one per CU (wide candidates' projections 54 -> 47 us), else
// two stages, so that two workgroups share a CU (stress state products: 975
// against 1,203 us for the depth loop with three)
#define MM_CONFIGS(X) X(256, 128, 8, 2, 3) X(128, 128, 4, 2, 2) X(128, 128, 4, 2, 3) X(128, 64, 4, 1, 4)

hipError_t launch_mm(const GemmArgs &a, int bm, int bn, hipStream_t st, hipEvent_t ev0,
                     hipEvent_t ev1) {
  const int total = ((a.R + bm - 1) / bm) * ((a.N + bn - 1) / bn);
  const dim3 grid(8 * ((total + 7) / 8));
  const int stages = (bm == 128 && bn == 128) ? (total <= 256 ? 3 : 2) : 0;
#define MM_LAUNCH(BM_, BN_, WM_, WN_, S_)                                                       \
  if (bm == BM_ && bn == BN_ && (stages == 0 || stages == S_)) {                                \
    hipExtLaunchKernelGGL((k_mm<BM_, BN_, WM_, WN_, S_>), grid, dim3(WM_ * WN_ * 64),           \
                          (uint32_t)mm_smem<BM_, BN_, S_>(), st, ev0, ev1, 0u, a);              \
    return hipGetLastError();                                                                   \
  }
  MM_CONFIGS(MM_LAUNCH)
#undef MM_LAUNCH
  return hipErrorInvalidValue;
}

static hipError_t mm_prepare() {
  hipError_t e = hipSuccess;
#define MM_SET(BM_, BN_, WM_, WN_, S_)                                                          \
  if (e == hipSuccess)                                                                          \
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_mm<BM_, BN_, WM_, WN_, S_>),      \
                            hipFuncAttributeMaxDynamicSharedMemorySize,                         \
                            (int)mm_smem<BM_, BN_, S_>());
  MM_CONFIGS(MM_SET)
#undef MM_SET
#define MM_LM_SET(BM_, BN_, WM_, WN_, SB_)                                                      \
  if (e == hipSuccess)                                                                          \
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_mm_lm<BM_, BN_, WM_, WN_, SB_>),  \
                            hipFuncAttributeMaxDynamicSharedMemorySize,                         \
                            (int)mm_lm_smem<BM_, BN_, SB_>());
  MM_LM_CONFIGS(MM_LM_SET)
#undef MM_LM_SET
  return e;
}

// Many activation rows (256 or more) and bf16 operands: the tiled product
// (k_mm), at least 64 tiles of 128 x 128
bool gemm_tiled_ok(const GemmArgs &a) {
  const int tiles = ((a.R + 127) / 128) * ((a.N + 127) / 128);
  return a.R >= 256 && tiles >= 64 && a.Kd % 64 == 0 && mm_ok(a);
}

hipError_t gemm_prepare() { return mm_prepare(); }

static int skinny_terms(const GemmArgs &a) {
  return (a.xtype == WT_F32 && !a.xround) ? 3 : 1;
}

bool skinny_ok(const GemmArgs &a) {
  if (a.wtype != WT_BF16 || a.Kd % 32 || a.ldw % 8 || reinterpret_cast<uintptr_t>(a.W) % 16)
    return false;
  if (reinterpret_cast<uintptr_t>(a.X) % 16) return false;
  if (a.xtype == WT_BF16) return a.ldx % 8 == 0 && a.Kd <= 32 * SK_WAVES * SK_KSW_B;
  return a.ldx % 4 == 0 && a.Kd <= 32 * SK_WAVES * SK_KSW_F;
}



bool gemm_rdev_ok(const GemmArgs &a) {
  return (a.R <= 8192 && skinny_ok(a)) || gemm_tiled_ok(a);
}

hipError_t launch_gemm(const GemmArgs &a, hipStream_t st) {
  if (a.R <= 0 || a.N <= 0) return hipSuccess;
  // a device row count up to 8192 rows: the contraction-split kernel, whose
  // workgroups past the count leave at once, keeps every wave busy; with a
  // long contraction (2048 or more) its activation re-reads (once per 16
  // outputs) cost more, and 128 x 64 tiles take over (few active row tiles:
  // the device count is often far below the bound, so narrow column tiles
  // give more active workgroups)
  const bool skinny_first = a.Rdev && a.R <= 8192 && skinny_ok(a) && a.Kd < 2048;
  if (!skinny_first && gemm_tiled_ok(a)) {
    int bm = 128, bn = 64;
    if (!(a.Rdev && a.R <= 8192)) mm_tile(a.R, a.N, &bm, &bn);
    return launch_mm(a, bm, bn, st, nullptr, nullptr);
  }
  if (a.kw && a.kw != a.Kd) return hipErrorInvalidValue;   // planes need the tiled kernel
  if (a.Rdev && !skinny_ok(a)) return hipErrorInvalidValue;  // device row counts need MFMA kernels
  if (skinny_ok(a)) {
    const int terms = skinny_terms(a);
    // split fp32 activations, a short contraction and many outputs: four
    // column tiles per workgroup (each split activation fragment feeds four
    // weight fragments) when that still makes 128 or more workgroups
    const int nrb0 = (a.R + 15) / 16, ncol4 = (a.N + 63) / 64;
    if (a.xtype == WT_F32 && terms == 3 && a.Kd <= 32 * SK_WAVES * 4 &&
        ncol4 * ((nrb0 + 1) / 2) >= 128) {
      hipLaunchKernelGGL((k_skinny_bf16<3, float, 4, 4, 2>), dim3(ncol4, (nrb0 + 1) / 2),
                         dim3(SK_WAVES * 64), 0, st, a, 2);
      return hipGetLastError();
    }
    // row blocks per workgroup: enough workgroups to fill the chip (about
    // 1024) before a weight tile is reused for more rows
    const int ncol = (a.N + 15) / 16, nrb = (a.R + 15) / 16;
    const int groups = std::max(1, std::min(nrb, 1024 / ncol));
    const int RB = std::min(SK_RB, (nrb + groups - 1) / groups);
    dim3 grid(ncol, (nrb + RB - 1) / RB);
    // register arrays sized to the contraction: short ones leave room for a
    // second workgroup per CU
    const bool shortk = a.Kd <= 32 * SK_WAVES * (a.xtype == WT_BF16 ? 8 : 4);
    const dim3 blk(SK_WAVES * 64);
    if (a.xtype == WT_BF16) {
      if (shortk) hipLaunchKernelGGL((k_skinny_bf16<1, uint16_t, 8>), grid, blk, 0, st, a, RB);
      else hipLaunchKernelGGL((k_skinny_bf16<1, uint16_t, SK_KSW_B>), grid, blk, 0, st, a, RB);
    } else if (terms == 1) {
      if (shortk) hipLaunchKernelGGL((k_skinny_bf16<1, float, 4>), grid, blk, 0, st, a, RB);
      else hipLaunchKernelGGL((k_skinny_bf16<1, float, SK_KSW_F>), grid, blk, 0, st, a, RB);
    } else {
      if (shortk) hipLaunchKernelGGL((k_skinny_bf16<3, float, 4>), grid, blk, 0, st, a, RB);
      else hipLaunchKernelGGL((k_skinny_bf16<3, float, SK_KSW_F>), grid, blk, 0, st, a, RB);
    }
    return hipGetLastError();
  }
  dim3 grid((a.N + GT - 1) / GT, (a.R + GT - 1) / GT);
  if (a.xtype == WT_F32 && a.wtype == WT_F32)
    hipLaunchKernelGGL((k_gemm_xwT<float, float>), grid, dim3(256), 0, st, a);
  else if (a.xtype == WT_F32 && a.wtype == WT_BF16)
    hipLaunchKernelGGL((k_gemm_xwT<float, uint16_t>), grid, dim3(256), 0, st, a);
  else if (a.xtype == WT_BF16 && a.wtype == WT_BF16)
    hipLaunchKernelGGL((k_gemm_xwT<uint16_t, uint16_t>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((k_gemm_xwT<uint16_t, float>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

// GRU cell, PyTorch GRUCell form with gate blocks (r, z, n):
//   r = sig(a_r + c_r), z = sig(a_z + c_z), n = tanh(a_n + r * c_n),
//   h' = (1 - z) n + z h
// where a = W_ih x + b_ih and c = W_hh h + b_hh.
__global__ __launch_bounds__(256) void k_gru_combine(int R, int s, const float *__restrict__ gi,
                                                     const int32_t *__restrict__ gidx,
                                                     const int32_t *__restrict__ gmap,
                                                     const float *__restrict__ gh, int ldgh,
                                                     const float *__restrict__ b_hh,
                                                     const float *__restrict__ Sprev,
                                                     const int32_t *__restrict__ pidx,
                                                     float *__restrict__ Snew,
                                                     uint16_t *__restrict__ S3) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= R * s) return;
  const int i = idx / s, j = idx - i * s;
  int gr = gidx ? gidx[i] : i;
  if (gmap) gr = gmap[gr];
  const float *a = gi + (size_t)gr * 3 * s;
  float cr, cz, cn, h;
  if (gh) {
    const int pr = pidx ? pidx[i] : i;   // the parent's row: its state and state part
    const float *c = gh + (size_t)pr * ldgh;
    cr = c[j]; cz = c[s + j]; cn = c[2 * s + j];
    h = Sprev[(size_t)pr * s + j];
  } else {
    cr = b_hh ? b_hh[j] : 0.f;
    cz = b_hh ? b_hh[s + j] : 0.f;
    cn = b_hh ? b_hh[2 * s + j] : 0.f;
    h = 0.f;
  }
  const float r = 1.f / (1.f + expf(-(a[j] + cr)));
  const float z = 1.f / (1.f + expf(-(a[s + j] + cz)));
  const float n = tanhf(a[2 * s + j] + r * cn);
  const float hn = (1.f - z) * n + z * h;
  Snew[(size_t)i * s + j] = hn;
  if (S3) {
    const uint16_t t0 = f32_to_bf16_rne(hn);
    const float r1 = hn - bf16_bits_to_f32(t0);
    const uint16_t t1 = f32_to_bf16_rne(r1);
    uint16_t *o = S3 + (size_t)i * STATE_PLANES * s + j;
    o[0] = t0;
    o[s] = t1;
  }
}

hipError_t launch_gru_combine(int R, int s, const float *gi, const int32_t *gidx,
                              const int32_t *gmap, const float *gh, int ldgh, const float *b_hh,
                              const float *Sprev, const int32_t *pidx, float *Snew, uint16_t *S3,
                              hipStream_t st) {
  const int n = R * s;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_gru_combine, dim3((n + 255) / 256), dim3(256), 0, st, R, s, gi, gidx, gmap,
                     gh, ldgh, b_hh, Sprev, pidx, Snew, S3);
  return hipGetLastError();
}

// Wcat rows n < r: W1[n][d .. d + s); rows r + m: W_hh[m] (made once per
// context, so that the low-rank head's state part and the GRU's state
// projection of the same branches are one product)
template <typename T>
__global__ void k_concat_state_weights(const T *__restrict__ W1, const T *__restrict__ W_hh,
                                       int r, int s, int d, T *__restrict__ Wcat) {
  const size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  if (i >= (size_t)(r + 3 * s) * s) return;
  const int n = (int)(i / s), k = (int)(i - (size_t)n * s);
  Wcat[i] = n < r ? W1[(size_t)n * (d + s) + d + k] : W_hh[(size_t)(n - r) * s + k];
}

hipError_t launch_concat_state_weights(const void *W1, const void *W_hh, int r, int s, int d,
                                       int wtype, void *Wcat, hipStream_t st) {
  const size_t n = (size_t)(r + 3 * s) * s;
  const dim3 grid((unsigned)((n + 255) / 256));
  if (wtype == WT_BF16)
    hipLaunchKernelGGL(k_concat_state_weights<uint16_t>, grid, dim3(256), 0, st,
                       static_cast<const uint16_t *>(W1), static_cast<const uint16_t *>(W_hh), r,
                       s, d, static_cast<uint16_t *>(Wcat));
  else
    hipLaunchKernelGGL(k_concat_state_weights<float>, grid, dim3(256), 0, st,
                       static_cast<const float *>(W1), static_cast<const float *>(W_hh), r, s, d,
                       static_cast<float *>(Wcat));
  return hipGetLastError();
}

// ---- distinct tokens (the GRU input projection depends on the token only)
// first[tok] holds (epoch << 32) | (2^32 - 1 - row) for the token's first row
// of the current round (a 64-bit maximum, so entries of earlier rounds lose
// and the table never needs clearing); row i represents its token when it is
// that first row.  Representatives get consecutive positions in row order.
constexpr int TD_B = 256;   // rows per block of the scans

__device__ __forceinline__ uint64_t td_tag(uint32_t epoch, int row) {
  return ((uint64_t)epoch << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)row);
}

__global__ void k_token_mark(int n, const int32_t *__restrict__ tok, unsigned long long *first,
                             uint32_t epoch) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) atomicMax(first + tok[i], (unsigned long long)td_tag(epoch, i));
}

// positions of the representatives inside each block of TD_B rows, and the
// block totals
__global__ __launch_bounds__(TD_B) void k_token_scan(int n, const int32_t *__restrict__ tok,
                                                     const unsigned long long *__restrict__ first,
                                                     uint32_t epoch, int32_t *lpos,
                                                     int32_t *btot) {
  __shared__ int sc[TD_B];
  const int tid = threadIdx.x, i = blockIdx.x * TD_B + tid;
  const int f = (i < n && first[tok[i]] == td_tag(epoch, i)) ? 1 : 0;
  sc[tid] = f;
  __syncthreads();
  for (int off = 1; off < TD_B; off <<= 1) {   // inclusive scan (Hillis-Steele)
    const int v = tid >= off ? sc[tid - off] : 0;
    __syncthreads();
    sc[tid] += v;
    __syncthreads();
  }
  if (i < n) lpos[i] = f ? sc[tid] - 1 : -1;
  if (tid == TD_B - 1) btot[blockIdx.x] = sc[tid];
}

// exclusive scan of the block totals (one workgroup, nb <= 1024 blocks) and
// the number of distinct tokens
__global__ __launch_bounds__(1024) void k_token_bases(int nb, int32_t *btot, int32_t *count) {
  __shared__ int sc[1024];
  const int tid = threadIdx.x;
  const int v0 = tid < nb ? btot[tid] : 0;
  sc[tid] = v0;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = tid >= off ? sc[tid - off] : 0;
    __syncthreads();
    sc[tid] += v;
    __syncthreads();
  }
  if (tid < nb) btot[tid] = sc[tid] - v0;
  if (tid == 1023) *count = sc[tid];
}

__global__ void k_token_place(int n, const int32_t *__restrict__ tok,
                              const int32_t *__restrict__ lpos, const int32_t *__restrict__ bbase,
                              int32_t *cidx, int32_t *uniq) {
  const int i = blockIdx.x * TD_B + threadIdx.x;
  if (i >= n || lpos[i] < 0) return;
  const int pos = bbase[blockIdx.x] + lpos[i];
  cidx[i] = pos;
  uniq[pos] = tok[i];
}

__global__ void k_token_map(int n, const int32_t *__restrict__ tok,
                            const unsigned long long *__restrict__ first,
                            const int32_t *__restrict__ cidx, int32_t *rowmap) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int rep = (int)(0xFFFFFFFFu - (uint32_t)first[tok[i]]);
  rowmap[i] = cidx[rep];
}

// The rest in one workgroup (TT_THREADS threads, each a run of up to TT_PER
// consecutive rows, so that one block scan of the run counts orders the
// representatives by row): positions, the distinct tokens, their count, and
// every row's position through its representative.  Each thread's loads are
// issued together (unrolled over the run); the positions this workgroup
// stored are read back with device-coherent loads.
constexpr int TT_THREADS = 1024, TT_PER = 16;
__global__ __launch_bounds__(TT_THREADS) void k_token_tables(int n, const int32_t *__restrict__ tok,
                                                             const unsigned long long *__restrict__ first,
                                                             uint32_t epoch, int32_t *cidx,
                                                             int32_t *uniq, int32_t *rowmap,
                                                             int32_t *count) {
  __shared__ int wtot[TT_THREADS / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per = (n + TT_THREADS - 1) / TT_THREADS;   // <= TT_PER (checked by the host)
  const int i0 = min(n, tid * per), cnt = min(n, i0 + per) - i0;
  int tk[TT_PER];
  uint64_t fv[TT_PER];
#pragma unroll
  for (int u = 0; u < TT_PER; ++u) tk[u] = u < cnt ? tok[i0 + u] : 0;
#pragma unroll
  for (int u = 0; u < TT_PER; ++u) fv[u] = u < cnt ? first[tk[u]] : 0ull;
  uint32_t repm = 0;   // bit u: row i0 + u represents its token
  int c = 0;
#pragma unroll
  for (int u = 0; u < TT_PER; ++u)
    if (u < cnt && fv[u] == td_tag(epoch, i0 + u)) { repm |= 1u << u; ++c; }
  // exclusive prefix of the run counts over the workgroup
  const int incl = wave_scan_add(c);
  if (lane == 63) wtot[wave] = incl;
  __syncthreads();
  int base = incl - c, total = 0;
  for (int w = 0; w < TT_THREADS / 64; ++w) {
    const int t = wtot[w];
    base += w < wave ? t : 0;
    total += t;
  }
#pragma unroll
  for (int u = 0; u < TT_PER; ++u)
    if (repm & (1u << u)) {
      cidx[i0 + u] = base;
      uniq[base] = tk[u];
      ++base;
    }
  if (tid == 0) *count = total;
  __syncthreads();
  int pos[TT_PER];
#pragma unroll
  for (int u = 0; u < TT_PER; ++u)
    pos[u] = u < cnt ? __hip_atomic_load(cidx + (int)(0xFFFFFFFFu - (uint32_t)fv[u]), __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT)
                     : 0;
#pragma unroll
  for (int u = 0; u < TT_PER; ++u)
    if (u < cnt) rowmap[i0 + u] = pos[u];
}

__global__ void k_zero_u64(unsigned long long *p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0ull;
}

hipError_t launch_token_dedupe(int n, const int32_t *tok, void *first, int V, uint32_t epoch,
                               int32_t *lpos, int32_t *btot, int32_t *cidx, int32_t *uniq,
                               int32_t *rowmap, int32_t *count, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const int nb = (n + TD_B - 1) / TD_B;
  if (nb > 1024) return hipErrorInvalidValue;
  auto *f = static_cast<unsigned long long *>(first);
  // epoch 1 starts a new cycle of the 32-bit epoch: tags left by the last
  // cycle would outrank it, so the table is cleared first (a kernel, so the
  // round stays free of memset nodes under graph capture)
  if (epoch == 1u)
    hipLaunchKernelGGL(k_zero_u64, dim3((V + 255) / 256), dim3(256), 0, st, f, V);
  hipLaunchKernelGGL(k_token_mark, dim3(nb), dim3(TD_B), 0, st, n, tok, f, epoch);
  // up to TT_PER rows per thread: the one-workgroup tables (one launch
  // instead of four); more: block scans over many workgroups
  if (n <= TT_PER * TT_THREADS) {
    hipLaunchKernelGGL(k_token_tables, dim3(1), dim3(TT_THREADS), 0, st, n, tok, f, epoch, cidx,
                       uniq, rowmap, count);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_token_scan, dim3(nb), dim3(TD_B), 0, st, n, tok, f, epoch, lpos, btot);
  hipLaunchKernelGGL(k_token_bases, dim3(1), dim3(1024), 0, st, nb, btot, count);
  hipLaunchKernelGGL(k_token_place, dim3(nb), dim3(TD_B), 0, st, n, tok, lpos, btot, cidx, uniq);
  hipLaunchKernelGGL(k_token_map, dim3(nb), dim3(TD_B), 0, st, n, tok, f, cidx, rowmap);
  return hipGetLastError();
}

}  // namespace dtree
