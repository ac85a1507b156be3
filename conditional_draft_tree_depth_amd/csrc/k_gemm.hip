// Row-gathered products with fp32 activations and stored (bf16/fp32) weights,
// and the GRU cell.
//
// Used for the path-independent projection uH = W1[:, :d] Hq, the per-branch
// part W1[:, d:] S of the low-rank head ("Resumen Técnico: Domino",
// Methodology 2: [H_i ; S_{i-1}] is projected to rank r), and the GRU input
// and state projections.  Activations stay fp32 (the GRU state is never
// rounded to bf16); bf16 weights are widened exactly to fp32; accumulation
// is fp32.  Tiles: 64 rows x 64 outputs per 256-thread workgroup, 16-wide k
// chunks staged in LDS.
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
      if (a.bias) v += a.bias[n];
      if (add) v += add[n];
      a.Y[(size_t)row * a.ldy + n] = v;
    }
  }
}

// Skinny product on MFMA: at most 16 activation rows per workgroup (rows of
// the B operand, staged in LDS as bf16), bf16 weight rows streamed from
// memory as the A operand, 16 weight rows per wave, fp32 accumulation.
// fp32 activations that must not be rounded (the GRU state) are split
// exactly into three bf16 terms x = hi + mid + lo (each term is the bf16
// rounding of what the previous ones left, so the remainder is below
// 2^-24 |x|); every term is multiplied by the same weight fragment.
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
constexpr int SK_WAVES = 4;

__device__ __forceinline__ bf16x8 sk_bf(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

template <int TERMS, typename XT>
__global__ __launch_bounds__(SK_WAVES * 64) void k_skinny_bf16(GemmArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int KS = a.Kd + 8;
  uint16_t *Xs = reinterpret_cast<uint16_t *>(smem);   // [TERMS][16][KS]
  const XT *X = static_cast<const XT *>(a.X);
  const int r0 = blockIdx.x * 16;
  const int nr = min(16, a.R - r0);
  for (int i = threadIdx.x; i < 16 * a.Kd; i += blockDim.x) {
    const int rr = i / a.Kd, k = i - rr * a.Kd;
    uint16_t t0 = 0, t1 = 0, t2 = 0;
    if (rr < nr) {
      const size_t xi = (size_t)(a.xidx ? a.xidx[r0 + rr] : r0 + rr) * a.ldx + k;
      if constexpr (sizeof(XT) == 2) {
        t0 = X[xi];
      } else {
        const float x = X[xi];
        t0 = f32_to_bf16_rne(x);
        if constexpr (TERMS == 3) {
          const float r1 = x - bf16_bits_to_f32(t0);
          t1 = f32_to_bf16_rne(r1);
          t2 = f32_to_bf16_rne(r1 - bf16_bits_to_f32(t1));
        }
      }
    }
    Xs[rr * KS + k] = t0;
    if constexpr (TERMS == 3) {
      Xs[(16 + rr) * KS + k] = t1;
      Xs[(32 + rr) * KS + k] = t2;
    }
  }
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lr = lane & 15, g = lane >> 4;
  const int tile = blockIdx.y * SK_WAVES + wave;
  if (tile * 16 >= a.N) return;
  const int n = min(tile * 16 + lr, a.N - 1);
  const uint16_t *Wt = static_cast<const uint16_t *>(a.W);
  const uint4 *pw = reinterpret_cast<const uint4 *>(Wt + (size_t)n * a.ldw + g * 32);
  const uint16_t *hp = Xs + lr * KS + g * 32;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  uint4 cw[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) cw[j] = pw[j];
  for (int kc = 0; kc < a.Kd; kc += 128) {
    uint4 nw[4];
    if (kc + 128 < a.Kd) {
#pragma unroll
      for (int j = 0; j < 4; ++j) nw[j] = pw[(kc + 128) / 8 + j];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int t = 0; t < TERMS; ++t) {
        const uint4 xv = *reinterpret_cast<const uint4 *>(hp + t * 16 * KS + kc + 8 * j);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sk_bf(cw[j]), sk_bf(xv), acc, 0, 0, 0);
      }
    }
    if (kc + 128 < a.Kd) {
#pragma unroll
      for (int j = 0; j < 4; ++j) cw[j] = nw[j];
    }
  }
  if (lr >= nr) return;
  const int row = r0 + lr;
  const float *add = a.addend ? a.addend + (size_t)((row / a.adiv) * a.amul + a.aoff) * a.lda : nullptr;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int nn = tile * 16 + 4 * g + t;
    if (nn >= a.N) continue;
    float v = acc[t];
    if (a.bias) v += a.bias[nn];
    if (add) v += add[nn];
    a.Y[(size_t)row * a.ldy + nn] = v;
  }
}

static int skinny_terms(const GemmArgs &a) {
  return (a.xtype == WT_F32 && !a.xround) ? 3 : 1;
}

size_t skinny_smem(int Kd, int terms) { return (size_t)terms * 16 * (Kd + 8) * 2; }

bool skinny_ok(const GemmArgs &a, size_t lds_max) {
  return a.wtype == WT_BF16 && a.Kd % 128 == 0 && a.ldw % 8 == 0 &&
         reinterpret_cast<uintptr_t>(a.W) % 16 == 0 && a.R <= 64 &&
         skinny_smem(a.Kd, skinny_terms(a)) <= lds_max;
}

hipError_t skinny_prepare(size_t lds_max) {
  const void *fns[] = {reinterpret_cast<const void *>(&k_skinny_bf16<1, uint16_t>),
                       reinterpret_cast<const void *>(&k_skinny_bf16<1, float>),
                       reinterpret_cast<const void *>(&k_skinny_bf16<3, float>)};
  for (const void *f : fns) {
    hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_max);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

static size_t g_lds_max = 65536;
void gemm_set_lds_max(size_t b) { g_lds_max = b; }

hipError_t launch_gemm(const GemmArgs &a, hipStream_t st) {
  if (a.R <= 0 || a.N <= 0) return hipSuccess;
  if (skinny_ok(a, g_lds_max)) {
    const int terms = skinny_terms(a);
    dim3 grid((a.R + 15) / 16, ((a.N + 15) / 16 + SK_WAVES - 1) / SK_WAVES);
    const size_t sm = skinny_smem(a.Kd, terms);
    if (a.xtype == WT_BF16)
      hipLaunchKernelGGL((k_skinny_bf16<1, uint16_t>), grid, dim3(SK_WAVES * 64), sm, st, a);
    else if (terms == 1)
      hipLaunchKernelGGL((k_skinny_bf16<1, float>), grid, dim3(SK_WAVES * 64), sm, st, a);
    else
      hipLaunchKernelGGL((k_skinny_bf16<3, float>), grid, dim3(SK_WAVES * 64), sm, st, a);
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
                                                     const float *__restrict__ gh,
                                                     const float *__restrict__ b_hh,
                                                     const float *__restrict__ Sprev,
                                                     const int32_t *__restrict__ pidx,
                                                     float *__restrict__ Snew) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= R * s) return;
  const int i = idx / s, j = idx - i * s;
  const float *a = gi + (size_t)i * 3 * s;
  float cr, cz, cn, h;
  if (gh) {
    const float *c = gh + (size_t)i * 3 * s;
    cr = c[j]; cz = c[s + j]; cn = c[2 * s + j];
    h = Sprev[(size_t)(pidx ? pidx[i] : i) * s + j];
  } else {
    cr = b_hh ? b_hh[j] : 0.f;
    cz = b_hh ? b_hh[s + j] : 0.f;
    cn = b_hh ? b_hh[2 * s + j] : 0.f;
    h = 0.f;
  }
  const float r = 1.f / (1.f + expf(-(a[j] + cr)));
  const float z = 1.f / (1.f + expf(-(a[s + j] + cz)));
  const float n = tanhf(a[2 * s + j] + r * cn);
  Snew[(size_t)i * s + j] = (1.f - z) * n + z * h;
}

hipError_t launch_gru_combine(int R, int s, const float *gi, const float *gh, const float *b_hh,
                              const float *Sprev, const int32_t *pidx, float *Snew,
                              hipStream_t st) {
  const int n = R * s;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_gru_combine, dim3((n + 255) / 256), dim3(256), 0, st, R, s, gi, gh, b_hh,
                     Sprev, pidx, Snew);
  return hipGetLastError();
}

}  // namespace dtree
