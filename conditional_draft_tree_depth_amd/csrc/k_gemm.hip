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

hipError_t launch_gemm(const GemmArgs &a, hipStream_t st) {
  if (a.R <= 0 || a.N <= 0) return hipSuccess;
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
