// Tree-attention verification: one layer's attention of the verification
// pass of a draft tree.  Every tree token attends to its request's verified
// prefix and to the tree tokens on its own root-to-node path, itself
// included ("Resumen Técnico: DominoTree", Componentes Principales 5: tree
// attention with an ancestor-only mask; "DARTree: Speculative Diffusion
// Decoding with Autoregressive Draft Trees", Metodología 2, verification).
// The mask is the one the round emits: row = query node, column = key node.
//
// Work decomposition.  The query rows of one request and KV head are the
// (node, query head) pairs that share that KV head (grouped-query
// attention): row r = node * G + g, query head kvh * G + g.  A workgroup
// owns 64 rows and one contiguous key range (a "split") of the request's
// keys; its four waves split every 64-key tile between them (16 keys each),
// so each K/V element is read from LDS exactly once per workgroup and every
// wave runs its own online softmax over its keys; the waves' partial results
// are merged once, at the end.  Splits of one row block are merged by a
// second kernel when there is more than one.
//
// Products on the matrix cores: S^T = K Q^T with v_mfma_f32_16x16x32_bf16
// (A = 16 keys x 32 dims from LDS, B = the wave's query fragments kept in
// registers), then O^T += V^T P^T with v_mfma_f32_16x16x16_bf16 (A = V^T
// from a transposed LDS copy of the tile, B = the softmax weights rounded to
// bf16 straight from the S^T accumulators: lane l holds query l % 16 and
// keys 4 (l / 16) + t, which is exactly the B layout of that instruction).
// Scores are kept in log2 units (scale * log2 e folded in) for exp2.
//
// Keys of a row block: prefix positions are visible to every row; tree key
// j (cache position prefix + j) is visible to node i when mask[i][j] = 1.
// Ancestors precede their descendants in the round's canonical order, so a
// row block whose last node is i_hi never needs tree keys past i_hi.
#include <hip/hip_runtime.h>
#include <cmath>
#include <cstdint>
#include <cstdio>

#include "common.hpp"
#include "kernels.hpp"

namespace dtree {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int TA_THREADS = 256;
constexpr int TA_QB = 64;      // query rows per workgroup
constexpr int TA_KT = 64;      // keys per tile (16 per wave)
constexpr int TA_KPAD = 8;     // bf16 padding of a K row in LDS
constexpr int TA_VROW = TA_KT + 4;   // bf16 per V^T row in LDS (4 of padding)
constexpr int TA_OPAD = 4;     // fp32 padding of an output row in LDS

struct TAParams {
  const uint16_t *Q, *K, *V;
  const int32_t *prefix_len, *n_nodes;
  const uint8_t *mask;
  float *O;
  float *part;   // [b][Hkv][S][Rpad][DH] unnormalised partial outputs (S > 1)
  float *ml;     // [b][Hkv][S][Rpad][2]: running max (log2 units), weight sum
  int b, n_max, Hq, Hkv, G, L_cap, S, RB, Rpad;
  float scale_log2;
};

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return (uint32_t)f32_to_bf16_rne(a) | ((uint32_t)f32_to_bf16_rne(b) << 16);
}

__device__ __forceinline__ bool request_ok(int P, int n, int n_max, int L_cap) {
  return P >= 0 && n >= 1 && n <= n_max && P <= L_cap - n;
}

// Work item of a linear workgroup id.  Workgroup i runs on XCD i % 8; the
// row blocks of one (request, KV head, split) read the same K/V, so the
// ids are permuted to put consecutive work items on one XCD (one L2).
__device__ __forceinline__ int work_item(int lin, int total) {
  if (total % 8) return lin;
  return (lin & 7) * (total >> 3) + (lin >> 3);
}

template <int DH>
__global__ __launch_bounds__(TA_THREADS) void k_tree_attn(TAParams p) {
  constexpr int NKS = DH / 32;        // 32-dim k-steps of Q.K
  constexpr int NDT = DH / 16;        // 16-dim output tiles
  constexpr int KROW = DH + TA_KPAD;  // bf16 per K row in LDS
  constexpr int KCH = TA_KT * DH / 8 / TA_THREADS;   // 16-byte K chunks per thread
  constexpr int VQ = 16 * DH / 8;     // (key quad, 8-dim chunk) pairs per tile
  constexpr int KBYTES = TA_KT * KROW * 2, VBYTES = DH * TA_VROW * 2;
  constexpr int OBYTES = TA_QB * (DH + TA_OPAD) * 4;
  // K tile, then the V^T tile; after the loop the same bytes hold the
  // merged output rows [TA_QB][DH + TA_OPAD] fp32
  __shared__ __align__(16) uint8_t smem[KBYTES + VBYTES > OBYTES ? KBYTES + VBYTES : OBYTES];
  __shared__ float mw[4][TA_QB], lw[4][TA_QB];
  uint16_t *Ks = reinterpret_cast<uint16_t *>(smem);
  uint16_t *Vt = reinterpret_cast<uint16_t *>(smem + KBYTES);
  float *Obuf = reinterpret_cast<float *>(smem);

  const int total = p.RB * p.Hkv * p.b * p.S;
  const int w = work_item(blockIdx.x, total);
  const int rb = w % p.RB;
  const int kvh = (w / p.RB) % p.Hkv;
  const int qs = w / (p.RB * p.Hkv);
  const int q = qs / p.S, s = qs - q * p.S;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 15, g = lane >> 4;
  const int G = p.G;
  const int P = p.prefix_len[q], n = p.n_nodes[q];
  const int r0 = rb * TA_QB;
  const size_t ostride = (size_t)p.Hq * DH;

  // rows this workgroup writes when it owns the whole key range
  auto write_rows = [&](float v) {
    const int rows = min(TA_QB, p.n_max * G - r0);
    for (int e = tid; e < rows * (DH / 4); e += TA_THREADS) {
      const int rr = r0 + e / (DH / 4), c = e % (DH / 4);
      const int i = rr / G, hq = kvh * G + rr % G;
      *reinterpret_cast<f32x4 *>(p.O + ((size_t)q * p.n_max + i) * ostride + (size_t)hq * DH + 4 * c) =
          f32x4{v, v, v, v};
    }
  };
  if (!request_ok(P, n, p.n_max, p.L_cap)) {   // the merge kernel marks the rows when S > 1
    if (p.S == 1) write_rows(NAN);
    return;
  }
  const int nrows = n * G;
  if (r0 >= nrows) {          // padding rows only
    if (p.S == 1) write_rows(0.f);
    return;
  }
  // keys of this row block: the prefix and tree nodes up to its last node
  const int node_hi = min(n, (min(r0 + TA_QB, nrows) - 1) / G + 1);
  const int Lb = P + node_hi;
  const int per = (((Lb + p.S - 1) / p.S) + TA_KT - 1) / TA_KT * TA_KT;
  const int kb = s * per, ke = min(Lb, kb + per);
  const size_t slot = (((size_t)q * p.Hkv + kvh) * p.S + s) * p.Rpad;
  if (kb >= ke) {             // an empty split contributes nothing
    for (int e = tid; e < TA_QB; e += TA_THREADS) {
      p.ml[(slot + r0 + e) * 2 + 0] = -INFINITY;
      p.ml[(slot + r0 + e) * 2 + 1] = 0.f;
    }
    for (int e = tid; e < TA_QB * DH / 4; e += TA_THREADS)
      *reinterpret_cast<f32x4 *>(p.part + (slot + r0) * DH + 4 * e) = f32x4{0.f, 0.f, 0.f, 0.f};
    return;
  }

  // query fragments (B operand of S^T = K Q^T): lane holds query row lr of
  // q-tile qt, dims 32 ks + 8 g .. + 8
  uint4 qf[4][NKS];
  const uint8_t *mrow[4];
#pragma unroll
  for (int qt = 0; qt < 4; ++qt) {
    const int r = r0 + 16 * qt + lr;
    const bool ok = r < nrows;
    const int i = ok ? r / G : 0, hq = kvh * G + (ok ? r % G : 0);
    const uint16_t *src = p.Q + ((size_t)q * p.n_max + i) * ostride + (size_t)hq * DH + 8 * g;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      qf[qt][ks] = ok ? *reinterpret_cast<const uint4 *>(src + 32 * ks) : make_uint4(0, 0, 0, 0);
    mrow[qt] = p.mask + ((size_t)q * p.n_max + i) * p.n_max;
  }

  const uint16_t *Kg = p.K + ((size_t)q * p.Hkv + kvh) * p.L_cap * DH;
  const uint16_t *Vg = p.V + ((size_t)q * p.Hkv + kvh) * p.L_cap * DH;
  // staged tile in registers: K chunks (key, 8 dims) and V quads (4 keys x 8 dims)
  uint4 kr[KCH], vr[4];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
      const int c = tid + TA_THREADS * u, key = c / (DH / 8), col = c % (DH / 8);
      const int k = k0 + key;
      kr[u] = k < ke ? *reinterpret_cast<const uint4 *>(Kg + (size_t)k * DH + 8 * col)
                     : make_uint4(0, 0, 0, 0);
    }
    if (tid < VQ) {
      const int kq = tid / (DH / 8), col = tid % (DH / 8);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int k = k0 + 4 * kq + u;
        vr[u] = k < ke ? *reinterpret_cast<const uint4 *>(Vg + (size_t)k * DH + 8 * col)
                       : make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
      const int c = tid + TA_THREADS * u, key = c / (DH / 8), col = c % (DH / 8);
      *reinterpret_cast<uint4 *>(Ks + key * KROW + 8 * col) = kr[u];
    }
    if (tid < VQ) {
      const int kq = tid / (DH / 8), col = tid % (DH / 8);
      // V^T rows 8 col + d, keys 4 kq .. 4 kq + 3
      const uint32_t *v32[4] = {reinterpret_cast<const uint32_t *>(&vr[0]),
                                reinterpret_cast<const uint32_t *>(&vr[1]),
                                reinterpret_cast<const uint32_t *>(&vr[2]),
                                reinterpret_cast<const uint32_t *>(&vr[3])};
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const int sh = (d & 1) * 16;
        const uint32_t e0 = (v32[0][d >> 1] >> sh) & 0xFFFFu, e1 = (v32[1][d >> 1] >> sh) & 0xFFFFu;
        const uint32_t e2 = (v32[2][d >> 1] >> sh) & 0xFFFFu, e3 = (v32[3][d >> 1] >> sh) & 0xFFFFu;
        *reinterpret_cast<uint2 *>(Vt + (8 * col + d) * TA_VROW + 4 * kq) =
            make_uint2(e0 | (e1 << 16), e2 | (e3 << 16));
      }
    }
  };

  float m[4], l[4];
  f32x4 o[NDT][4];
#pragma unroll
  for (int qt = 0; qt < 4; ++qt) {
    m[qt] = -INFINITY;
    l[qt] = 0.f;
#pragma unroll
    for (int nt = 0; nt < NDT; ++nt) o[nt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  fetch(kb);
  for (int k0 = kb; k0 < ke; k0 += TA_KT) {
    stage();
    __syncthreads();
    if (k0 + TA_KT < ke) fetch(k0 + TA_KT);   // lands while this tile is used

    // S^T for this wave's 16 keys and the 64 query rows
    f32x4 sc[4];
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) sc[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const uint4 a = *reinterpret_cast<const uint4 *>(Ks + (16 * wave + lr) * KROW + 32 * ks + 8 * g);
#pragma unroll
      for (int qt = 0; qt < 4; ++qt)
        sc[qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(qf[qt][ks]), sc[qt],
                                                         0, 0, 0);
    }
    // lane: query lr of each q-tile, keys kk0 + t
    const int kk0 = k0 + 16 * wave + 4 * g;
    const bool tree = k0 + TA_KT > P;   // the tile holds tree keys (uniform)
    i16x4 pk[4];
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) {
      float v[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int kk = kk0 + t;
        bool vis = kk < ke;
        if (tree && vis && kk >= P) vis = mrow[qt][kk - P] != 0;
        v[t] = vis ? sc[qt][t] * p.scale_log2 : -INFINITY;
      }
      float mx = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mn = fmaxf(m[qt], mx);
      const float mu = mn == -INFINITY ? 0.f : mn;
      const float alpha = exp2f(m[qt] - mu);
      float e[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) e[t] = exp2f(v[t] - mu);
      l[qt] = l[qt] * alpha + ((e[0] + e[1]) + (e[2] + e[3]));
      m[qt] = mn;
      if (alpha != 1.f) {
#pragma unroll
        for (int nt = 0; nt < NDT; ++nt) o[nt][qt] *= alpha;
      }
      const uint32_t lo = pack_bf16(e[0], e[1]), hi = pack_bf16(e[2], e[3]);
      pk[qt] = __builtin_bit_cast(i16x4, make_uint2(lo, hi));
    }
    // O^T += V^T P^T over the wave's 16 keys
#pragma unroll
    for (int nt = 0; nt < NDT; ++nt) {
      const uint2 a = *reinterpret_cast<const uint2 *>(Vt + (16 * nt + lr) * TA_VROW + 16 * wave + 4 * g);
      const i16x4 av = __builtin_bit_cast(i16x4, a);
#pragma unroll
      for (int qt = 0; qt < 4; ++qt)
        o[nt][qt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, pk[qt], o[nt][qt], 0, 0, 0);
    }
    __syncthreads();
  }

  // ---- merge the four waves: common max, rescale, sum in a fixed order
#pragma unroll
  for (int qt = 0; qt < 4; ++qt) {
    float lt = l[qt];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    if (g == 0) {
      mw[wave][16 * qt + lr] = m[qt];
      lw[wave][16 * qt + lr] = lt;
    }
  }
  __syncthreads();
  float fself[4], lsum[4], mall[4];
#pragma unroll
  for (int qt = 0; qt < 4; ++qt) {
    const int row = 16 * qt + lr;
    float M = fmaxf(fmaxf(mw[0][row], mw[1][row]), fmaxf(mw[2][row], mw[3][row]));
    const float Mu = M == -INFINITY ? 0.f : M;
    float L = 0.f;
#pragma unroll
    for (int wv = 0; wv < 4; ++wv) L += lw[wv][row] * exp2f(mw[wv][row] - Mu);
    fself[qt] = exp2f(m[qt] - Mu);
    lsum[qt] = L;
    mall[qt] = M;
  }
  constexpr int OROW = DH + TA_OPAD;
  for (int wv = 0; wv < 3; ++wv) {
    if (wave == wv) {
#pragma unroll
      for (int qt = 0; qt < 4; ++qt)
#pragma unroll
        for (int nt = 0; nt < NDT; ++nt) {
          float *dst = Obuf + (16 * qt + lr) * OROW + 16 * nt + 4 * g;
          f32x4 v = o[nt][qt] * fself[qt];
          if (wv > 0) v += *reinterpret_cast<const f32x4 *>(dst);
          *reinterpret_cast<f32x4 *>(dst) = v;
        }
    }
    __syncthreads();
  }
  if (wave != 3) return;
#pragma unroll
  for (int qt = 0; qt < 4; ++qt) {
    const int r = r0 + 16 * qt + lr;
    if (r >= p.n_max * G) continue;
    const int i = r / G, hq = kvh * G + r % G;
    const bool live = r < nrows;
    if (p.S == 1) {
      const float inv = 1.f / lsum[qt];
      float *dst = p.O + ((size_t)q * p.n_max + i) * ostride + (size_t)hq * DH + 4 * g;
#pragma unroll
      for (int nt = 0; nt < NDT; ++nt) {
        const f32x4 acc =
            *reinterpret_cast<const f32x4 *>(Obuf + (16 * qt + lr) * OROW + 16 * nt + 4 * g) +
            o[nt][qt] * fself[qt];
        *reinterpret_cast<f32x4 *>(dst + 16 * nt) = live ? acc * inv : f32x4{0.f, 0.f, 0.f, 0.f};
      }
    } else {
      float *dst = p.part + (slot + r) * DH + 4 * g;
#pragma unroll
      for (int nt = 0; nt < NDT; ++nt) {
        const f32x4 acc =
            *reinterpret_cast<const f32x4 *>(Obuf + (16 * qt + lr) * OROW + 16 * nt + 4 * g) +
            o[nt][qt] * fself[qt];
        *reinterpret_cast<f32x4 *>(dst + 16 * nt) = acc;
      }
      if (g == 0) {
        p.ml[(slot + r) * 2 + 0] = mall[qt];
        p.ml[(slot + r) * 2 + 1] = lsum[qt];
      }
    }
  }
}

// Merge of the splits of every row: common max, weights 2^(m_s - M).
template <int DH>
__global__ __launch_bounds__(256) void k_tree_attn_merge(TAParams p) {
  const int per_row = DH / 4;
  const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t rows = (size_t)p.b * p.n_max * p.Hq;
  if (e >= rows * per_row) return;
  const int c = (int)(e % per_row);
  const size_t orow = e / per_row;                 // (q, i, hq)
  const int hq = (int)(orow % p.Hq);
  const int i = (int)((orow / p.Hq) % p.n_max);
  const int q = (int)(orow / ((size_t)p.Hq * p.n_max));
  const int kvh = hq / p.G, r = i * p.G + hq % p.G;
  float *dst = p.O + orow * DH + 4 * c;
  const int P = p.prefix_len[q], n = p.n_nodes[q];
  if (!request_ok(P, n, p.n_max, p.L_cap)) {
    *reinterpret_cast<f32x4 *>(dst) = f32x4{NAN, NAN, NAN, NAN};
    return;
  }
  if (i >= n) {
    *reinterpret_cast<f32x4 *>(dst) = f32x4{0.f, 0.f, 0.f, 0.f};
    return;
  }
  const size_t base = ((size_t)q * p.Hkv + kvh) * p.S * p.Rpad + r;
  float M = -INFINITY;
  for (int s = 0; s < p.S; ++s) M = fmaxf(M, p.ml[(base + (size_t)s * p.Rpad) * 2]);
  const float Mu = M == -INFINITY ? 0.f : M;
  f32x4 acc{0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
  for (int s = 0; s < p.S; ++s) {
    const size_t at = base + (size_t)s * p.Rpad;
    const float f = exp2f(p.ml[at * 2] - Mu);
    L += p.ml[at * 2 + 1] * f;
    acc += *reinterpret_cast<const f32x4 *>(p.part + at * DH + 4 * c) * f;
  }
  *reinterpret_cast<f32x4 *>(dst) = acc * (1.f / L);
}

}  // namespace

int tree_attn_splits(int batch, int n_max, int Hq, int Hkv, int L_cap, int requested) {
  const int G = Hq / Hkv;
  const int RB = (n_max * G + TA_QB - 1) / TA_QB;
  const int cap = (L_cap + 255) / 256;     // at least 256 keys per split
  if (requested > 0) return requested;
  const long base = (long)batch * Hkv * RB;
  if (base >= 512) return 1;
  int S = (int)((512 + base - 1) / base);
  S = S < cap ? S : cap;
  S = S > 64 ? 64 : S;
  return S < 1 ? 1 : S;
}

size_t tree_attn_workspace(int batch, int n_max, int Hq, int Hkv, int dh, int S) {
  if (S <= 1) return 0;
  const int G = Hq / Hkv;
  const size_t Rpad = (size_t)(n_max * G + TA_QB - 1) / TA_QB * TA_QB;
  const size_t rows = (size_t)batch * Hkv * S * Rpad;
  const size_t part = (rows * dh * 4 + 255) & ~(size_t)255;
  return part + rows * 2 * 4;
}

hipError_t launch_tree_attn(const TreeAttnArgs &a, hipStream_t st) {
  TAParams p{};
  p.Q = static_cast<const uint16_t *>(a.Q);
  p.K = static_cast<const uint16_t *>(a.K);
  p.V = static_cast<const uint16_t *>(a.V);
  p.prefix_len = a.prefix_len;
  p.n_nodes = a.n_nodes;
  p.mask = a.mask;
  p.O = a.O;
  p.b = a.batch; p.n_max = a.n_max; p.Hq = a.Hq; p.Hkv = a.Hkv; p.G = a.Hq / a.Hkv;
  p.L_cap = a.L_cap; p.S = a.splits;
  p.RB = (a.n_max * p.G + TA_QB - 1) / TA_QB;
  p.Rpad = p.RB * TA_QB;
  p.scale_log2 = a.scale * 1.4426950408889634f;
  if (p.S > 1) {
    uint8_t *ws = static_cast<uint8_t *>(a.workspace);
    const size_t rows = (size_t)p.b * p.Hkv * p.S * p.Rpad;
    p.part = reinterpret_cast<float *>(ws);
    p.ml = reinterpret_cast<float *>(ws + ((rows * a.dh * 4 + 255) & ~(size_t)255));
  }
  const unsigned grid = (unsigned)(p.RB * p.Hkv * p.b * p.S);
  const size_t merge = (size_t)p.b * p.n_max * p.Hq * (a.dh / 4);
  if (a.dh == 128) {
    hipLaunchKernelGGL(k_tree_attn<128>, dim3(grid), dim3(TA_THREADS), 0, st, p);
    if (p.S > 1)
      hipLaunchKernelGGL(k_tree_attn_merge<128>, dim3((unsigned)((merge + 255) / 256)), dim3(256),
                         0, st, p);
  } else {
    hipLaunchKernelGGL(k_tree_attn<64>, dim3(grid), dim3(TA_THREADS), 0, st, p);
    if (p.S > 1)
      hipLaunchKernelGGL(k_tree_attn_merge<64>, dim3((unsigned)((merge + 255) / 256)), dim3(256),
                         0, st, p);
  }
  return hipGetLastError();
}

}  // namespace dtree
