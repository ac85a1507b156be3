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
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace dtree {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int TA_THREADS = 256;
constexpr int TA_WROWS = 32;          // query rows per wave (two 16-row q-tiles)
constexpr int TA_QB = 4 * TA_WROWS;   // query rows per workgroup
constexpr int TA_KT = 64;             // keys per tile
constexpr int TA_KPAD = 8;            // bf16 padding of a K row in LDS
constexpr int TA_VROW = TA_KT + 4;    // bf16 per V^T row in LDS (4 of padding)
constexpr float TA_TAU = 8.f;         // lazy softmax reference: slack in log2 units

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

// two fp32 values to bf16, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

__device__ __forceinline__ bool request_ok(int P, int n, int n_max, int L_cap) {
  return P >= 0 && n >= 1 && n <= n_max && P <= L_cap - n;
}

// Max / sum over the lanes l, l ^ 16, l ^ 32, l ^ 48 (the four lane groups
// that hold one query row's keys), with the gfx950 lane-swap instructions:
// each swap leaves a lane holding its own value and its partner's, in some
// order; max and + are symmetric, so every lane of the four gets the same bits.
__device__ __forceinline__ float swap_pair_max(float v, bool x32) {
  const auto r = x32 ? __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false)
                     : __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float swap_pair_sum(float v, bool x32) {
  const auto r = x32 ? __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false)
                     : __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float group4_max(float v) {
  return swap_pair_max(swap_pair_max(v, false), true);
}
__device__ __forceinline__ float group4_sum(float v) {
  return swap_pair_sum(swap_pair_sum(v, false), true);
}

// Work item of a linear workgroup id.  Workgroup i runs on XCD i % 8; the
// row blocks of one (request, KV head, split) read the same K/V, so the
// ids are permuted to put consecutive work items on one XCD (one L2).
__device__ __forceinline__ int work_item(int lin, int total) {
  if (total % 8) return lin;
  return (lin & 7) * (total >> 3) + (lin >> 3);
}

template <int DH>
__global__ __launch_bounds__(TA_THREADS, 2) void k_tree_attn(TAParams p) {
  constexpr int NKS = DH / 32;        // 32-dim k-steps of Q.K
  constexpr int NDT = DH / 16;        // 16-dim output tiles
  constexpr int KROW = DH + TA_KPAD;  // bf16 per K row in LDS
  constexpr int KCH = TA_KT * DH / 8 / TA_THREADS;   // 16-byte K chunks per thread
  constexpr int VQ = 16 * DH / 8;     // (key quad, 8-dim chunk) pairs per tile
  // two tile buffers: tile t is read from buffer t & 1 while tile t + 1 is
  // written into the other one
  __shared__ __align__(16) uint16_t Ksb[2][TA_KT * KROW];
  __shared__ __align__(16) uint16_t Vtb[2][DH * TA_VROW];

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

  // this wave's 32 query rows: fragments of the B operand of S^T = K Q^T
  // (lane: row lr of q-tile qt, dims 32 ks + 8 g .. + 8) and mask rows
  const int wr0 = r0 + TA_WROWS * wave;
  uint4 qf[2][NKS];
  const uint8_t *mrow[2];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int r = wr0 + 16 * qt + lr;
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
  // Tile loads through buffer descriptors whose size ends at key ke: the
  // hardware returns zeros for every key at or past ke (partial tiles need
  // no per-lane test), and each load is one 32-bit offset add.
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(Kg), (short)0, ke * DH * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(Vg), (short)0, ke * DH * 2, 0x00020000);
  // K chunk u of this thread: key tid / (DH / 8) + u * 256 / (DH / 8), dims
  // 8 (tid % (DH / 8)) .. + 8, i.e. byte offset kbase + 4096 u; V quad: keys
  // 4 (tid & 15) + u, dims 8 (tid >> 4) .. + 8
  const int kbase = (tid / (DH / 8)) * DH * 2 + (tid % (DH / 8)) * 16;
  const int vbase = 4 * (tid & 15) * DH * 2 + (tid >> 4) * 16;
  auto ld = [](__amdgpu_buffer_rsrc_t r, int off) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
  };
  auto fetch_tile = [&](int k0) {
    const int t0 = k0 * DH * 2;
#pragma unroll
    for (int u = 0; u < KCH; ++u) kr[u] = ld(krs, t0 + kbase + 4096 * u);
    if (tid < VQ) {
#pragma unroll
      for (int u = 0; u < 4; ++u) vr[u] = ld(vrs, t0 + vbase + u * DH * 2);
    }
  };
  auto stage = [&](int buf) {
    uint16_t *Ks = Ksb[buf], *Vt = Vtb[buf];
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
      const int c = tid + TA_THREADS * u, key = c / (DH / 8), col = c % (DH / 8);
      *reinterpret_cast<uint4 *>(Ks + key * KROW + 8 * col) = kr[u];
    }
    if (tid < VQ) {
      // V^T rows 8 col + d, keys 4 kq .. 4 kq + 3; the 16 lanes of a row
      // group write 16 different key quads of one row (distinct banks)
      const int kq = tid & 15, col = tid >> 4;
      const uint32_t w0[4] = {vr[0].x, vr[0].y, vr[0].z, vr[0].w};
      const uint32_t w1[4] = {vr[1].x, vr[1].y, vr[1].z, vr[1].w};
      const uint32_t w2[4] = {vr[2].x, vr[2].y, vr[2].z, vr[2].w};
      const uint32_t w3[4] = {vr[3].x, vr[3].y, vr[3].z, vr[3].w};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        // low halves (dim 2m) and high halves (dim 2m + 1) of the 4 keys
        *reinterpret_cast<uint2 *>(Vt + (8 * col + 2 * m) * TA_VROW + 4 * kq) =
            make_uint2(__builtin_amdgcn_perm(w1[m], w0[m], 0x05040100u),
                       __builtin_amdgcn_perm(w3[m], w2[m], 0x05040100u));
        *reinterpret_cast<uint2 *>(Vt + (8 * col + 2 * m + 1) * TA_VROW + 4 * kq) =
            make_uint2(__builtin_amdgcn_perm(w1[m], w0[m], 0x07060302u),
                       __builtin_amdgcn_perm(w3[m], w2[m], 0x07060302u));
      }
    }
  };

  // online softmax with a lazily moved reference: the reference m only
  // moves when a score exceeds it by more than TA_TAU (log2 units), so the
  // weights 2^(x - m) stay below 2^TA_TAU and rescales are rare
  float mref[2] = {-INFINITY, -INFINITY}, lsum[2] = {0.f, 0.f};
  f32x4 o[2][NDT];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int nt = 0; nt < NDT; ++nt) o[qt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // one tile: MASKED tiles hold tree keys or run past ke (the mask and the
  // bounds are tested per key); the others are full tiles of prefix keys
  // Tile k0 is in buffer buf; the registers hold tile k0 + TA_KT (if any),
  // which goes to the other buffer after this tile's products, followed by
  // the loads of tile k0 + 2 TA_KT and one barrier.  A buffer is rewritten
  // only after the barrier that ends the tile that read it.
  auto tile = [&](int k0, int buf, auto masked_c) {
    constexpr bool MASKED = decltype(masked_c)::value;
    const uint16_t *Ks = Ksb[buf], *Vt = Vtb[buf];

    // S^T: four 16-key blocks x two q-tiles; lane: query lr, keys 16 kb4 + 4 g + t
    f32x4 sc[2][4];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4) sc[qt][k4] = f32x4{0.f, 0.f, 0.f, 0.f};
    // K fragments are read from LDS two steps ahead of their products (a
    // ring of three), so the LDS latency overlaps the matrix cores
    {
      constexpr int NF = 4 * NKS;
      // order: k-step outer, key block inner, so consecutive products go to
      // different accumulators
      auto kfrag = [&](int f) {
        const int ks = f / 4, k4 = f % 4;
        return *reinterpret_cast<const uint4 *>(Ks + (16 * k4 + lr) * KROW + 32 * ks + 8 * g);
      };
      uint4 ring[3];
      ring[0] = kfrag(0);
      ring[1] = kfrag(1);
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        if (f + 2 < NF) ring[(f + 2) % 3] = kfrag(f + 2);
        __builtin_amdgcn_sched_barrier(0);   // keep the read ahead of the products
        const int ks = f / 4, k4 = f % 4;
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
          sc[qt][k4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ring[f % 3]),
                                                               as_bf16x8(qf[qt][ks]), sc[qt][k4], 0, 0, 0);
      }
    }
    // masked and out-of-range keys get a raw score of -inf
    const float c2 = p.scale_log2;   // > 0: the max of raw scores scales to the max
    float x[2][16];   // raw scores q.k
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4)
#pragma unroll
        for (int t = 0; t < 4; ++t) x[qt][4 * k4 + t] = sc[qt][k4][t];
    if constexpr (MASKED) {
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4)
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int kk = k0 + 16 * k4 + 4 * g + t, j = kk - P;
            const int jc = min(max(j, 0), p.n_max - 1);   // in bounds: load unconditionally
            const uint32_t mb = mrow[qt][jc];
            const bool vis = (kk < ke) & ((j < 0) | (mb != 0u));
            x[qt][4 * k4 + t] = vis ? x[qt][4 * k4 + t] : -INFINITY;
          }
    }
    // tile max of each query row: own 16 keys, then the lanes l ^ 16, l ^ 32
    float mx[2];
    bool move[2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      float m = x[qt][0];
#pragma unroll
      for (int e = 1; e < 16; ++e) m = fmaxf(m, x[qt][e]);
      mx[qt] = group4_max(m) * c2;
      move[qt] = mx[qt] > mref[qt] + TA_TAU;
    }
    if (__any(move[0] | move[1])) {
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
        if (move[qt]) {
          const float alpha = __builtin_amdgcn_exp2f(mref[qt] - mx[qt]);   // 0 while mref = -inf
          lsum[qt] *= alpha;
#pragma unroll
          for (int nt = 0; nt < NDT; ++nt) o[qt][nt] *= alpha;
          mref[qt] = mx[qt];
        }
    }
    uint4 pk[2][2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      const float mu = mref[qt] == -INFINITY ? 0.f : mref[qt];
      float e[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) e[k] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[qt][k], c2, -mu));
      float ls = 0.f;
#pragma unroll
      for (int k = 0; k < 16; ++k) ls += e[k];
      lsum[qt] += ls;
      // k-step c of O^T += V^T P^T: keys 32 c + 4 g + t and 32 c + 16 + 4 g + t
#pragma unroll
      for (int c = 0; c < 2; ++c)
        pk[qt][c] = make_uint4(pack_bf16(e[8 * c + 0], e[8 * c + 1]), pack_bf16(e[8 * c + 2], e[8 * c + 3]),
                               pack_bf16(e[8 * c + 4], e[8 * c + 5]), pack_bf16(e[8 * c + 6], e[8 * c + 7]));
    }
    // O^T += V^T P^T (A = V^T rows 16 nt + lr, the same keys in the same
    // order); V^T fragments two steps ahead of their products, as above
    {
      constexpr int NF = 2 * NDT;
      // order: k-step outer, output tile inner (independent accumulators)
      auto vfrag = [&](int f) {
        const int c = f / NDT, nt = f % NDT;
        const uint16_t *vrow = Vt + (16 * nt + lr) * TA_VROW + 32 * c + 4 * g;
        const uint2 lo = *reinterpret_cast<const uint2 *>(vrow);
        const uint2 hi = *reinterpret_cast<const uint2 *>(vrow + 16);
        return make_uint4(lo.x, lo.y, hi.x, hi.y);
      };
      uint4 ring[3];
      ring[0] = vfrag(0);
      ring[1] = vfrag(1);
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        if (f + 2 < NF) ring[(f + 2) % 3] = vfrag(f + 2);
        __builtin_amdgcn_sched_barrier(0);
        const int c = f / NDT, nt = f % NDT;
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
          o[qt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ring[f % 3]), as_bf16x8(pk[qt][c]),
                                                              o[qt][nt], 0, 0, 0);
      }
    }
    if (k0 + TA_KT < ke) {
      stage(buf ^ 1);
      if (k0 + 2 * TA_KT < ke) fetch_tile(k0 + 2 * TA_KT);
    }
    __syncthreads();
  };

  // full tiles of prefix keys first (the bulk), then the rest
  const int pe = min(ke, P);
  const int kplain = pe > kb ? kb + (pe - kb) / TA_KT * TA_KT : kb;
  fetch_tile(kb);
  stage(0);
  if (kb + TA_KT < ke) fetch_tile(kb + TA_KT);
  __syncthreads();
  int k0 = kb, buf = 0;
  for (; k0 < kplain; k0 += TA_KT, buf ^= 1) tile(k0, buf, std::false_type());
  for (; k0 < ke; k0 += TA_KT, buf ^= 1) tile(k0, buf, std::true_type());

  // ---- this wave's rows: lane holds query wr0 + 16 qt + lr, dims 16 nt + 4 g + t
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const float lt = group4_sum(lsum[qt]);
    const int r = wr0 + 16 * qt + lr;
    if (r >= p.n_max * G) continue;
    const int i = r / G, hq = kvh * G + r % G;
    const bool live = r < nrows;
    if (p.S == 1) {
      const float inv = 1.f / lt;
      float *dst = p.O + ((size_t)q * p.n_max + i) * ostride + (size_t)hq * DH + 4 * g;
#pragma unroll
      for (int nt = 0; nt < NDT; ++nt)
        *reinterpret_cast<f32x4 *>(dst + 16 * nt) = live ? o[qt][nt] * inv : f32x4{0.f, 0.f, 0.f, 0.f};
    } else {
      float *dst = p.part + (slot + r) * DH + 4 * g;
#pragma unroll
      for (int nt = 0; nt < NDT; ++nt) *reinterpret_cast<f32x4 *>(dst + 16 * nt) = o[qt][nt];
      if (g == 0) {
        p.ml[(slot + r) * 2 + 0] = mref[qt];
        p.ml[(slot + r) * 2 + 1] = lt;
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
  if (requested > 0) return requested;
  // Choose the key splits S by a small cost model, in units of one tile's
  // time: workgroups run two per CU (512 at once), so the kernel takes
  // ceil(blocks * S / 512) rounds of ceil(tiles / S) tiles, and every split
  // adds partial outputs for the merge (measured at about half a tile of
  // time per split at these shapes).  Splits keep at least 256 keys.
  const int G = Hq / Hkv;
  const long base = (long)batch * Hkv * ((n_max * G + TA_QB - 1) / TA_QB);
  const long tiles = (L_cap + TA_KT - 1) / TA_KT;
  const int cap = (L_cap + 255) / 256;
  int best = 1;
  double best_cost = 1e30;
  for (int S = 1; S <= cap && S <= 64; ++S) {
    const double cost = (double)((base * S + 511) / 512) * (double)((tiles + S - 1) / S) + 0.5 * S;
    if (cost < best_cost) {
      best_cost = cost;
      best = S;
    }
  }
  return best;
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
