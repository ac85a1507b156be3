// Sequential best-first tree builder ("Resumen Técnico: DominoTree",
// Componentes Principales 1 and 2): a max-priority queue of draft nodes keyed
// by cumulative corrected log-probability; every pop runs the GRU one step
// along the popped node's own path, corrects the next depth's Top-M
// candidates with that state and pushes the node's Top-k children.  The
// pages compare exactly this node-at-a-time loop with the depth-wise batched
// build ("DARTree: Speculative Diffusion Decoding with Autoregressive Draft
// Trees", Planteamiento del Problema 3 and Resultados Experimentales,
// Ablación: latency).
//
// Per pop, two launches on the round's stream (no host synchronisation):
//   k_heap_step   one workgroup per request: corrects the node whose state
//                 product has just been computed (log-softmax over the M
//                 candidates, Top-K, children pushed), pops the best open
//                 node and runs its GRU combine from the candidate's input
//                 projection and its parent's stored state product;
//   a GEMM        [u | W_hh S + b_hh] = [W1[:, d:] ; W_hh] . S of the popped
//                 node, stored in the node's slot for its own children.
// The queue is the open set of the request's node table; a pop is a
// workgroup-wide arg-max in the builder's total order: key = score + beta *
// depth (fp32, rounded after each operation) descending, then depth
// ascending, then the token path lexicographically ascending.  Node ids are
// in push order; a node's expansion slot is 1 + the step that popped it
// (the root uses slot 0).
#include <hip/hip_runtime.h>
#include <cmath>
#include <cstdint>

#include "common.hpp"
#include "kernels.hpp"

namespace dtree {
namespace {

constexpr int HP_THREADS = 256;

struct HeapStepParams {
  int t, B, D, M, K, s, r, markov, V, vec, wl;
  float beta;
  const void *W2;
  int w2_bf16;
  const int32_t *C;
  const float *Cl, *uH;
  const int32_t *root;
  const float *S_root, *b_hh;
  HeapBufs h;
};

__device__ __forceinline__ float sel_key(float score, int dep, float beta) {
  return __fadd_rn(score, __fmul_rn(beta, (float)dep));
}

// a strictly before b in the builder's total order (a != b, both pushed)
__device__ bool heap_before(int a, int b, const int32_t *tok, const int32_t *par,
                            const int32_t *dep, const float *score, float beta) {
  const float ka = sel_key(score[a], dep[a], beta), kb = sel_key(score[b], dep[b], beta);
  if (ka != kb) return ka > kb;
  if (dep[a] != dep[b]) return dep[a] < dep[b];
  // same depth: the first differing token from the root decides; walk up to
  // the deepest common ancestor
  while (par[a] != par[b]) {
    a = par[a];
    b = par[b];
  }
  return tok[a] < tok[b];
}

// packed pop order of one node: ord(key) << 32 | (2^32 - 1 - depth), larger
// is better (equal values: the token path decides); 0 marks a node that is
// not open (popped, or the root)
__device__ __forceinline__ uint64_t pop_value(float score, int dep, float beta) {
  return ((uint64_t)f32_ord(sel_key(score, dep, beta)) << 32) |
         (uint64_t)(0xFFFFFFFFu - (uint32_t)dep);
}
__device__ __forceinline__ int pop_depth(uint64_t v) {
  return (int)(0xFFFFFFFFu - (uint32_t)v);
}

// LDS of one heap step: the pop values of the request's nodes [NH], every
// depth's uH [D r], C and Cl [D M], u [r], ell and keys [M]
struct HeapStepLds {
  size_t pv, uH, C, Cl, u, ell, keys, total;
};
__host__ __device__ inline HeapStepLds heap_step_layout(int NH, int D, int M, int r) {
  HeapStepLds L{};
  size_t o = 0;
  auto take = [&](size_t b) { size_t at = o; o += (b + 15) & ~(size_t)15; return at; };
  L.pv = take((size_t)NH * 8);
  L.uH = take((size_t)D * r * 4);
  L.C = take((size_t)D * M * 4);
  L.Cl = take((size_t)D * M * 4);
  L.u = take((size_t)r * 4);
  L.ell = take((size_t)M * 4);
  L.keys = take((size_t)M * 8);
  L.total = o;
  return L;
}

typedef unsigned hu32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t heap_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           0x00020000);
}
// 16 bytes at byte offset off of a buffer; zeros past its end
__device__ __forceinline__ hu32x4 heap_ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}

// Copies bytes [from, bytes) of a buffer to LDS in 16-byte pieces, U pieces
// per thread in flight (bytes a multiple of 16).
template <int U>
__device__ __forceinline__ void heap_stage16(uint8_t *dst, __amdgpu_buffer_rsrc_t r,
                                             uint32_t from, uint32_t bytes, int tid) {
  for (uint32_t base = from; base < bytes; base += U * 16 * HP_THREADS) {
    hu32x4 v[U];
#pragma unroll
    for (int j = 0; j < U; ++j) v[j] = heap_ld16(r, base + 16 * (tid + j * HP_THREADS));
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const uint32_t o = base + 16 * (tid + j * HP_THREADS);
      if (o < bytes) *reinterpret_cast<hu32x4 *>(dst + o) = v[j];
    }
  }
}

// One step of the best-first loop for one request (one workgroup): expand
// the node the previous step popped (its state product is in slot t) and
// pop the next one.  Round trips to memory: (1) the step record, the pop
// values, every depth's correction tables and the state product, all
// issued together; (2) the M rows of W2; (3) the popped node's candidate,
// parent slot and score; (4) the GRU inputs.
__global__ __launch_bounds__(HP_THREADS) void k_heap_step(HeapStepParams p) {
  extern __shared__ __align__(16) uint8_t smem[];
  const HeapBufs &h = p.h;
  const HeapStepLds L = heap_step_layout(h.NH, p.D, p.M, p.r);
  uint64_t *pv_s = reinterpret_cast<uint64_t *>(smem + L.pv);
  float *uH_s = reinterpret_cast<float *>(smem + L.uH);
  int *C_s = reinterpret_cast<int *>(smem + L.C);
  float *Cl_s = reinterpret_cast<float *>(smem + L.Cl);
  float *u_s = reinterpret_cast<float *>(smem + L.u);
  float *ell = reinterpret_cast<float *>(smem + L.ell);
  uint64_t *keys = reinterpret_cast<uint64_t *>(smem + L.keys);
  __shared__ int best_s, tie_s;
  __shared__ uint64_t wbest[HP_THREADS / 64];
  const int q = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t nb = (size_t)q * h.NH;
  int32_t *tok = h.tok + nb, *par = h.par + nb, *dep = h.dep + nb;
  int2 *gref = reinterpret_cast<int2 *>(h.gref) + nb;
  float *score = h.score + nb;
  uint64_t *pvg = h.pv + nb;
  const int ldu = p.r + 3 * p.s;
  const size_t slots = (size_t)h.Bcap + 1;
  float *Sq = h.S + (size_t)q * slots * p.s;
  const float *UHq = h.UH + (size_t)q * slots * ldu;
  const size_t tq = (size_t)q * p.D;

  // ---- round trip 1
  int nn = 1;
  int4 ex = make_int4(0, 0, 0, 0);   // step 0 expands the root (depth 0, score 0)
  if (p.t > 0) {
    nn = h.nnodes[q];
    ex = reinterpret_cast<const int4 *>(h.ex)[q];
  }
  const int nnb = min(h.NH, 1 + p.K * p.t);   // nn <= nnb
  for (int base = 0; base < nnb; base += 8 * HP_THREADS) {
    uint64_t v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = base + j * HP_THREADS + tid;
      v[j] = i < nnb ? pvg[i] : 0ull;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = base + j * HP_THREADS + tid;
      if (i < nnb) pv_s[i] = (i > 0 && i < nn) ? v[j] : 0ull;
    }
  }
  if (p.vec) {
    const uint32_t nUH = (uint32_t)(p.D * p.r * 4), nC = (uint32_t)(p.D * p.M * 4),
                   nU = (uint32_t)(p.r * 4);
    const __amdgpu_buffer_rsrc_t rU = heap_rsrc(p.uH + tq * p.r, nUH),
                                 rC = heap_rsrc(p.C + tq * p.M, nC),
                                 rL = heap_rsrc(p.Cl + tq * p.M, nC),
                                 rR = heap_rsrc(UHq + (size_t)p.t * ldu, nU);
    // the usual sizes in one batch of loads, the rest (if any) after it
    constexpr uint32_t BU = 4 * 16 * HP_THREADS, BC = 2 * 16 * HP_THREADS, BR = 16 * HP_THREADS;
    hu32x4 a[4], c[2], l[2], w;
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] = heap_ld16(rU, 16 * (tid + j * HP_THREADS));
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      c[j] = heap_ld16(rC, 16 * (tid + j * HP_THREADS));
      l[j] = heap_ld16(rL, 16 * (tid + j * HP_THREADS));
    }
    w = heap_ld16(rR, 16 * tid);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t o = 16 * (tid + j * HP_THREADS);
      if (o < nUH) *reinterpret_cast<hu32x4 *>(reinterpret_cast<uint8_t *>(uH_s) + o) = a[j];
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t o = 16 * (tid + j * HP_THREADS);
      if (o < nC) {
        *reinterpret_cast<hu32x4 *>(reinterpret_cast<uint8_t *>(C_s) + o) = c[j];
        *reinterpret_cast<hu32x4 *>(reinterpret_cast<uint8_t *>(Cl_s) + o) = l[j];
      }
    }
    if (16u * tid < nU) *reinterpret_cast<hu32x4 *>(reinterpret_cast<uint8_t *>(u_s) + 16 * tid) = w;
    heap_stage16<4>(reinterpret_cast<uint8_t *>(uH_s), rU, BU, nUH, tid);
    heap_stage16<2>(reinterpret_cast<uint8_t *>(C_s), rC, BC, nC, tid);
    heap_stage16<2>(reinterpret_cast<uint8_t *>(Cl_s), rL, BC, nC, tid);
    heap_stage16<1>(reinterpret_cast<uint8_t *>(u_s), rR, BR, nU, tid);
  } else {
    for (int k = tid; k < p.D * p.r; k += HP_THREADS) uH_s[k] = p.uH[tq * p.r + k];
    for (int k = tid; k < p.D * p.M; k += HP_THREADS) {
      C_s[k] = p.C[tq * p.M + k];
      Cl_s[k] = p.Cl[tq * p.M + k];
    }
    for (int k = tid; k < p.r; k += HP_THREADS) u_s[k] = UHq[(size_t)p.t * ldu + k];
  }
  if (p.t == 0) {
    if (tid == 0) {
      tok[0] = p.root[q];
      par[0] = -1;
      dep[0] = 0;
      score[0] = 0.f;
      gref[0] = make_int2(-1, 0);
      pvg[0] = 0ull;
      pv_s[0] = 0ull;
    }
    for (int k = tid; k < p.s; k += HP_THREADS) Sq[k] = p.S_root[(size_t)q * p.s + k];
  }
  __syncthreads();

  // ---- round trip 2: correction and children of node e
  const int e = ex.x;
  if (e >= 0) {
    const int dd = ex.y;
    for (int k = tid; k < p.r; k += HP_THREADS) u_s[k] += uH_s[dd * p.r + k];
    __syncthreads();
    const int *cq = C_s + dd * p.M;
    const float *clq = Cl_s + dd * p.M;
    if (p.vec) {
      // ell[j] = Cl[j] + W2[C[j]] . u: wl lanes per candidate, each over up
      // to 16 pieces of 16 bytes of the row, all in flight at once
      const int wl = p.wl, per = HP_THREADS / wl;
      const int ce = p.w2_bf16 ? 8 : 4;            // elements per piece
      const int nch = p.r / ce, cpl = (nch + wl - 1) / wl;
      const uint32_t rowb = (uint32_t)(p.r * (p.w2_bf16 ? 2 : 4));
      const __amdgpu_buffer_rsrc_t rW = heap_rsrc(p.W2, (uint32_t)p.V * rowb);
      for (int j0 = 0; j0 < p.M; j0 += per) {
        const int j = j0 + tid / wl, part = tid % wl;
        const int tk = j < p.M ? max(cq[j], 0) : 0;
        hu32x4 wv[16];
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (i < cpl) {
            const int c = part + wl * i;
            wv[i] = heap_ld16(rW, (j < p.M && c < nch) ? (uint32_t)tk * rowb + 16u * c : 0u);
          }
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (i < cpl) {
            const int c = part + wl * i;
            if (c < nch) {
              const float *uu = u_s + c * ce;
              if (p.w2_bf16) {
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                  acc += __uint_as_float(wv[i][x] << 16) * uu[2 * x];
                  acc += __uint_as_float(wv[i][x] & 0xFFFF0000u) * uu[2 * x + 1];
                }
              } else {
#pragma unroll
                for (int x = 0; x < 4; ++x) acc += __uint_as_float(wv[i][x]) * uu[x];
              }
            }
          }
        if (wl > 1) acc += xchg_f32<1>(acc);
        if (wl > 2) acc += xchg_f32<2>(acc);
        if (wl > 4) acc += xchg_f32<4>(acc);
        if (wl > 8) acc += xchg_f32<8>(acc);
        if (wl > 16) acc += xchg_f32<16>(acc);
        if (wl > 32) acc += xchg_f32<32>(acc);
        if (j < p.M && part == 0) ell[j] = clq[j] + acc;
      }
    } else {
      for (int j0 = 0; j0 < p.M; j0 += HP_THREADS / 8) {
        const int j = j0 + (tid >> 3), part = tid & 7;
        float acc = 0.f;
        if (j < p.M) {
          const int tk = max(cq[j], 0);
          if (p.w2_bf16) {
            const uint16_t *w = static_cast<const uint16_t *>(p.W2) + (size_t)tk * p.r;
            for (int k = part; k < p.r; k += 8) acc += bf16_bits_to_f32(w[k]) * u_s[k];
          } else {
            const float *w = static_cast<const float *>(p.W2) + (size_t)tk * p.r;
            for (int k = part; k < p.r; k += 8) acc += w[k] * u_s[k];
          }
        }
        acc += xchg_f32<1>(acc);
        acc += xchg_f32<2>(acc);
        acc += xchg_f32<4>(acc);
        if (j < p.M && part == 0) ell[j] = clq[j] + acc;
      }
    }
    __syncthreads();
    // log-softmax over the M candidates (wave 0), Top-K by rank
    if (wave == 0) {
      float m = -INFINITY;
      for (int j = lane; j < p.M; j += 64) m = fmaxf(m, ell[j]);
      m = wave_max_f32(m);
      float se = 0.f;
      for (int j = lane; j < p.M; j += 64) se += expf(ell[j] - m);
      const float lse = m + logf(wave_sum_f32(se));
      for (int j = lane; j < p.M; j += 64) keys[j] = make_key(ell[j] - lse, (uint32_t)cq[j]);
    }
    __syncthreads();
    const float se_score = __int_as_float(ex.z);
    for (int j = tid; j < p.M; j += HP_THREADS) {
      const uint64_t kj = keys[j];
      int rank = 0;
      for (int i = 0; i < p.M; ++i) rank += keys[i] > kj;
      if (rank < p.K) {
        const int c = nn + rank;
        const float sc = __fadd_rn(se_score, key_val(kj));
        const uint64_t v = pop_value(sc, dd + 1, p.beta);
        tok[c] = cq[j];
        par[c] = e;
        dep[c] = dd + 1;
        score[c] = sc;
        gref[c] = make_int2(j, p.t);   // e's expansion slot is t
        pvg[c] = v;
        pv_s[c] = v;
      }
    }
    nn += p.K;
    __syncthreads();
  }

  // ---- pop: arg-max of the pop values (LDS only); nodes that share the
  // maximum (equal key and depth) are ordered by token path (rare)
  uint64_t bk = 0ull;
  int bi = -1;
  bool dup = false;   // a second node of this thread has the same value
  for (int i = 1 + tid; i < nn; i += HP_THREADS) {
    const uint64_t k = pv_s[i];
    if (k == 0ull) continue;
    if (bi < 0 || k > bk) { bk = k; bi = i; dup = false; }
    else if (k == bk) dup = true;
  }
  const uint64_t wk = group_max_u64<64>(bk);
  if (lane == 0) wbest[wave] = wk;
  if (tid == 0) best_s = -1, tie_s = 0;
  __syncthreads();
  uint64_t top = wbest[0];
  for (int w = 1; w < HP_THREADS / 64; ++w) top = wbest[w] > top ? wbest[w] : top;
  if (bi >= 0 && bk == top)
    if (atomicAdd(&tie_s, dup ? 2 : 1) == 0) best_s = bi;
  __syncthreads();
  int best = best_s;
  if (tie_s > 1) {
    if (tid == 0) {
      int b = -1;
      for (int i = 1; i < nn; ++i)
        if (pv_s[i] == top && (b < 0 || heap_before(i, b, tok, par, dep, score, p.beta))) b = i;
      best_s = b;
    }
    __syncthreads();
    best = best_s;
  }
  float *Snew = Sq + (size_t)(p.t + 1) * p.s;
  const int db = best >= 0 ? pop_depth(top) : 0;
  const bool grow = best >= 0 && db < p.D;
  // ---- round trip 3: the popped node's candidate, parent slot and score
  int2 g = make_int2(0, 0);
  float sb = 0.f;
  if (grow) {
    g = gref[best];
    sb = score[best];
  }
  if (tid == 0) {
    h.pops[(size_t)q * h.Bcap + p.t] = best;
    h.nnodes[q] = nn;
    if (best >= 0) pvg[best] = 0ull;
    reinterpret_cast<int4 *>(h.ex)[q] =
        grow ? make_int4(best, db, __float_as_int(sb), 0) : make_int4(-1, 0, 0, 0);
  }
  if (!grow) {   // nothing to expand: the slot's product input is zeros
    for (int k = tid; k < p.s; k += HP_THREADS) Snew[k] = 0.f;
    return;
  }
  // ---- round trip 4: GRU step of the popped node (PyTorch GRUCell gates r, z, n)
  const float *gi = h.gi + ((tq + db - 1) * p.M + g.x) * 3 * p.s;
  const float *gh = p.markov ? p.b_hh : UHq + (size_t)g.y * ldu + p.r;
  const float *Sp = Sq + (size_t)g.y * p.s;
  auto cell = [&](float xr, float xz, float xn, float cr, float cz, float cn, float hp) {
    const float rg = 1.f / (1.f + expf(-(xr + cr)));
    const float zg = 1.f / (1.f + expf(-(xz + cz)));
    const float ng = tanhf(xn + rg * cn);
    return (1.f - zg) * ng + zg * hp;
  };
  if (p.vec) {
    for (int k4 = tid; k4 < p.s / 4; k4 += HP_THREADS) {
      const float4 xr = reinterpret_cast<const float4 *>(gi)[k4];
      const float4 xz = reinterpret_cast<const float4 *>(gi + p.s)[k4];
      const float4 xn = reinterpret_cast<const float4 *>(gi + 2 * p.s)[k4];
      float4 cr = make_float4(0.f, 0.f, 0.f, 0.f), cz = cr, cn = cr, hp = cr;
      if (gh) {
        cr = reinterpret_cast<const float4 *>(gh)[k4];
        cz = reinterpret_cast<const float4 *>(gh + p.s)[k4];
        cn = reinterpret_cast<const float4 *>(gh + 2 * p.s)[k4];
      }
      if (!p.markov) hp = reinterpret_cast<const float4 *>(Sp)[k4];
      float4 o;
      o.x = cell(xr.x, xz.x, xn.x, cr.x, cz.x, cn.x, hp.x);
      o.y = cell(xr.y, xz.y, xn.y, cr.y, cz.y, cn.y, hp.y);
      o.z = cell(xr.z, xz.z, xn.z, cr.z, cz.z, cn.z, hp.z);
      o.w = cell(xr.w, xz.w, xn.w, cr.w, cz.w, cn.w, hp.w);
      reinterpret_cast<float4 *>(Snew)[k4] = o;
    }
  } else {
    for (int k = tid; k < p.s; k += HP_THREADS) {
      const float cr = gh ? gh[k] : 0.f, cz = gh ? gh[p.s + k] : 0.f, cn = gh ? gh[2 * p.s + k] : 0.f;
      Snew[k] = cell(gi[k], gi[p.s + k], gi[2 * p.s + k], cr, cz, cn, p.markov ? 0.f : Sp[k]);
    }
  }
}

// Emission of the popped set: the root, then the popped nodes in canonical
// order (depth ascending, token path lexicographically ascending), parents
// re-indexed, the ancestor-or-self mask (same contract as the depth-wise
// round).
__global__ __launch_bounds__(HP_THREADS) void k_heap_emit(int B, int D, HeapBufs h, int32_t *otok,
                                                          int32_t *opar, int32_t *odep,
                                                          float *oscore, uint8_t *omask,
                                                          int32_t *on_nodes) {
  extern __shared__ __align__(16) uint8_t smem[];
  int *idx = reinterpret_cast<int *>(smem);   // [NH]: node -> position among the popped (or -1)
  int *sel = idx + h.NH;                      // [B]: popped node ids in pop order
  uint32_t *lk = reinterpret_cast<uint32_t *>(sel + B);   // [B] (parent rank << 18) | token
  int *rnk = reinterpret_cast<int *>(lk + B);             // [B] rank within its depth
  int *pos = rnk + B;                                     // [B] output row
  int *byd = pos + B;                                     // [B] popped ids grouped by depth
  int *ptok = byd + B;                                    // [B] the popped nodes' fields,
  int *ppar = ptok + B;                                   //     staged once
  int *pdep = ppar + B;
  float *pscore = reinterpret_cast<float *>(pdep + B);
  __shared__ int cnt[33], start[33], fill[33];
  __shared__ int nsel_s;
  const int q = blockIdx.x, tid = threadIdx.x;
  const size_t nb = (size_t)q * h.NH;
  const int32_t *pops = h.pops + (size_t)q * h.Bcap;
  const int N = B + 1;
  for (int i = tid; i < h.NH; i += HP_THREADS) idx[i] = -1;
  if (tid < 33) cnt[tid] = 0, fill[tid] = 0;
  if (tid == 0) nsel_s = B;
  __syncthreads();
  // the pops are a prefix: the first empty one ends it
  for (int i = tid; i < B; i += HP_THREADS)
    if (pops[i] < 0) atomicMin(&nsel_s, i);
  __syncthreads();
  const int nsel = nsel_s;
  for (int i = tid; i < nsel; i += HP_THREADS) {
    const int n = pops[i];
    sel[i] = n;
    idx[n] = i;
    ptok[i] = h.tok[nb + n];
    ppar[i] = h.par[nb + n];
    pdep[i] = h.dep[nb + n];
    pscore[i] = h.score[nb + n];
    atomicAdd(&cnt[pdep[i]], 1);
  }
  __syncthreads();
  if (tid == 0) {
    int a = 0;
    for (int d = 0; d <= 32; ++d) {
      start[d] = a;
      a += cnt[d];
    }
  }
  __syncthreads();
  for (int i = tid; i < nsel; i += HP_THREADS) {
    const int d = pdep[i];
    byd[start[d] + atomicAdd(&fill[d], 1)] = i;
  }
  __syncthreads();
  // ranks depth by depth: key = (rank of the parent << 18) | token
  for (int d = 1; d <= D; ++d) {
    for (int k = tid; k < cnt[d]; k += HP_THREADS) {
      const int i = byd[start[d] + k];
      const int pn = ppar[i];
      const uint32_t pr = pn == 0 ? 0u : (uint32_t)rnk[idx[pn]];
      lk[i] = (pr << 18) | (uint32_t)ptok[i];
    }
    __syncthreads();
    for (int k = tid; k < cnt[d]; k += HP_THREADS) {
      const int i = byd[start[d] + k];
      int r = 0;
      for (int m = 0; m < cnt[d]; ++m) r += lk[byd[start[d] + m]] < lk[i];
      rnk[i] = r;
      pos[i] = 1 + start[d] + r;
    }
    __syncthreads();
  }
  // outputs; the request's N x N mask bytes are cleared with 16-byte stores
  // where aligned
  int32_t *tq = otok + (size_t)q * N, *pq = opar + (size_t)q * N, *dq = odep + (size_t)q * N;
  float *sq = oscore + (size_t)q * N;
  uint8_t *mq = omask + (size_t)q * N * N;
  {
    const size_t nbytes = (size_t)N * N;
    const size_t head = (16 - (reinterpret_cast<uintptr_t>(mq) & 15)) & 15;
    const size_t h0 = head < nbytes ? head : nbytes;
    const size_t nvec = (nbytes - h0) / 16;
    for (size_t i = tid; i < h0; i += HP_THREADS) mq[i] = 0;
    uint4 *mv = reinterpret_cast<uint4 *>(mq + h0);
    for (size_t i = tid; i < nvec; i += HP_THREADS) mv[i] = make_uint4(0, 0, 0, 0);
    for (size_t i = h0 + nvec * 16 + tid; i < nbytes; i += HP_THREADS) mq[i] = 0;
  }
  for (int i = tid; i < N; i += HP_THREADS) {
    if (i == 0) {
      tq[0] = h.tok[nb];
      pq[0] = -1;
      dq[0] = 0;
      sq[0] = 0.f;
    } else if (i > nsel) {
      tq[i] = -1;
      pq[i] = -1;
      dq[i] = -1;
      sq[i] = -INFINITY;
    }
  }
  __syncthreads();
  for (int i = tid; i < nsel; i += HP_THREADS) {
    const int o = pos[i];
    const int pn = ppar[i];
    tq[o] = ptok[i];
    pq[o] = pn == 0 ? 0 : pos[idx[pn]];
    dq[o] = pdep[i];
    sq[o] = pscore[i];
    uint8_t *row = mq + (size_t)o * N;
    row[0] = 1;
    for (int a = i; a >= 0; a = ppar[a] == 0 ? -1 : idx[ppar[a]]) row[pos[a]] = 1;
  }
  if (tid == 0) {
    mq[0] = 1;
    on_nodes[q] = nsel + 1;
  }
}

}  // namespace

size_t heap_step_smem(int NH, int D, int M, int r) { return heap_step_layout(NH, D, M, r).total; }
size_t heap_emit_smem(int NH, int B) { return (size_t)NH * 4 + (size_t)B * 4 * 9; }

hipError_t launch_heap_step(const HeapStepArgs &a, hipStream_t st) {
  HeapStepParams p{};
  p.t = a.t; p.B = a.B; p.D = a.D; p.M = a.M; p.K = a.K; p.s = a.s; p.r = a.r;
  p.markov = a.markov; p.beta = a.beta; p.W2 = a.W2; p.w2_bf16 = a.w2_bf16;
  p.C = a.C; p.Cl = a.Cl; p.uH = a.uH; p.root = a.root; p.S_root = a.S_root; p.b_hh = a.b_hh;
  p.h = a.h;
  p.V = a.V;
  // 16-byte loads where every row and table allows them
  const auto al16 = [](const void *x) { return (reinterpret_cast<uintptr_t>(x) & 15) == 0; };
  int wl = 1;
  while (wl < 64 && (size_t)a.M * wl * 2 <= HP_THREADS) wl *= 2;
  const int ce = a.w2_bf16 ? 8 : 4;
  const size_t w2_bytes = (size_t)a.V * a.r * (a.w2_bf16 ? 2 : 4);
  p.wl = wl;
  p.vec = a.r % ce == 0 && a.s % 4 == 0 && (a.D * a.M) % 4 == 0 &&
          (a.r / ce + wl - 1) / wl <= 16 && w2_bytes < (1u << 31) && al16(a.W2) &&
          al16(a.C) && al16(a.Cl) && al16(a.uH) && (!a.b_hh || al16(a.b_hh)) && al16(a.h.S) &&
          al16(a.h.UH) && al16(a.h.gi);
  hipLaunchKernelGGL(k_heap_step, dim3(a.batch), dim3(HP_THREADS),
                     heap_step_smem(a.h.NH, a.D, a.M, a.r), st, p);
  return hipGetLastError();
}

hipError_t launch_heap_emit(int batch, int B, int D, const HeapBufs &h, int32_t *tok,
                            int32_t *parent, int32_t *depth, float *score, uint8_t *mask,
                            int32_t *n_nodes, hipStream_t st) {
  hipLaunchKernelGGL(k_heap_emit, dim3(batch), dim3(HP_THREADS), heap_emit_smem(h.NH, B), st, B, D,
                     h, tok, parent, depth, score, mask, n_nodes);
  return hipGetLastError();
}

hipError_t heap_prepare(size_t lds_bytes) {
  hipError_t e = set_lds_limit(reinterpret_cast<const void *>(&k_heap_step), lds_bytes);
  if (e == hipSuccess) e = set_lds_limit(reinterpret_cast<const void *>(&k_heap_emit), lds_bytes);
  return e;
}

}  // namespace dtree
