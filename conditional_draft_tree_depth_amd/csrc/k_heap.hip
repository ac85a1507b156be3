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
  int t, B, D, M, K, s, r, markov;
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

__global__ __launch_bounds__(HP_THREADS) void k_heap_step(HeapStepParams p) {
  extern __shared__ __align__(16) uint8_t smem[];
  float *u_s = reinterpret_cast<float *>(smem);   // [r] (padded to even)
  float *ell = u_s + ((p.r + 1) & ~1);            // [M] (padded to even)
  uint64_t *keys = reinterpret_cast<uint64_t *>(ell + ((p.M + 1) & ~1));   // [M]
  __shared__ int best_s[HP_THREADS];
  __shared__ int nn_s;
  const int q = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const HeapBufs &h = p.h;
  const size_t nb = (size_t)q * h.NH;
  int32_t *tok = h.tok + nb, *par = h.par + nb, *dep = h.dep + nb, *cand = h.cand + nb,
          *slot = h.slot + nb;
  float *score = h.score + nb;
  uint8_t *popped = h.popped + nb;
  const int ldu = p.r + 3 * p.s;
  const size_t slots = (size_t)h.Bcap + 1;
  float *Sq = h.S + (size_t)q * slots * p.s;
  const float *UHq = h.UH + (size_t)q * slots * ldu;

  int e = -1, eslot = 0;
  if (p.t == 0) {
    if (tid == 0) {
      tok[0] = p.root[q];
      par[0] = -1;
      dep[0] = 0;
      score[0] = 0.f;
      cand[0] = -1;
      slot[0] = 0;
      popped[0] = 1;
      nn_s = 1;
    }
    for (int k = tid; k < p.s; k += HP_THREADS) Sq[k] = p.S_root[(size_t)q * p.s + k];
    e = 0;
  } else {
    if (tid == 0) nn_s = h.nnodes[q];
    if (h.expanded[(size_t)q * h.Bcap + p.t - 1]) {
      e = h.pops[(size_t)q * h.Bcap + p.t - 1];
      eslot = p.t;
    }
  }
  __syncthreads();
  int nn = nn_s;

  // ---- correction and children of node e (its state product is in slot eslot)
  if (e >= 0) {
    const int dd = dep[e];
    const float *ur = UHq + (size_t)eslot * ldu;
    const float *uh = p.uH + ((size_t)q * p.D + dd) * p.r;
    for (int k = tid; k < p.r; k += HP_THREADS) u_s[k] = ur[k] + uh[k];
    __syncthreads();
    const int32_t *cq = p.C + ((size_t)q * p.D + dd) * p.M;
    const float *clq = p.Cl + ((size_t)q * p.D + dd) * p.M;
    for (int j = wave; j < p.M; j += HP_THREADS / 64) {
      const int tk = cq[j] < 0 ? 0 : cq[j];
      float acc = 0.f;
      if (p.w2_bf16) {
        const uint16_t *w = static_cast<const uint16_t *>(p.W2) + (size_t)tk * p.r;
        for (int k = lane; k < p.r; k += 64) acc += bf16_bits_to_f32(w[k]) * u_s[k];
      } else {
        const float *w = static_cast<const float *>(p.W2) + (size_t)tk * p.r;
        for (int k = lane; k < p.r; k += 64) acc += w[k] * u_s[k];
      }
      acc = wave_sum_f32(acc);
      if (lane == 0) ell[j] = clq[j] + acc;
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
    for (int j = tid; j < p.M; j += HP_THREADS) {
      const uint64_t kj = keys[j];
      int rank = 0;
      for (int i = 0; i < p.M; ++i) rank += keys[i] > kj;
      if (rank < p.K) {
        const int c = nn + rank;
        tok[c] = cq[j];
        par[c] = e;
        dep[c] = dd + 1;
        score[c] = __fadd_rn(score[e], key_val(kj));
        cand[c] = j;
        slot[c] = -1;
        popped[c] = 0;
      }
    }
    nn += p.K;
    __syncthreads();   // children visible to the whole workgroup
  }

  // ---- pop: arg-max over the open nodes
  int best = -1;
  for (int i = 1 + tid; i < nn; i += HP_THREADS)
    if (!popped[i] && (best < 0 || heap_before(i, best, tok, par, dep, score, p.beta))) best = i;
  best_s[tid] = best;
  __syncthreads();
  for (int w = HP_THREADS / 2; w > 0; w >>= 1) {
    if (tid < w) {
      const int a = best_s[tid], b = best_s[tid + w];
      if (b >= 0 && (a < 0 || heap_before(b, a, tok, par, dep, score, p.beta))) best_s[tid] = b;
    }
    __syncthreads();
  }
  best = best_s[0];
  const size_t pt = (size_t)q * h.Bcap + p.t;
  float *Snew = Sq + (size_t)(p.t + 1) * p.s;
  const bool grow = best >= 0 && dep[best] < p.D;
  if (tid == 0) {
    h.pops[pt] = best;
    h.expanded[pt] = grow ? 1 : 0;
    h.nnodes[q] = nn;
    if (best >= 0) popped[best] = 1;
    if (grow) slot[best] = p.t + 1;
  }
  if (!grow) {   // nothing to expand: the slot's product input is zeros
    for (int k = tid; k < p.s; k += HP_THREADS) Snew[k] = 0.f;
    return;
  }
  // ---- GRU step of the popped node (PyTorch GRUCell gates r, z, n)
  const int pn = par[best];
  const int ps = pn == 0 ? 0 : slot[pn];
  const float *gi = h.gi + (((size_t)q * p.D + dep[best] - 1) * p.M + cand[best]) * 3 * p.s;
  const float *gh = p.markov ? p.b_hh : UHq + (size_t)ps * ldu + p.r;
  const float *Sp = Sq + (size_t)ps * p.s;
  for (int k = tid; k < p.s; k += HP_THREADS) {
    const float cr = gh ? gh[k] : 0.f, cz = gh ? gh[p.s + k] : 0.f, cn = gh ? gh[2 * p.s + k] : 0.f;
    const float rg = 1.f / (1.f + expf(-(gi[k] + cr)));
    const float zg = 1.f / (1.f + expf(-(gi[p.s + k] + cz)));
    const float ng = tanhf(gi[2 * p.s + k] + rg * cn);
    const float hp = p.markov ? 0.f : Sp[k];
    Snew[k] = (1.f - zg) * ng + zg * hp;
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
  __shared__ int cnt[33], start[33], fill[33];
  __shared__ int nsel_s;
  const int q = blockIdx.x, tid = threadIdx.x;
  const size_t nb = (size_t)q * h.NH;
  const int32_t *tok = h.tok + nb, *par = h.par + nb, *dep = h.dep + nb;
  const float *score = h.score + nb;
  const int32_t *pops = h.pops + (size_t)q * h.Bcap;
  const int N = B + 1;
  for (int i = tid; i < h.NH; i += HP_THREADS) idx[i] = -1;
  if (tid < 33) cnt[tid] = 0, fill[tid] = 0;
  if (tid == 0) {
    int n = 0;
    while (n < B && pops[n] >= 0) ++n;
    nsel_s = n;
  }
  __syncthreads();
  const int nsel = nsel_s;
  for (int i = tid; i < nsel; i += HP_THREADS) {
    sel[i] = pops[i];
    idx[pops[i]] = i;
    atomicAdd(&cnt[dep[pops[i]]], 1);
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
    const int d = dep[sel[i]];
    byd[start[d] + atomicAdd(&fill[d], 1)] = i;
  }
  __syncthreads();
  // ranks depth by depth: key = (rank of the parent << 18) | token
  for (int d = 1; d <= D; ++d) {
    for (int k = tid; k < cnt[d]; k += HP_THREADS) {
      const int i = byd[start[d] + k];
      const int pn = par[sel[i]];
      const uint32_t pr = pn == 0 ? 0u : (uint32_t)rnk[idx[pn]];
      lk[i] = (pr << 18) | (uint32_t)tok[sel[i]];
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
  // outputs
  int32_t *tq = otok + (size_t)q * N, *pq = opar + (size_t)q * N, *dq = odep + (size_t)q * N;
  float *sq = oscore + (size_t)q * N;
  uint8_t *mq = omask + (size_t)q * N * N;
  for (size_t i = tid; i < (size_t)N * N; i += HP_THREADS) mq[i] = 0;
  for (int i = tid; i < N; i += HP_THREADS) {
    if (i == 0) {
      tq[0] = tok[0];
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
    const int n = sel[i], o = pos[i];
    const int pn = par[n];
    tq[o] = tok[n];
    pq[o] = pn == 0 ? 0 : pos[idx[pn]];
    dq[o] = dep[n];
    sq[o] = score[n];
    uint8_t *row = mq + (size_t)o * N;
    row[0] = 1;
    for (int a = n; a != 0; a = par[a]) row[pos[idx[a]]] = 1;
  }
  if (tid == 0) {
    mq[0] = 1;
    on_nodes[q] = nsel + 1;
  }
}

}  // namespace

size_t heap_step_smem(int r, int M) {
  return (size_t)((r + 1) & ~1) * 4 + (size_t)((M + 1) & ~1) * 4 + (size_t)M * 8;
}
size_t heap_emit_smem(int NH, int B) { return (size_t)NH * 4 + (size_t)B * 4 * 5; }

hipError_t launch_heap_step(const HeapStepArgs &a, hipStream_t st) {
  HeapStepParams p{};
  p.t = a.t; p.B = a.B; p.D = a.D; p.M = a.M; p.K = a.K; p.s = a.s; p.r = a.r;
  p.markov = a.markov; p.beta = a.beta; p.W2 = a.W2; p.w2_bf16 = a.w2_bf16;
  p.C = a.C; p.Cl = a.Cl; p.uH = a.uH; p.root = a.root; p.S_root = a.S_root; p.b_hh = a.b_hh;
  p.h = a.h;
  hipLaunchKernelGGL(k_heap_step, dim3(a.batch), dim3(HP_THREADS), heap_step_smem(a.r, a.M), st, p);
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
