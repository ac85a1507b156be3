// K4: deferred pruning and the compact verification tree.
//
// DARTree page, Methodology 2: after the superarbol is built, ONE global
// Top-B over all its materialised prefixes (root excluded) replaces the
// sequential best-first heap; with a non-positive depth bonus beta the key
// score + beta * depth never increases from a node to its children, which
// is why (Lemma 1) the selected set equals the heap's and is closed under
// parents.  The selected nodes are emitted in canonical order (depth, then
// token path), parents re-indexed, with the ancestor-or-self mask that
// tree-attention verification uses ("Resumen Técnico: DominoTree", Main
// components 5).  The closure is checked; a violation sets status bit 0.
//
// One workgroup per request.  Selection: up to TB_RANK_MAX nodes, the rank
// of every node among all keys is counted directly (a few threads per node);
// larger superarbols find the B-th largest key by radix passes and rank only
// the selected keys among themselves.  The mask comes from each
// selected node's ancestor at every depth: j is an ancestor-or-self of i iff
// depth(j) <= depth(i) and i's ancestor at depth(j) is j.
#include "common.hpp"
#include "kernels.hpp"

namespace dtree {

constexpr int TB_THREADS = 1024;
constexpr int TB_MAXDEP = 32;   // depths 0 .. 31
constexpr int TB_RANK_MAX = 256;   // superarbols up to this size: rank counting

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

// LDS: keys (selection), later the canonical scratch, then the ancestor
// table; ids (sorted order or selection ranks); the rest.
struct TBLayout {
  size_t keys, ids, map, onode, opar, odep, canon, hist, skey, total;
};

__host__ __device__ inline TBLayout tb_layout(int NT, int B) {
  const int Nsa = NT - 1;
  int npad = 1;
  while (npad < Nsa) npad <<= 1;
  const int N = B + 1;
  TBLayout L;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o += (bytes + 15) & ~(size_t)15; return at; };
  const size_t kb = (size_t)npad * 8, ab = (size_t)N * TB_MAXDEP * 2;
  L.keys = take(kb > ab ? kb : ab);
  L.ids = take((size_t)npad * 4);
  L.map = take((size_t)NT * 2);
  L.onode = take((size_t)N * 4);
  L.opar = take((size_t)N * 4);
  L.odep = take((size_t)N * 4);
  L.canon = take((size_t)N * 4);
  L.hist = take((size_t)(256 + 8) * 4);   // radix histogram, then scalars
  L.skey = take((size_t)N * 8);           // selected keys (radix path)
  L.total = o;
  return L;
}

__global__ __launch_bounds__(TB_THREADS) void k_topb_emit(int NT, int B, float beta, int Bmax,
                                                          TreeBufs t, int32_t *__restrict__ otok,
                                                          int32_t *__restrict__ opar,
                                                          int32_t *__restrict__ odep,
                                                          float *__restrict__ oscore,
                                                          uint8_t *__restrict__ omask,
                                                          int32_t *__restrict__ on_nodes) {
  extern __shared__ __align__(16) uint8_t smem[];
  const TBLayout L = tb_layout(NT, B);
  const int q = blockIdx.x, tid = threadIdx.x;
  const int Nsa = NT - 1;
  const int Bsel = B < Nsa ? B : Nsa;
  const int npad = next_pow2(Nsa > 1 ? Nsa : 1);
  const int N = B + 1;
  const int nn = Bsel + 1;
  const size_t nb = (size_t)q * t.NT;   // workspace stride (caps), NT = this round's nodes

  uint64_t *keys = reinterpret_cast<uint64_t *>(smem + L.keys);   // [npad]
  int32_t *ids = reinterpret_cast<int32_t *>(smem + L.ids);       // [npad] sorted order
  int32_t *rank = ids;                                            // [npad] or selection ranks
  int2 *cpos = reinterpret_cast<int2 *>(smem + L.keys);           // [Bsel] (node, position)
  int16_t *map = reinterpret_cast<int16_t *>(smem + L.map);       // [NT] node -> out index
  int32_t *onode = reinterpret_cast<int32_t *>(smem + L.onode);   // [N] out -> node
  int32_t *opar_s = reinterpret_cast<int32_t *>(smem + L.opar);   // [N]
  int32_t *odep_s = reinterpret_cast<int32_t *>(smem + L.odep);   // [N]
  uint32_t *canon = reinterpret_cast<uint32_t *>(smem + L.canon); // [N] (depth, path) keys
  int16_t *anc = reinterpret_cast<int16_t *>(smem + L.keys);      // [N][TB_MAXDEP], last

  // selection keys: fp32 key = score + beta*depth, rounded after each op
  for (int i = tid; i < npad; i += TB_THREADS) {
    uint64_t k = 0;
    if (i < Nsa) {
      const int n = i + 1;
      const int dep = t.n_dep[nb + n];
      const float key = __fadd_rn(t.n_score[nb + n], __fmul_rn(beta, (float)dep));
      k = make_key(key, ((uint32_t)dep << 27) | t.n_lex[nb + n]);
    }
    keys[i] = k;
    ids[i] = i + 1;
  }
  for (int i = tid; i < NT; i += TB_THREADS) map[i] = -1;
  __syncthreads();

  // the selected nodes in selection order: onode[1 + rank] (keys are distinct)
  if (Nsa > TB_RANK_MAX) {
    // The Bsel-th largest key by radix passes of 8 bits, most significant
    // first: each pass counts the digits of the keys that still match the
    // prefix found so far and keeps the digit where the count from the top
    // reaches the number of keys still wanted.  The keys >= it are exactly
    // the selection; their order comes from ranks among them.
    uint32_t *hist = reinterpret_cast<uint32_t *>(smem + L.hist);
    int *ctl = reinterpret_cast<int *>(hist + 256);
    uint64_t *skey = reinterpret_cast<uint64_t *>(smem + L.skey);
    const int lane = tid & 63;
    uint64_t prefix = 0, pmask = 0;
    int need = Bsel;
    for (int b = tid; b < 256; b += TB_THREADS) hist[b] = 0u;
    __syncthreads();
    for (int shift = 56; shift >= 0; shift -= 8) {
      for (int i = tid; i < Nsa; i += TB_THREADS) {
        const uint64_t k = keys[i];
        if ((k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid < 64) {
        // lane l: digits 255 - 4l .. 252 - 4l (counts from the top), then
        // clears them for the next pass
        uint32_t c[4], sum = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          c[j] = hist[255 - 4 * lane - j];
          hist[255 - 4 * lane - j] = 0u;
          sum += c[j];
        }
        uint32_t before = (uint32_t)wave_scan_add((int)sum) - sum;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (before < (uint32_t)need && before + c[j] >= (uint32_t)need) {
            ctl[0] = 255 - 4 * lane - j;
            ctl[1] = (int)before;
            ctl[2] = (int)c[j];
          }
          before += c[j];
        }
      }
      __syncthreads();
      prefix |= (uint64_t)(uint32_t)ctl[0] << shift;
      pmask |= 0xFFull << shift;
      need -= ctl[1];
      // every key left in this digit's bucket is wanted: the selection is
      // the keys whose masked value reaches the prefix
      if (ctl[2] == need) break;
    }
    __syncthreads();
    if (tid == 0) ctl[2] = 0;
    __syncthreads();
    for (int i = tid; i < Nsa; i += TB_THREADS)
      if ((keys[i] & pmask) >= prefix) {
        const int at = atomicAdd(&ctl[2], 1);
        if (at < Bsel) {   // (exactly Bsel: the keys are distinct)
          skey[at] = keys[i];
          ids[at] = i + 1;
        }
      }
    __syncthreads();
    for (int i = tid; i < Bsel; i += TB_THREADS) {
      const uint64_t k = skey[i];
      int rk = 0;
      for (int j = 0; j < Bsel; ++j) rk += skey[j] > k ? 1 : 0;
      if (rk < Bsel) onode[1 + rk] = ids[i];
    }
  } else {
    int tpn = 1;   // threads per node, a power of two
    while (tpn * 2 * Nsa <= TB_THREADS && tpn < 16) tpn *= 2;
    const int i = tid / tpn, part = tid & (tpn - 1);
    const uint64_t ki = i < Nsa ? keys[i] : 0ull;
    int cnt = 0;
    const int per = (Nsa + tpn - 1) / tpn, j0 = part * per, j1 = min(Nsa, j0 + per);
    int j = j0;
    for (; j + 8 <= j1; j += 8) {
      uint64_t v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = keys[j + u];
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < 8; ++u) cnt += v[u] > ki;
    }
    for (; j < j1; ++j) cnt += keys[j] > ki;
    // the tpn threads of a node are adjacent lanes
    if (tpn >= 2) cnt += (int)xchg_u32<1>((uint32_t)cnt);
    if (tpn >= 4) cnt += (int)xchg_u32<2>((uint32_t)cnt);
    if (tpn >= 8) cnt += (int)xchg_u32<4>((uint32_t)cnt);
    if (tpn >= 16) cnt += (int)xchg_u32<8>((uint32_t)cnt);
    if (i < Nsa && part == 0) rank[i] = cnt;
    __syncthreads();
    for (int i2 = tid; i2 < Nsa; i2 += TB_THREADS)
      if (rank[i2] < Bsel) onode[1 + rank[i2]] = i2 + 1;
  }
  __syncthreads();

  // canonical order of the selected nodes: (depth, lexicographic path)
  for (int i = tid; i < Bsel; i += TB_THREADS) {
    const int n = onode[1 + i];
    canon[i] = ((uint32_t)t.n_dep[nb + n] << 27) | t.n_lex[nb + n];
    t.sel[(size_t)q * Bmax + i] = n;
  }
  for (int i = Bsel + tid; i < Bmax; i += TB_THREADS) t.sel[(size_t)q * Bmax + i] = -1;
  __syncthreads();
  // canonical position of each selected node (the keys are no longer needed)
  for (int i = tid; i < Bsel; i += TB_THREADS) {
    const uint32_t ci = canon[i];
    int rk = 0;
    for (int j = 0; j < Bsel; ++j) rk += canon[j] < ci;
    const int n = onode[1 + i];
    cpos[i] = make_int2(n, 1 + rk);
    map[n] = (int16_t)(1 + rk);
  }
  __syncthreads();
  for (int i = tid; i < Bsel; i += TB_THREADS) onode[cpos[i].y] = cpos[i].x;
  if (tid == 0) { map[0] = 0; onode[0] = 0; }
  __syncthreads();

  // outputs, parent re-indexing and the closure check
  for (int i = tid; i < N; i += TB_THREADS) {
    const size_t o = (size_t)q * N + i;
    if (i < nn) {
      const int n = onode[i];
      const int pn = t.n_par[nb + n];
      int pi = -1;
      if (i > 0) {
        pi = map[pn];
        if (pi < 0) atomicOr(t.status, 1u);
      }
      const int dn = t.n_dep[nb + n];
      otok[o] = t.n_tok[nb + n];
      opar[o] = pi;
      odep[o] = dn;
      oscore[o] = t.n_score[nb + n];
      opar_s[i] = pi;
      odep_s[i] = min(dn, TB_MAXDEP - 1);
    } else {
      otok[o] = -1; opar[o] = -1; odep[o] = -1; oscore[o] = -INFINITY;
      opar_s[i] = -1;
      odep_s[i] = -1;
    }
  }
  if (tid == 0) on_nodes[q] = nn;
  for (int i = tid; i < N * TB_MAXDEP; i += TB_THREADS) anc[i] = -1;
  __syncthreads();

  // ancestor of every emitted node at each depth on its path (parents come
  // first in canonical order, so the walk ends at the root)
  for (int i = tid; i < nn; i += TB_THREADS) {
    int x = i, steps = 0;
    while (x >= 0 && steps < TB_MAXDEP) {
      anc[i * TB_MAXDEP + odep_s[x]] = (int16_t)x;
      x = x > 0 ? opar_s[x] : -1;
      ++steps;
    }
  }
  __syncthreads();
  // mask[i][j] = 1 iff j is i or an ancestor of i
  uint8_t *mq = omask + (size_t)q * N * N;
  for (int e = tid; e < N * N; e += TB_THREADS) {
    const int i = e / N, j = e - i * N;
    uint8_t v = 0;
    if (i < nn && j < nn) {
      const int dj = odep_s[j];
      v = (dj <= odep_s[i] && anc[i * TB_MAXDEP + dj] == j) ? 1 : 0;
    }
    mq[e] = v;
  }
}

size_t topb_smem(int NT, int B) { return tb_layout(NT, B).total; }

hipError_t topb_prepare(size_t smem) {
  return hipFuncSetAttribute(reinterpret_cast<const void *>(&k_topb_emit),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
}

hipError_t launch_topb_emit(int b, int NT, int B, float beta, int Bmax, const TreeBufs &t,
                            int32_t *tok, int32_t *parent, int32_t *depth, float *score,
                            uint8_t *mask, int32_t *n_nodes, hipStream_t st) {
  hipLaunchKernelGGL(k_topb_emit, dim3(b), dim3(TB_THREADS), topb_smem(NT, B), st, NT, B, beta,
                     Bmax, t, tok, parent, depth, score, mask, n_nodes);
  return hipGetLastError();
}

}  // namespace dtree
