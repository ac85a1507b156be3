// K4: deferred pruning and the compact verification tree.
//
// DARTree page, Metodología 2: after the superarbol is built, ONE global
// Top-B over all its materialised prefixes (root excluded) replaces the
// sequential best-first heap; with a non-positive depth bonus beta the key
// score + beta * depth never increases from a node to its children, which
// is why (Lemma 1) the selected set equals the heap's and is closed under
// parents.  The selected nodes are emitted in canonical order (depth, then
// token path), parents re-indexed, with the ancestor-or-self mask that
// tree-attention verification uses ("Resumen Técnico: DominoTree",
// Componentes Principales 5).  The closure is checked; a violation sets status bit 0.
//
// One workgroup per request.  Selection: up to TB_RANK_MAX nodes, the rank
// of every node among all keys is counted directly (a few threads per node);
// larger superarbols find the B-th largest key by radix passes and rank only
// the selected keys among themselves.  The mask is built as a bitmap in
// LDS, band of rows by band: each emitted node walks its parent chain and
// sets its row's bits, then the band is written out with aligned 16-byte
// stores (single bytes only where a band's edge is unaligned).
#include "common.hpp"
#include "kernels.hpp"

namespace dtree {

constexpr int TB_THREADS = 1024;
constexpr int TB_MAXDEP = 32;   // depths 0 .. 31: a parent chain has at most 32 nodes
constexpr int TB_RANK_MAX = 256;   // superarbols up to this size: rank counting

// low 4 bits of b as 4 bytes of 0/1 (bit k -> byte k): the product puts a
// copy of bit k at bit 7m + k of term m, and only m = k lands on bit 8m
__device__ __forceinline__ uint32_t spread4(uint32_t b) {
  return ((b & 15u) * 0x00204081u) & 0x01010101u;
}

// LDS: keys (selection), later the canonical scratch, then the mask bitmap
// of one band of rows; ids (sorted order or selection ranks); the rest.
struct TBLayout {
  size_t keys, ids, map, onode, opar, canon, hist, skey, total;
  int band_rows;   // mask rows per bitmap band
};

__host__ __device__ inline TBLayout tb_layout(int NT, int B) {
  const int Nsa = NT - 1;
  int npad = 1;
  while (npad < Nsa) npad <<= 1;
  const int N = B + 1;
  TBLayout L;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o += (bytes + 15) & ~(size_t)15; return at; };
  // at least 64 bytes per emitted row: bands of at least 512 rows
  const size_t kb = (size_t)npad * 8, ab = (size_t)N * 64 + 64;
  const size_t rb = kb > ab ? kb : ab;
  L.keys = take(rb);
  const size_t bits = rb * 8 - 64;   // two spare words for the 16-bit reads
  L.band_rows = (int)(bits / (size_t)N < (size_t)N ? bits / (size_t)N : (size_t)N);
  L.ids = take((size_t)npad * 4);
  L.map = take((size_t)NT * 2);
  L.onode = take((size_t)N * 4);
  L.opar = take((size_t)N * 4);
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
  uint32_t *canon = reinterpret_cast<uint32_t *>(smem + L.canon); // [N] (depth, path) keys
  uint32_t *bm = reinterpret_cast<uint32_t *>(smem + L.keys);     // mask bitmap band, last

  // selection keys: fp32 key = score + beta*depth, rounded after each op
  // (the node fields of up to 8 strides loaded before any is used)
  constexpr int KB_UNROLL = 8;
  for (int i0 = tid; i0 < npad; i0 += TB_THREADS * KB_UNROLL) {
    int dep[KB_UNROLL];
    float sc[KB_UNROLL];
    uint32_t lex[KB_UNROLL];
#pragma unroll
    for (int u = 0; u < KB_UNROLL; ++u) {
      const int i = i0 + u * TB_THREADS;
      dep[u] = 0; sc[u] = 0.f; lex[u] = 0u;
      if (i < Nsa) {
        dep[u] = t.n_dep[nb + i + 1];
        sc[u] = t.n_score[nb + i + 1];
        lex[u] = t.n_lex[nb + i + 1];
      }
    }
#pragma unroll
    for (int u = 0; u < KB_UNROLL; ++u) {
      const int i = i0 + u * TB_THREADS;
      if (i < npad) {
        uint64_t k = 0;
        if (i < Nsa) {
          const float key = __fadd_rn(sc[u], __fmul_rn(beta, (float)dep[u]));
          k = make_key(key, ((uint32_t)dep[u] << 27) | lex[u]);
        }
        keys[i] = k;
        ids[i] = i + 1;
      }
    }
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
      // the keys' leading digits are mostly equal (scores of one range):
      // the lanes sharing the first active lane's digit add once, together
      for (int i0 = tid - lane; i0 < Nsa; i0 += TB_THREADS) {
        const int i = i0 + lane;
        const uint64_t k = i < Nsa ? keys[i] : 0ull;
        const bool act = i < Nsa && (k & pmask) == prefix;
        const uint32_t dg = (uint32_t)(k >> shift) & 255u;
        const uint64_t live = __ballot(act);
        if (live) {
          const int lead = (int)__builtin_ctzll(live);
          const uint32_t ld = (uint32_t)__shfl((int)dg, lead);
          const uint64_t same = __ballot(act && dg == ld);
          if (lane == lead) atomicAdd(&hist[ld], (uint32_t)__popcll(same));
          if (act && dg != ld) atomicAdd(&hist[dg], 1u);
        }
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
    const int tpn = split_width(Bsel, TB_THREADS);
    const int part = tid & (tpn - 1);
    for (int base = 0; base < Bsel; base += TB_THREADS / tpn) {
      const int i = base + tid / tpn;
      const uint64_t k = i < Bsel ? skey[i] : 0ull;
      int rk = i < Bsel ? count_split<true>(skey, Bsel, k, part, tpn) : 0;
      rk = sum_adjacent(rk, tpn);
      if (i < Bsel && part == 0 && rk < Bsel) {
        onode[1 + rk] = ids[i];
        canon[rk] = key_tie(k);
      }
    }
  } else {
    const int tpn = split_width(Nsa, TB_THREADS);   // Nsa <= TB_RANK_MAX: one pass
    const int i = tid / tpn, part = tid & (tpn - 1);
    const uint64_t ki = i < Nsa ? keys[i] : 0ull;
    int cnt = i < Nsa ? count_split<true>(keys, Nsa, ki, part, tpn) : 0;
    cnt = sum_adjacent(cnt, tpn);
    if (i < Nsa && part == 0) rank[i] = cnt;
    __syncthreads();
    for (int i2 = tid; i2 < Nsa; i2 += TB_THREADS)
      if (rank[i2] < Bsel) {
        onode[1 + rank[i2]] = i2 + 1;
        canon[rank[i2]] = key_tie(keys[i2]);
      }
  }
  __syncthreads();

  // canonical order of the selected nodes: (depth, lexicographic path), the
  // tie field of their keys (canon, in selection order); the node fields of
  // each thread's first selected node load while the positions are counted
  int my_par = 0, my_tok = 0;
  float my_sc = 0.f;
  if (tid < Bsel) {
    const int n = onode[1 + tid];
    my_par = t.n_par[nb + n];
    my_tok = t.n_tok[nb + n];
    my_sc = t.n_score[nb + n];
  }
  for (int i = tid; i < Bsel; i += TB_THREADS) t.sel[(size_t)q * Bmax + i] = onode[1 + i];
  for (int i = Bsel + tid; i < Bmax; i += TB_THREADS) t.sel[(size_t)q * Bmax + i] = -1;
  if (tid == 0) map[0] = 0;
  {
    const int tpn = split_width(Bsel, TB_THREADS);
    const int part = tid & (tpn - 1);
    for (int base = 0; base < Bsel; base += TB_THREADS / tpn) {
      const int i = base + tid / tpn;
      const uint32_t ci = i < Bsel ? canon[i] : 0u;
      int rk = i < Bsel ? count_split<false>(canon, Bsel, ci, part, tpn) : 0;
      rk = sum_adjacent(rk, tpn);
      if (i < Bsel && part == 0) {
        const int n = onode[1 + i];
        cpos[i] = make_int2(n, 1 + rk);
        map[n] = (int16_t)(1 + rk);
      }
    }
  }
  __syncthreads();

  // outputs at the canonical positions, parent re-indexing and the closure
  // check (slot 0: the root)
  if (tid == 0) {
    const size_t o = (size_t)q * N;
    otok[o] = t.n_tok[nb];
    opar[o] = -1;
    odep[o] = t.n_dep[nb];
    oscore[o] = t.n_score[nb];
    opar_s[0] = -1;
    // a round whose persistent depth loop could not run (status bit 1)
    // marks itself: n_nodes = 0
    on_nodes[q] = (*t.status & 2u) ? 0 : nn;
  }
  for (int i = tid; i < Bsel; i += TB_THREADS) {
    int pn = my_par, tok = my_tok;
    float sc = my_sc;
    if (i >= TB_THREADS) {
      const int n = cpos[i].x;
      pn = t.n_par[nb + n];
      tok = t.n_tok[nb + n];
      sc = t.n_score[nb + n];
    }
    const int pos = cpos[i].y;
    const int pi = map[pn];
    if (pi < 0) atomicOr(t.status, 1u);
    const size_t o = (size_t)q * N + pos;
    otok[o] = tok;
    opar[o] = pi;
    odep[o] = (int32_t)(canon[i] >> 27);
    oscore[o] = sc;
    opar_s[pos] = pi;
  }
  for (int i = nn + tid; i < N; i += TB_THREADS) {
    const size_t o = (size_t)q * N + i;
    otok[o] = -1; opar[o] = -1; odep[o] = -1; oscore[o] = -INFINITY;
    opar_s[i] = -1;
  }
  __syncthreads();

  // mask[i][j] = 1 iff j is i or an ancestor of i: bands of rows as bitmaps
  // (bit (i - r0) * N + j), every emitted node setting its chain's bits
  // (parents come first in canonical order, so each walk ends at the root)
  uint8_t *mq = omask + (size_t)q * N * N;
  for (int r0 = 0; r0 < N; r0 += L.band_rows) {
    const int r1 = min(N, r0 + L.band_rows);
    const int nbits = (r1 - r0) * N;
    const int nw = (nbits + 31) / 32 + 1;
    for (int w = tid; w < nw; w += TB_THREADS) bm[w] = 0u;
    __syncthreads();
    for (int i = r0 + tid; i < min(r1, nn); i += TB_THREADS) {
      const int row = (i - r0) * N;
      int x = i, steps = 0;
      while (x >= 0 && steps < TB_MAXDEP) {
        atomicOr(&bm[(row + x) >> 5], 1u << ((row + x) & 31));
        x = x > 0 ? opar_s[x] : -1;
        ++steps;
      }
    }
    __syncthreads();
    uint8_t *g = mq + (size_t)r0 * N;
    const int head = min(nbits, (int)((16u - ((uint32_t)reinterpret_cast<uintptr_t>(g) & 15u)) & 15u));
    const int nchunk = (nbits - head) >> 4;
    const int tail = head + (nchunk << 4);
    for (int c = tid; c < nchunk; c += TB_THREADS) {
      const int p = head + (c << 4), w = p >> 5;
      const uint32_t b16 = __builtin_amdgcn_alignbit(bm[w + 1], bm[w], (uint32_t)(p & 31));
      *reinterpret_cast<uint4 *>(g + p) = make_uint4(spread4(b16), spread4(b16 >> 4),
                                                     spread4(b16 >> 8), spread4(b16 >> 12));
    }
    for (int e = tid; e < head; e += TB_THREADS) g[e] = (uint8_t)((bm[e >> 5] >> (e & 31)) & 1u);
    for (int e = tail + tid; e < nbits; e += TB_THREADS)
      g[e] = (uint8_t)((bm[e >> 5] >> (e & 31)) & 1u);
    __syncthreads();   // the next band reuses the bitmap
  }
}

size_t topb_smem(int NT, int B) { return tb_layout(NT, B).total; }

hipError_t topb_prepare(size_t lds_bytes) {
  return set_lds_limit(reinterpret_cast<const void *>(&k_topb_emit), lds_bytes);
}

hipError_t launch_topb_emit(int b, int NT, int B, float beta, int Bmax, const TreeBufs &t,
                            int32_t *tok, int32_t *parent, int32_t *depth, float *score,
                            uint8_t *mask, int32_t *n_nodes, hipStream_t st) {
  hipLaunchKernelGGL(k_topb_emit, dim3(b), dim3(TB_THREADS), topb_smem(NT, B), st, NT, B, beta,
                     Bmax, t, tok, parent, depth, score, mask, n_nodes);
  return hipGetLastError();
}

}  // namespace dtree
