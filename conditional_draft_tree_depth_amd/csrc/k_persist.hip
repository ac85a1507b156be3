// Depth loop of the depth-wise build as ONE persistent kernel (small batches).
//
// The low-rank head is linear ("Resumen Técnico: Domino", Methodology 2), so
// the corrected logits of candidate j for a branch with state S are
//   ell_j = Cl_j + W2[C_j] . (uH + W1[:, d:] S) = g_j + G_j . S,
// with g = Cl + W2[C] uH and G = W2[C] W1[:, d:] fixed for the round once the
// Top-M candidates are known (k_corr_tables).  The hidden units of the GRU
// are split over the persistent workgroups (16 units each, their W_hh rows
// resident in LDS, their W_ih rows in registers); after a GRU step every
// workgroup publishes, for every new
// branch, its partial sum of G_j . S over its own units, and raises its
// arrival flag.  Once every flag is up, every workgroup adds the partials in
// the same fixed order and runs the same selection (log-softmax over M,
// Top-K per branch, Top-W per request; DARTree page, Methodology 1), so one
// grid-wide hand-off per depth suffices.  While waiting, each workgroup
// computes the GRU input projections of its units for the next depth's
// candidates (the survivors' tokens are among them).
//
// GRU products run on MFMA: weights are the A operand, activations the B
// operand; the fp32 state is split exactly into three bf16 terms.
#include "common.hpp"
#include "kernels.hpp"

namespace dtree {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
__device__ __forceinline__ bf16x8 pk_bf(uint4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ f32x4 mfma(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(pk_bf(a), pk_bf(b), c, 0, 0, 0);
}

// ---------------------------------------------------------------- tables
// One workgroup: 16 candidate rows (flattened (request, depth, j)) x 64 state
// columns, on MFMA: A = the candidates' W2 rows, B = W1[:, d + n] (staged
// transposed in LDS so each lane reads 8 consecutive k), fp32 sums over the
// rank r (zero-padded to a multiple of 32).  The workgroups of column block 0
// also produce g = Cl + W2[C] . uH (one wave per row, fp32).
constexpr int CT_NB = 64;   // state columns per workgroup

__host__ __device__ inline size_t ct_smem(int r) {
  const int rp = (r + 31) & ~31;
  return (size_t)(CT_NB + 16) * (rp + 8) * 2;
}

__global__ __launch_bounds__(256) void k_corr_tables(int rows, int M, int D, int r, int s, int d,
                                                     int ldw1, const uint16_t *__restrict__ W2,
                                                     const uint16_t *__restrict__ W1,
                                                     const int32_t *__restrict__ C,
                                                     const float *__restrict__ Cl,
                                                     const float *__restrict__ uH,
                                                     float *__restrict__ G, float *__restrict__ g) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int rp = (r + 31) & ~31, KS = rp + 8;
  uint16_t *w1t = reinterpret_cast<uint16_t *>(smem);          // [CT_NB][KS]: W1[k][d + n0 + n]
  uint16_t *w2s = w1t + CT_NB * KS;                            // [16][KS]:   W2[C[row]][k]
  const int row0 = blockIdx.y * 16, n0 = blockIdx.x * CT_NB, tid = threadIdx.x;
  for (int i = tid; i < rp * CT_NB; i += blockDim.x) {
    const int k = i / CT_NB, n = i - k * CT_NB;
    w1t[n * KS + k] = (k < r && n0 + n < s) ? W1[(size_t)k * ldw1 + d + n0 + n] : (uint16_t)0;
  }
  for (int i = tid; i < 16 * rp; i += blockDim.x) {
    const int rr = i / rp, k = i - rr * rp, row = row0 + rr;
    uint16_t v = 0;
    if (row < rows && k < r) v = W2[(size_t)(C[row] < 0 ? 0 : C[row]) * r + k];
    w2s[rr * KS + k] = v;
  }
  __syncthreads();
  const int wave = tid >> 6, lane = tid & 63, lr = lane & 15, gq = lane >> 4;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int ks = 0; ks < rp / 32; ++ks) {
    const uint4 a = *reinterpret_cast<const uint4 *>(w2s + lr * KS + ks * 32 + gq * 8);
    const uint4 bv = *reinterpret_cast<const uint4 *>(w1t + (wave * 16 + lr) * KS + ks * 32 + gq * 8);
    acc = mfma(a, bv, acc);
  }
  // lane holds D[row 4 gq + t][column wave*16 + lr]
  const int n = n0 + wave * 16 + lr;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int row = row0 + 4 * gq + t;
    if (row < rows && n < s) G[(size_t)row * s + n] = acc[t];
  }
  if (blockIdx.x == 0) {
    for (int rr = wave; rr < 16; rr += 4) {
      const int row = row0 + rr;
      if (row >= rows) continue;
      const float *uh = uH + (size_t)(row / M) * r;   // row / M = request * D + depth
      float part = 0.f;
      for (int k = lane; k < r; k += 64) part += bf16_bits_to_f32(w2s[rr * KS + k]) * uh[k];
      part = wave_sum_f32(part);
      if (lane == 0) g[row] = Cl[row] + part;
    }
  }
}

// ---------------------------------------------------------------- persistent
constexpr int PK_WAVES = 8;
constexpr int PK_THREADS = PK_WAVES * 64;
constexpr int PK_UW = 16;           // hidden units per workgroup
constexpr int PK_GR = 3 * PK_UW;    // gate rows per workgroup (r, z, n blocks)
constexpr int PK_ROWS = 16;         // max expanded branches (all requests) per depth
constexpr int PK_MAXC = 32;         // max candidates (all requests) per depth
constexpr int PK_MAXZ = 512;        // max children (all requests) per depth
constexpr int PK_MAXELL = 512;      // max branches x candidates (all requests)
constexpr int PK_KSW = 10;          // W_ih k-steps (32 wide) held per wave: e <= 2560
constexpr int PK_HKS = 4;           // W_hh k-steps per wave: s <= 1024
constexpr unsigned PK_SPIN = 1u << 20;

struct PKLayout {
  size_t whh, red, gic, ghs, ell, ex, lpkey, snew, ckey, clex, cmeta, gs, ctok, gtab, sinfo,
      finfo, misc, total;
};

__host__ __device__ inline PKLayout pk_layout(int s) {
  PKLayout L;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o += (bytes + 15) & ~(size_t)15; return at; };
  L.whh = take((size_t)PK_GR * (s + 8) * 2);
  L.red = take((size_t)PK_WAVES * 3 * 16 * 16 * 4);
  L.gic = take((size_t)PK_MAXC * PK_GR * 4);
  L.ghs = take((size_t)3 * 16 * 16 * 4);
  L.ell = take((size_t)PK_MAXELL * 4);
  L.ex = take((size_t)PK_MAXELL * 4);
  L.lpkey = take((size_t)PK_MAXELL * 8);
  L.snew = take((size_t)2 * PK_ROWS * PK_UW * 4);
  L.ckey = take((size_t)PK_MAXZ * 8);
  L.clex = take((size_t)PK_MAXZ * 4);
  L.cmeta = take((size_t)PK_MAXZ * 4);
  L.gs = take((size_t)PK_MAXC * PK_UW * 4);
  L.ctok = take((size_t)2 * PK_MAXC * 4);
  L.gtab = take((size_t)PK_MAXC * 4);
  L.sinfo = take((size_t)PK_ROWS * 8 * 4);
  L.finfo = take((size_t)PK_ROWS * 4 * 4);
  L.misc = take(64 * 4);
  L.total = o;
  return L;
}

struct PKParams {
  int b, D, M, K, W, s, e, V, NWG;
  const uint16_t *W_ih, *W_hh, *Emb;
  const float *b_ih, *b_hh;
  const int32_t *C, *root;
  const float *G, *g;
  float *S0, *S1;        // [b * Wmax, s]
  float *part;           // [2][NWG][PK_MAXELL]
  uint32_t *flags;       // [NWG * 64]
  uint32_t epoch0;
  TreeBufs t;
};

// Hand-off between the persistent workgroups.  Everything another workgroup
// reads is stored with agent-scope relaxed atomic stores (pk_put), which are
// coherent across the XCDs without writing back whole L2 caches; each thread
// waits until its stores have completed before the workgroup raises its flag.
// The reader polls the flags, then one agent-scope acquire fence makes its
// plain loads see those values.
__device__ __forceinline__ void pk_put(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void pk_arrive(uint32_t *flags, uint32_t epoch) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0)
    __hip_atomic_store(&flags[blockIdx.x * 64], epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Returns false if some workgroup failed to arrive within the spin limit
// (status bit 1 is then set and the caller leaves the loop).
__device__ __forceinline__ bool pk_wait(uint32_t *flags, int nwg, uint32_t epoch, uint32_t *status,
                                        int *bad) {
  if (threadIdx.x == 0) *bad = 0;
  __syncthreads();
  if (threadIdx.x < nwg) {
    unsigned n = 0;
    while (__hip_atomic_load(&flags[threadIdx.x * 64], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
           epoch) {
      if (++n > PK_SPIN) {
        atomicOr(status, 2u);
        *bad = 1;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  return *bad == 0;
}

// GRU input projection of this workgroup's 48 gate rows for nrow (<= 16)
// token rows: out[row][gr] = W_ih[gate row] . Emb[tok(row)] + b_ih.  The
// weights sit in registers (k-step ks = wave + 8 i covers k in
// [32 ks, 32 ks + 32), lane group g its 8 consecutive k); the eight waves'
// partial sums over their k-steps are added in LDS.
__device__ void pk_gi(const PKParams &p, const uint4 (&wr)[PK_KSW][3], const int32_t *toks,
                      int nrow, float *red, float *out) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lr = lane & 15, g = lane >> 4;
  const int j0 = blockIdx.x * PK_UW, nks = p.e >> 5;
  const bool live = lr < nrow;
  const uint16_t *xrow = p.Emb + (size_t)toks[live ? lr : 0] * p.e + g * 8;
  uint4 xb[PK_KSW];
#pragma unroll
  for (int i = 0; i < PK_KSW; ++i) {
    const int ks = wave + PK_WAVES * i;
    xb[i] = make_uint4(0u, 0u, 0u, 0u);
    if (ks < nks && live) xb[i] = *reinterpret_cast<const uint4 *>(xrow + ks * 32);
  }
  f32x4 acc[3] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int i = 0; i < PK_KSW; ++i) {
    const int ks = wave + PK_WAVES * i;
    if (ks < nks) {
#pragma unroll
      for (int m = 0; m < 3; ++m) acc[m] = mfma(wr[i][m], xb[i], acc[m]);
    }
  }
#pragma unroll
  for (int m = 0; m < 3; ++m)
#pragma unroll
    for (int t = 0; t < 4; ++t) red[((wave * 3 + m) * 16 + 4 * g + t) * 16 + lr] = acc[m][t];
  __syncthreads();
  for (int i = threadIdx.x; i < nrow * PK_GR; i += blockDim.x) {
    const int row = i / PK_GR, gr = i - row * PK_GR;
    const int m = gr / PK_UW, u = gr - m * PK_UW;
    float v = p.b_ih ? p.b_ih[m * p.s + j0 + u] : 0.f;
#pragma unroll
    for (int wv = 0; wv < PK_WAVES; ++wv) v += red[((wv * 3 + m) * 16 + u) * 16 + row];
    out[i] = v;
  }
  __syncthreads();
}

__device__ __forceinline__ uint4 pack_bf16x8(const uint16_t (&h)[8]) {
  return make_uint4(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16),
                    h[4] | ((uint32_t)h[5] << 16), h[6] | ((uint32_t)h[7] << 16));
}

__global__ __launch_bounds__(PK_THREADS) void k_depth_persistent(PKParams p) {
  extern __shared__ __align__(16) uint8_t smem[];
  const PKLayout L = pk_layout(p.s);
  uint16_t *whh = reinterpret_cast<uint16_t *>(smem + L.whh);
  float *red = reinterpret_cast<float *>(smem + L.red);
  float *gic = reinterpret_cast<float *>(smem + L.gic);      // [cand][48] input part
  float *ghs = reinterpret_cast<float *>(smem + L.ghs);      // [3][16 units][16 rows]
  float *ell = reinterpret_cast<float *>(smem + L.ell);
  float *ex = reinterpret_cast<float *>(smem + L.ex);
  uint64_t *lpkey = reinterpret_cast<uint64_t *>(smem + L.lpkey);
  float *snew = reinterpret_cast<float *>(smem + L.snew);    // [2][16 rows][16 units]
  uint64_t *ckey = reinterpret_cast<uint64_t *>(smem + L.ckey);
  uint32_t *clex = reinterpret_cast<uint32_t *>(smem + L.clex);
  int32_t *cmeta = reinterpret_cast<int32_t *>(smem + L.cmeta);
  float *gsl = reinterpret_cast<float *>(smem + L.gs);       // [cand][16] G slice
  int32_t *ctok = reinterpret_cast<int32_t *>(smem + L.ctok); // [2][cand]
  float *gtab = reinterpret_cast<float *>(smem + L.gtab);    // [cand]
  int32_t *sinfo = reinterpret_cast<int32_t *>(smem + L.sinfo);
  int32_t *finfo = reinterpret_cast<int32_t *>(smem + L.finfo);
  int *misc = reinterpret_cast<int *>(smem + L.misc);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, g = lane >> 4;
  const int w = blockIdx.x, j0 = w * PK_UW;
  const int s = p.s, KS = s + 8, M = p.M, b = p.b, D = p.D, K = p.K;
  const int nks_h = s >> 5;
  const bool leader = w == 0;
  const int bM = b * M;

  // weights of this workgroup's 16 units: W_hh rows -> LDS, W_ih rows -> registers
  {
    const int per_row = s >> 3, total = PK_GR * per_row;
#pragma unroll 8
    for (int i = tid; i < total; i += blockDim.x) {
      const int row = i / per_row, k8 = (i - row * per_row) * 8;
      const int m = row / PK_UW, u = row - m * PK_UW;
      *reinterpret_cast<uint4 *>(whh + row * KS + k8) =
          *reinterpret_cast<const uint4 *>(p.W_hh + (size_t)(m * s + j0 + u) * s + k8);
    }
  }
  uint4 wr[PK_KSW][3];
  {
    const int nks = p.e >> 5;
#pragma unroll
    for (int i = 0; i < PK_KSW; ++i) {
      const int ks = wave + PK_WAVES * i;
#pragma unroll
      for (int m = 0; m < 3; ++m) {
        wr[i][m] = make_uint4(0u, 0u, 0u, 0u);
        if (ks < nks)
          wr[i][m] = *reinterpret_cast<const uint4 *>(p.W_ih + (size_t)(m * s + j0 + lr) * p.e +
                                                       ks * 32 + g * 8);
      }
    }
  }
  // root state: the GRU consumes each request's last verified token from h = 0
  for (int q = tid; q < b; q += blockDim.x) ctok[PK_MAXC + q] = min(max(p.root[q], 0), p.V - 1);
  for (int i = tid; i < bM * PK_UW; i += blockDim.x) {
    const int cj = i / PK_UW, u = i - cj * PK_UW, q = cj / M, jj = cj - q * M;
    gsl[i] = p.G[((size_t)(q * D + 0) * M + jj) * s + j0 + u];
  }
  __syncthreads();
  pk_gi(p, wr, ctok + PK_MAXC, b, red, gic);
  float *Scur = p.S0, *Snext = p.S1;
  float *sn_cur = snew, *sn_nxt = snew + PK_ROWS * PK_UW;
  for (int i = tid; i < b * PK_UW; i += blockDim.x) {
    const int q = i / PK_UW, u = i - q * PK_UW;
    const float *a = gic + q * PK_GR;
    const float cr = p.b_hh ? p.b_hh[j0 + u] : 0.f;
    const float cz = p.b_hh ? p.b_hh[s + j0 + u] : 0.f;
    const float cn = p.b_hh ? p.b_hh[2 * s + j0 + u] : 0.f;
    const float r = 1.f / (1.f + expf(-(a[u] + cr)));
    const float z = 1.f / (1.f + expf(-(a[PK_UW + u] + cz)));
    const float n = tanhf(a[2 * PK_UW + u] + r * cn);
    const float h = (1.f - z) * n;
    sn_cur[q * PK_UW + u] = h;
    pk_put(Scur + (size_t)q * s + j0 + u, h);
  }
  __syncthreads();
  // partial corrected logits of depth 0 over this workgroup's units
  for (int i = tid; i < bM; i += blockDim.x) {
    const int q = i / M;
    float acc = 0.f;
#pragma unroll
    for (int u = 0; u < PK_UW; ++u) acc += gsl[i * PK_UW + u] * sn_cur[q * PK_UW + u];
    pk_put(p.part + (size_t)w * PK_MAXELL + i, acc);
  }
  for (int q = tid; q < b; q += blockDim.x) {
    finfo[q * 4 + 0] = 0;                       // node id
    finfo[q * 4 + 1] = 0;                       // lexicographic rank
    finfo[q * 4 + 2] = __float_as_int(0.f);     // score
  }
  for (int i = tid; i < bM; i += blockDim.x)
    ctok[i] = max(p.C[((size_t)(i / M) * D + 0) * M + (i % M)], 0);
  pk_arrive(p.flags, p.epoch0 + 1);
  // while the others arrive: input projections of depth 0's candidates
  pk_gi(p, wr, ctok, min(bM, 16), red, gic);
  if (bM > 16) pk_gi(p, wr, ctok + 16, bM - 16, red, gic + 16 * PK_GR);
  if (!pk_wait(p.flags, p.NWG, p.epoch0 + 1, p.t.status, misc)) return;

  int A = 1, off = 1;   // branches expanded at this depth; node id of its first child
  for (int dd = 0; dd < D; ++dd) {
    const int rows = b * A;
    const int Z = A * K;
    const int An = Z < p.W ? Z : p.W;
    const int E = rows * M;
    const bool more = dd + 1 < D;
    const float *pp = p.part + (size_t)(dd & 1) * p.NWG * PK_MAXELL;
    // ---- one round trip: partial sums, tables, states of the current branches
    // two threads per entry (workgroups [0,32) and [32,64)) when E <= 256,
    // else one thread per entry in two batches; summed in a fixed order
    const bool act = tid < E;
    const bool split = E <= PK_THREADS / 2;
    const int ent = split ? (tid & (PK_THREADS / 2 - 1)) : tid;
    const int vhalf = split ? (tid >> 8) * 32 : 0;
    const bool lact = ent < E;
    float x[32];
#pragma unroll
    for (int v = 0; v < 32; ++v)
      x[v] = (lact && vhalf + v < p.NWG) ? pp[(size_t)(vhalf + v) * PK_MAXELL + ent] : 0.f;
    float gval = 0.f;
    if (act) gval = p.g[((size_t)(tid / (A * M)) * D + dd) * M + (tid % M)];
    if (tid < bM) {
      ctok[tid] = max(p.C[((size_t)(tid / M) * D + dd) * M + (tid % M)], 0);
      if (dd + 1 < D) ctok[PK_MAXC + tid] = max(p.C[((size_t)(tid / M) * D + dd + 1) * M + (tid % M)], 0);
    }
    float gv = 0.f;
    if (more && tid < bM * PK_UW) {
      const int cj = tid / PK_UW, u = tid - cj * PK_UW, q = cj / M, jj = cj - q * M;
      gv = p.G[((size_t)(q * D + dd + 1) * M + jj) * s + j0 + u];
    }
    {
      float part_sum = 0.f;
#pragma unroll
      for (int v = 0; v < 32; ++v) part_sum += x[v];
      if (!split && lact) {
#pragma unroll
        for (int v = 0; v < 32; ++v)
          x[v] = 32 + v < p.NWG ? pp[(size_t)(32 + v) * PK_MAXELL + ent] : 0.f;
#pragma unroll
        for (int v = 0; v < 32; ++v) part_sum += x[v];
      }
      if (split && tid >= PK_THREADS / 2 && lact) ex[ent] = part_sum;   // upper half
      __syncthreads();
      if (act) ell[tid] = gval + (split ? part_sum + ex[tid] : part_sum);
    }
    if (more && tid < bM * PK_UW) gsl[tid] = gv;
    // states of the current branches: loaded now, in flight during the selection
    float4 sf[PK_HKS][2];
#pragma unroll
    for (int i = 0; i < PK_HKS; ++i) {
      const int ks = wave + PK_WAVES * i;
      sf[i][0] = make_float4(0.f, 0.f, 0.f, 0.f);
      sf[i][1] = sf[i][0];
      if (more && ks < nks_h && lr < rows) {
        const float *sp = Scur + (size_t)lr * s + ks * 32 + g * 8;
        sf[i][0] = *reinterpret_cast<const float4 *>(sp);
        sf[i][1] = *reinterpret_cast<const float4 *>(sp + 4);
      }
    }
    // ---- selection, one thread per (branch, candidate): log-softmax over M
    float lval = 0.f, mx = -INFINITY;
    int row = 0, jj = 0;
    if (act) {
      row = tid / M;
      jj = tid - row * M;
      lval = ell[tid];
      for (int j = 0; j < M; ++j) mx = fmaxf(mx, ell[row * M + j]);
      ex[tid] = expf(lval - mx);
    }
    __syncthreads();
    uint64_t mykey = 0ull;
    float lp = 0.f;
    if (act) {
      float sum = 0.f;
      for (int j = 0; j < M; ++j) sum += ex[row * M + j];
      lp = lval - (mx + logf(sum));
      const int q = row / A;
      mykey = make_key(lp, (uint32_t)ctok[q * M + jj]);
      lpkey[tid] = mykey;
    }
    __syncthreads();
    // Top-K children of each branch (log-prob desc, token asc) by rank
    if (act) {
      int rank = 0;
      for (int j = 0; j < M; ++j) rank += lpkey[row * M + j] > mykey;
      if (rank < K) {
        const int q = row / A, a = row - q * A;
        const int c = q * Z + a * K + rank;
        const float sc = __fadd_rn(__int_as_float(finfo[row * 4 + 2]), lp);
        const uint32_t lex = ((uint32_t)finfo[row * 4 + 1] << 18) | (uint32_t)ctok[q * M + jj];
        ckey[c] = make_key(sc, lex);
        clex[c] = lex;
        cmeta[c] = jj;
      }
    }
    __syncthreads();
    // Top-W survivors of each request (score desc, token path asc) by rank
    if (tid < b * Z) {
      const int q = tid / Z, z = tid - q * Z;
      const uint64_t kc = ckey[tid];
      int rank = 0;
      for (int c2 = 0; c2 < Z; ++c2) rank += ckey[q * Z + c2] > kc;
      if (rank < An) {
        int32_t *si = sinfo + (q * An + rank) * 8;
        si[0] = off + z;                        // node id
        si[1] = q * A + z / K;                  // parent's row among the current branches
        si[3] = cmeta[tid];                     // candidate index
        si[4] = (int32_t)clex[tid];
        si[5] = __float_as_int(key_val(kc));    // score
      }
    }
    __syncthreads();
    if (tid < b * An) {
      const int q = tid / An;
      const uint32_t li = (uint32_t)sinfo[tid * 8 + 4];
      int rank = 0;
      for (int j = 0; j < An; ++j) rank += (uint32_t)sinfo[(q * An + j) * 8 + 4] < li;
      sinfo[tid * 8 + 6] = rank;
    }
    __syncthreads();
    // ---- state projection of every current branch (three-term split of S)
    if (more) {
      f32x4 acc[3] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int i = 0; i < PK_HKS; ++i) {
        const int ks = wave + PK_WAVES * i;
        if (ks < nks_h) {
          const float xs[8] = {sf[i][0].x, sf[i][0].y, sf[i][0].z, sf[i][0].w,
                               sf[i][1].x, sf[i][1].y, sf[i][1].z, sf[i][1].w};
          uint16_t hh[8], mi[8], lo[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            hh[q] = f32_to_bf16_rne(xs[q]);
            const float r1 = xs[q] - bf16_bits_to_f32(hh[q]);
            mi[q] = f32_to_bf16_rne(r1);
            lo[q] = f32_to_bf16_rne(r1 - bf16_bits_to_f32(mi[q]));
          }
          const uint4 bh = pack_bf16x8(hh), bm = pack_bf16x8(mi), bl = pack_bf16x8(lo);
#pragma unroll
          for (int m = 0; m < 3; ++m) {
            const uint4 a = *reinterpret_cast<const uint4 *>(whh + (m * PK_UW + lr) * KS + ks * 32 + g * 8);
            acc[m] = mfma(a, bh, acc[m]);
            acc[m] = mfma(a, bm, acc[m]);
            acc[m] = mfma(a, bl, acc[m]);
          }
        }
      }
#pragma unroll
      for (int m = 0; m < 3; ++m)
#pragma unroll
        for (int t = 0; t < 4; ++t) red[((wave * 3 + m) * 16 + 4 * g + t) * 16 + lr] = acc[m][t];
    }
    __syncthreads();
    if (more) {
      for (int i = tid; i < 3 * 16 * rows; i += blockDim.x) {
        const int m = i / (16 * rows), rem = i - m * 16 * rows, u = rem / rows, row = rem - u * rows;
        float v = p.b_hh ? p.b_hh[m * s + j0 + u] : 0.f;
#pragma unroll
        for (int wv = 0; wv < PK_WAVES; ++wv) v += red[((wv * 3 + m) * 16 + u) * 16 + row];
        ghs[(m * 16 + u) * 16 + row] = v;
      }
    }
    __syncthreads();
    // node records of this depth (written once, by one workgroup); global
    // stores are issued only right before the arrival fence, which waits for them
    const int Zc = Z, offc = off, Ac = A, Anc = An;
    auto write_records = [&]() {
      if (!leader) return;
      for (int c = tid; c < b * Zc; c += blockDim.x) {
        const int q = c / Zc, z = c - q * Zc;
        const size_t id = (size_t)q * p.t.NT + offc + z;
        p.t.n_tok[id] = (int32_t)(clex[c] & 0x3FFFFu);
        p.t.n_par[id] = finfo[(q * Ac + z / K) * 4 + 0];
        p.t.n_dep[id] = dd + 1;
        p.t.n_score[id] = key_val(ckey[c]);
        p.t.n_lex[id] = clex[c];
      }
      for (int i = tid; i < b * Anc; i += blockDim.x) {
        const int q = i / Anc, rk = i - q * Anc;
        p.t.surv_hist[((size_t)q * (D + 1) + dd + 1) * p.t.Wmax + rk] = sinfo[i * 8 + 0];
      }
    };
    if (!more) {
      write_records();
      break;
    }

    // ---- GRU step of the survivors for this workgroup's units
    const int nrow = b * An;
    if (tid < nrow * PK_UW) {
      const int i = tid / PK_UW, u = tid - i * PK_UW;
      const int q = i / An;
      const int pr = sinfo[i * 8 + 1], jc = sinfo[i * 8 + 3];
      const float *a = gic + (q * M + jc) * PK_GR;
      const float h = sn_cur[pr * PK_UW + u];
      const float r = 1.f / (1.f + expf(-(a[u] + ghs[(0 * 16 + u) * 16 + pr])));
      const float z = 1.f / (1.f + expf(-(a[PK_UW + u] + ghs[(1 * 16 + u) * 16 + pr])));
      const float n = tanhf(a[2 * PK_UW + u] + r * ghs[(2 * 16 + u) * 16 + pr]);
      const float hn = (1.f - z) * n + z * h;
      sn_nxt[i * PK_UW + u] = hn;
    }
    write_records();
    __syncthreads();
    // new states and partial corrected logits of depth dd+1 over this
    // workgroup's units (the frontier update waits for the records above)
    if (tid < nrow * PK_UW) {
      const int i = tid / PK_UW, u = tid - i * PK_UW;
      pk_put(Snext + (size_t)i * s + j0 + u, sn_nxt[i * PK_UW + u]);
    }
    float *pn = p.part + ((size_t)((dd + 1) & 1) * p.NWG + w) * PK_MAXELL;
    if (tid < nrow * M) {
      const int i = tid / M, j = tid - i * M, q = i / An;
      float acc = 0.f;
#pragma unroll
      for (int u = 0; u < PK_UW; ++u) acc += gsl[(q * M + j) * PK_UW + u] * sn_nxt[i * PK_UW + u];
      pk_put(pn + tid, acc);
    }
    for (int i = tid; i < nrow; i += blockDim.x) {
      finfo[i * 4 + 0] = sinfo[i * 8 + 0];
      finfo[i * 4 + 1] = sinfo[i * 8 + 6];
      finfo[i * 4 + 2] = sinfo[i * 8 + 5];
    }
    pk_arrive(p.flags, p.epoch0 + dd + 2);
    // while waiting: input projections of depth dd+1's candidates
    if (dd + 2 < D) {
      pk_gi(p, wr, ctok + PK_MAXC, min(bM, 16), red, gic);
      if (bM > 16) pk_gi(p, wr, ctok + PK_MAXC + 16, bM - 16, red, gic + 16 * PK_GR);
    }
    if (!pk_wait(p.flags, p.NWG, p.epoch0 + dd + 2, p.t.status, misc)) return;
    float *tmp = Scur; Scur = Snext; Snext = tmp;
    float *tn = sn_cur; sn_cur = sn_nxt; sn_nxt = tn;
    off += Z;
    A = An;
  }
}

// ---------------------------------------------------------------- host side
bool persist_eligible(int b, int D, int M, int K, int W, int s, int e, int r, int wtype,
                      size_t lds_max) {
  if (wtype != WT_BF16 || s % 128 || e % 128 || s % PK_UW) return false;
  if (s > 32 * PK_HKS * PK_WAVES || e > 32 * PK_KSW * PK_WAVES || D > 31) return false;
  if (s / PK_UW > 64) return false;   // grid-wide hand-offs get slow past 64 workgroups
  if (b * W > PK_ROWS || b * M > PK_MAXC || (long long)b * W * M > PK_MAXELL) return false;
  if ((long long)b * W * K > PK_MAXZ) return false;
  if (r > 512) return false;   // the correction-table tile must fit in LDS
  return pk_layout(s).total <= lds_max;
}

size_t persist_flag_words(int s) { return (size_t)(s / PK_UW) * 64; }
size_t persist_part_floats(int s) { return (size_t)2 * (s / PK_UW) * PK_MAXELL; }
size_t persist_gitab_floats(int s, int D) { (void)s; (void)D; return 16; }

hipError_t persist_prepare(int s) {
  if (s % PK_UW) return hipSuccess;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_depth_persistent),
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)pk_layout(s).total);
  if (e != hipSuccess) return e;
  return hipFuncSetAttribute(reinterpret_cast<const void *>(&k_corr_tables),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)ct_smem(512));
}

hipError_t launch_corr_tables(int rows, int M, int D, int r, int s, int d, int ldw1,
                              const void *W2, const void *W1, const int32_t *C, const float *Cl,
                              const float *uH, float *G, float *g, hipStream_t st) {
  dim3 grid((s + CT_NB - 1) / CT_NB, (rows + 15) / 16);
  const size_t sm = ct_smem(r);
  hipLaunchKernelGGL(k_corr_tables, grid, dim3(256), sm, st, rows, M, D, r, s, d, ldw1,
                     static_cast<const uint16_t *>(W2), static_cast<const uint16_t *>(W1), C, Cl,
                     uH, G, g);
  return hipGetLastError();
}

hipError_t launch_depth_persistent(const PersistArgs &a, hipStream_t st) {
  PKParams p{};
  p.b = a.b; p.D = a.D; p.M = a.M; p.K = a.K; p.W = a.W; p.s = a.s; p.e = a.e; p.V = a.V;
  p.NWG = a.s / PK_UW;
  p.W_ih = static_cast<const uint16_t *>(a.W_ih);
  p.W_hh = static_cast<const uint16_t *>(a.W_hh);
  p.Emb = static_cast<const uint16_t *>(a.Emb);
  p.b_ih = a.b_ih; p.b_hh = a.b_hh; p.C = a.C; p.root = a.root; p.G = a.G; p.g = a.g;
  p.S0 = a.S0; p.S1 = a.S1; p.part = a.part; p.flags = a.flags; p.epoch0 = a.epoch0;
  p.t = a.t;
  void *args[] = {&p};
  return hipLaunchCooperativeKernel(reinterpret_cast<const void *>(&k_depth_persistent),
                                    dim3(p.NWG), dim3(PK_THREADS), args, pk_layout(a.s).total, st);
}

}  // namespace dtree

