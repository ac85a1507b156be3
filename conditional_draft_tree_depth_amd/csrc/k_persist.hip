// Depth loop of the depth-wise build as ONE persistent kernel (small batches).
//
// The low-rank head is linear ("Resumen Técnico: Domino", Metodología 2), so
// the corrected logits of candidate j for a branch with state S are
//   ell_j = Cl_j + W2[C_j] . (uH + W1[:, d:] S) = g_j + G_j . S,
// with g = Cl + W2[C] uH and G = W2[C] W1[:, d:] fixed for the round once the
// Top-M candidates are known (k_corr_tables).
//
// The GRU's hidden units are split over the workgroups of one cooperative
// launch.  Producers (8 units each, their W_ih rows in registers) compute the
// input projections W_ih Emb[tok] + b_ih of the root tokens and of every
// depth's candidates ahead of time; nothing they do waits on anyone.
// Consumers (16 units each, their W_hh rows in registers) run the depth loop:
// after a GRU step each publishes, for every new branch, its partial sum of
// G_j . S over its own units and raises its arrival flag; once every flag is
// up, every consumer adds the partials in the same fixed order and runs the
// same selection (log-softmax over M, Top-K per branch, Top-W per request;
// DARTree page, Metodología 1), so one grid-wide hand-off per depth suffices.
//
// GRU products run on MFMA: weights are the A operand, activations the B
// operand; the fp32 state is split exactly into three bf16 terms.
#include <algorithm>
#include <type_traits>

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
// columns, on MFMA with fragments read straight from global memory: A = the
// candidates' W2 rows (gathered by token), B = W1t rows, W1t = W1[:, d:]^T
// zero-padded to a multiple of 32 in the rank (made once per context), fp32
// sums over the rank.  The first waves of the row block also produce
// g = Cl + W2[C] . uH (one wave per row, fp32).
constexpr int CT_NB = 64;   // state columns per workgroup
constexpr int CT_THREADS = 256;
constexpr int CT_MAXKS = 16;   // rank <= 512

__global__ __launch_bounds__(CT_THREADS) void k_corr_tables(int rows, int M, int r, int s,
                                                     const uint16_t *__restrict__ W2,
                                                     const uint16_t *__restrict__ W1t,
                                                     const int32_t *__restrict__ C,
                                                     const float *__restrict__ Cl,
                                                     const float *__restrict__ uH,
                                                     float *__restrict__ G, float *__restrict__ g) {
  const int rp = (r + 31) & ~31, nks = rp >> 5;
  const int row0 = blockIdx.y * 16, n0 = blockIdx.x * CT_NB, tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, lr = lane & 15, gq = lane >> 4;
  const int arow = row0 + lr;
  const int tok = arow < rows ? max(C[arow], 0) : -1;
  const int n = n0 + wave * 16 + lr;
  uint4 a[CT_MAXKS], bv[CT_MAXKS];
#pragma unroll
  for (int ks = 0; ks < CT_MAXKS; ++ks) {
    const int k = ks * 32 + gq * 8;
    a[ks] = make_uint4(0u, 0u, 0u, 0u);
    bv[ks] = a[ks];
    if (ks < nks) {
      if (tok >= 0 && k < r) a[ks] = *reinterpret_cast<const uint4 *>(W2 + (size_t)tok * r + k);
      if (n < s) bv[ks] = *reinterpret_cast<const uint4 *>(W1t + (size_t)n * rp + k);
    }
  }
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < CT_MAXKS; ++ks)
    if (ks < nks) acc = mfma(a[ks], bv[ks], acc);
  // lane holds D[row 4 gq + t][column wave*16 + lr]; G is stored
  // [request * D + depth][state unit][candidate] so that a run of state units
  // of one depth is one contiguous block
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int row = row0 + 4 * gq + t;
    if (row < rows && n < s) {
      const int qd = row / M, jj = row - qd * M;
      G[((size_t)qd * s + n) * M + jj] = acc[t];
    }
  }
  // g: one wave per row, spread over the column blocks of this row block
  for (int rr = blockIdx.x * (CT_THREADS / 64) + wave; rr < 16;
       rr += gridDim.x * (CT_THREADS / 64)) {
    const int row = row0 + rr;
    if (row >= rows) break;
    const uint16_t *w2 = W2 + (size_t)max(C[row], 0) * r;
    const float *uh = uH + (size_t)(row / M) * r;   // row / M = request * D + depth
    float part = 0.f;
    for (int k = lane; k < r; k += 64) part += bf16_bits_to_f32(w2[k]) * uh[k];
    part = wave_sum_f32(part);
    if (lane == 0) g[row] = Cl[row] + part;
  }
}

// W1t[n][k] = W1[k][d + n] for k < r, zero for r <= k < rp
__global__ void k_transpose_w1s(const uint16_t *__restrict__ W1, int r, int s, int d, int ldw1,
                                uint16_t *__restrict__ W1t) {
  const int rp = (r + 31) & ~31;
  const size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  if (i >= (size_t)s * rp) return;
  const int n = (int)(i / rp), k = (int)(i - (size_t)n * rp);
  W1t[i] = k < r ? W1[(size_t)k * ldw1 + d + n] : (uint16_t)0;
}

// ---------------------------------------------------------------- persistent
constexpr int PK_WAVES = 8;
constexpr int PK_THREADS = PK_WAVES * 64;
constexpr int PK_CU = 16;           // units per consumer (16 or 32)
constexpr int PK_HALF = PK_CU / 16; // 16-unit halves per consumer
constexpr int PK_NMT = 3 * PK_HALF; // W_hh row tiles per consumer (gates x halves)
constexpr int PK_XS = 1024 / PK_CU / 8;   // partial-sum vectors per thread (consumers / 8)
constexpr int PK_PU = 8;            // units per producer
static_assert(PK_CU == 16 || PK_CU == 32, "consumer width");
static_assert(1024 / PK_CU <= 64, "pk_wait polls consumer flags with the first wave");
constexpr int PK_PPC = PK_CU / PK_PU;   // producers feeding one consumer
constexpr int PK_ROWS = 16;         // max expanded branches (all requests) per depth
constexpr int PK_MAXC = 32;         // max candidates (all requests) per depth
constexpr int PK_MAXZ = 512;        // max children (all requests) per depth
constexpr int PK_MAXELL = 512;      // max branches x candidates (all requests)
constexpr int PK_MAXD = 31;         // max depth
constexpr int PK_KSW = 10;          // W_ih k-steps (32 wide) per producer wave: e <= 2560
constexpr int PK_HKS = 4;           // W_hh k-steps per consumer wave: s <= 1024
constexpr int PK_SMAX = 32 * PK_HKS * 8;   // largest state size
constexpr int PK_SLOTS = 3 * PK_ROWS;      // (term, branch) columns of the state fragments
constexpr unsigned PK_SPIN = 1u << 20;

struct PKLayout {
  size_t red, stage, gis, gsl, ghs, bhh, ell, ex, lpkey, snew, ckey, clex, cmeta, cpar, ctok,
      sinfo, finfo, misc, total;
};

__host__ __device__ inline PKLayout pk_layout() {
  PKLayout L;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o += (bytes + 15) & ~(size_t)15; return at; };
  // per-wave MFMA tiles; before them, the current branches' state fragments
  L.red = take(std::max((size_t)PK_WAVES * PK_NMT * 16 * 16 * 4, (size_t)(PK_SMAX / 32) * PK_SLOTS * 64));
  L.stage = take((size_t)PK_WAVES * PK_MAXELL * 4);   // partial sums, 8 groups of consumers
  L.gis = take((size_t)PK_MAXC * 3 * PK_CU * 4);      // input part of this depth's candidates
  L.gsl = take((size_t)PK_MAXC * PK_CU * 4);          // G slice of the next depth
  L.ghs = take((size_t)PK_NMT * 16 * 16 * 4);         // state part of the current branches
  L.bhh = take((size_t)3 * PK_CU * 4);
  L.ell = take((size_t)PK_MAXELL * 4);
  L.ex = take((size_t)PK_MAXELL * 4);
  L.lpkey = take((size_t)PK_MAXELL * 8);
  L.snew = take((size_t)2 * PK_ROWS * PK_CU * 4);
  L.ckey = take((size_t)PK_MAXZ * 8);
  L.clex = take((size_t)PK_MAXZ * 4);
  L.cmeta = take((size_t)PK_MAXZ * 4);
  L.cpar = take((size_t)PK_MAXZ * 4);
  L.ctok = take((size_t)PK_MAXC * 4);
  L.sinfo = take((size_t)PK_ROWS * 8 * 4);
  L.finfo = take((size_t)PK_ROWS * 4 * 4);
  L.misc = take(64 * 4);
  L.total = o;
  return L;
}

struct PKParams {
  int b, D, M, K, W, s, e, V, NC, NP;
  const uint16_t *W_ih, *W_hh, *Emb;
  const float *b_ih, *b_hh;
  const int32_t *C, *root;
  const float *G, *g;
  uint16_t *T0, *T1;     // published states: [s/32 k-steps][48 slots][32] bf16
  float *part;           // [2][NC][PK_MAXELL]
  float *gitab;          // [D slots][PK_MAXC][3s]: slot 0 roots, slot t+1 depth t
  uint32_t *flags;       // [(NC + NP) * 64]: consumer arrivals, then producer slots
  uint32_t *host_fail;   // host-visible word, set when a wait ran out (or null)
  uint32_t spin;         // polls before a wait gives up
  uint32_t epoch0;
  int markov;            // nonzero: every GRU step starts from a zero state
  TreeBufs t;
};

// Hand-off between workgroups.  Everything another workgroup reads is stored
// with agent-scope relaxed atomic stores (pk_put), which are coherent across
// the XCDs without writing back whole L2 caches; each thread waits until its
// stores have completed before the workgroup raises its flag.  Readers poll
// the flags and then read the published values with device-coherent loads
// (pk_get, pk_get4, and the copies below with the same cache policy), which
// miss in the XCD-private caches, so no cache-wide invalidation is needed.
constexpr int PK_COHERENT = 16;   // cache-policy bits of a device-coherent load
__device__ __forceinline__ void pk_put(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float pk_get(const float *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Device-coherent 16-byte load at byte offset off of a buffer (reads past the
// buffer's size return zeros).
typedef unsigned pk_u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t pk_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ float4 pk_get4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const pk_u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, PK_COHERENT);
  return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
                     __uint_as_float(v.w));
}

// Copies nchunk 16-byte chunks straight from global memory into LDS (no
// registers in between): chunk ci lands at dst + 4 ci and comes from src(ci);
// AUX is the loads' cache policy.  Wave w issues copy instructions w,
// w + PK_WAVES, ...; each covers 64 chunks, lanes past nchunk copy chunk 0
// again into the destination's tail, so dst must hold nchunk rounded up to 64
// chunks.
template <int AUX, class F>
__device__ __forceinline__ void pk_dma(float *dst, int nchunk, F src) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int ninstr = (nchunk + 63) >> 6;
  for (int in = wave; in < ninstr; in += PK_WAVES) {
    const int ci = in * 64 + lane;
    __builtin_amdgcn_global_load_lds(src(ci < nchunk ? ci : 0),
                                     (__attribute__((address_space(3))) void *)(dst + in * 256),
                                     16, 0, AUX);
  }
}

__device__ __forceinline__ void pk_raise(uint32_t *flag, uint32_t epoch) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_store(flag, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Threads i < n poll flags[i * 64] >= epoch, threads 64 .. 64 + npf - 1 poll
// pf[(i - 64) * 64] >= pepoch (">=" modulo 2^32: the epoch wraps); false if any wait exceeded the spin limit
// (status bit 1 is then set, 1 is stored to the host-visible word host_fail,
// and the caller leaves).  A wait can only run out if some workgroup of the
// grid never became resident next to the waiting ones.
__device__ __forceinline__ bool pk_wait(const uint32_t *flags, int n, uint32_t epoch,
                                        const uint32_t *pf, int npf, uint32_t pepoch,
                                        uint32_t *status, uint32_t *host_fail, unsigned spin,
                                        int *bad) {
  if (threadIdx.x == 0) *bad = 0;
  __syncthreads();
  const uint32_t *f = nullptr;
  uint32_t want = 0;
  const int tid = threadIdx.x;
  if (tid < n) { f = flags + tid * 64; want = epoch; }
  else if (tid >= 64 && tid < 64 + npf) { f = pf + (tid - 64) * 64; want = pepoch; }
  if (f) {
    unsigned k = 0;
    // flags and epochs are 32-bit counters that wrap: compare by difference
    while ((int32_t)(__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) - want) < 0) {
      if (++k > spin) {
        atomicOr(status, 2u);
        if (host_fail) __hip_atomic_store(host_fail, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        *bad = 1;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  __syncthreads();
  return *bad == 0;
}

__device__ __forceinline__ uint4 pack_bf16x8(const uint16_t (&h)[8]) {
  return make_uint4(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16),
                    h[4] | ((uint32_t)h[5] << 16), h[6] | ((uint32_t)h[7] << 16));
}

// Exact x / d for 0 <= x < 2^16 and 1 <= d < 2^16 with one high multiply:
// m = floor(2^32 / d) + 1 exceeds 2^32 / d by less than 1 / d per unit of x.
struct PkDiv {
  uint32_t m;   // 0 stands for d == 1
  __device__ explicit PkDiv(uint32_t d) : m(d == 1 ? 0u : 0xFFFFFFFFu / d + 1u) {}
  __device__ __forceinline__ int operator()(int x) const {
    return m ? (int)__umulhi((uint32_t)x, m) : x;
  }
};

// All-reduce of v over aligned groups of n lanes (n a power of two <= 64);
// every lane of a group ends with the same bits for a commutative op.
template <class Op>
__device__ __forceinline__ float pk_group_reduce(float v, int n, Op op) {
  if (n >= 2) v = op(v, xchg_f32<1>(v));
  if (n >= 4) v = op(v, xchg_f32<2>(v));
  if (n >= 8) v = op(v, xchg_f32<4>(v));
  if (n >= 16) v = op(v, xchg_f32<8>(v));
  if (n >= 32) v = op(v, xchg_f32<16>(v));
  if (n >= 64) v = op(v, xchg_f32<32>(v));
  return v;
}

// Published states.  A state row h of the current branches enters the W_hh
// products as the exact three-term bf16 split h = hi + mid + lo; term t of
// branch row r is column slot t * rp + r of the MFMA B operand (rp = 5, 8 or
// 16 by the number of branches, so that the 3 x rows columns fill as few
// 16-column passes as possible).  State units 32 k .. 32 k + 31 (the units of
// one or two consumers) form k-step k: [k-step][3 rp slots][32 units] in bf16, so a consumer
// copies the whole table with one contiguous transfer and every lane reads
// its fragment (slot pass * 16 + lane % 16, units 8 (lane / 16) ..) as 16
// contiguous bytes.  Pass p column j accumulates slot 16 p + j, so the terms
// of row r end up in columns r, r + rp and r + 2 rp (mod 16).
__host__ __device__ inline int pk_rp(int rows) { return rows <= 5 ? 5 : rows <= 8 ? 8 : 16; }
__host__ __device__ inline int pk_npass(int rows) { return rows <= 5 ? 1 : rows <= 8 ? 2 : 3; }

__device__ __forceinline__ void split3(float x, uint16_t &hi, uint16_t &mi, uint16_t &lo) {
  hi = f32_to_bf16_rne(x);
  const float r1 = x - bf16_bits_to_f32(hi);
  mi = f32_to_bf16_rne(r1);
  lo = f32_to_bf16_rne(r1 - bf16_bits_to_f32(mi));
}

// Publishes state value h of branch row `row` (of `rows`) and unit u (0 ..
// PK_CU - 1, lanes of a pair u, u ^ 1 both active) of consumer c into table T.
__device__ __forceinline__ void pk_put_state(uint16_t *T, int c, int rows, int row, int u, float h) {
  uint16_t t3[3];
  split3(h, t3[0], t3[1], t3[2]);
  const int rp = pk_rp(rows);
#pragma unroll
  for (int t = 0; t < 3; ++t) {
    const uint32_t mine = t3[t];
    const uint32_t other = xchg_u32<1>(mine);   // unit u ^ 1
    if ((u & 1) == 0) {
      uint32_t *dst = reinterpret_cast<uint32_t *>(
          T + ((size_t)((c / (32 / PK_CU)) * 3 * rp + t * rp + row) * 32 + (c % (32 / PK_CU)) * PK_CU + u));
      __hip_atomic_store(dst, mine | (other << 16), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Visits n values ld(0..n-1) with op, loading 8 at a time back to back
// before their first use (a scheduling barrier keeps the loads together, so
// the LDS latency is paid once per 8 values); the order of op is fixed.
template <class T, class Ld, class Op>
__device__ __forceinline__ void pk_scan(int n, Ld ld, Op op) {
  int j = 0;
  for (; j + 8 <= n; j += 8) {
    T v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = ld(j + k);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < 8; ++k) op(v[k]);
  }
  for (; j < n; ++j) op(ld(j));
}

// ---- producer: GRU input projections of every table slot for 8 units.
// A tiles: tile 0 rows 0-7 gate r, rows 8-15 gate z; tile 1 rows 0-7 gate n
// (rows 8-15 zero).  B tiles: 16 token rows each, both in flight at once.
__device__ void pk_producer(const PKParams &p, uint8_t *smem) {
  const PKLayout L = pk_layout();
  float *red = reinterpret_cast<float *>(smem + L.red);        // [8][2 mt][2 nt][16 col][16 arow]
  float *bih = reinterpret_cast<float *>(smem + L.bhh);        // [3][8]
  int32_t *toks = reinterpret_cast<int32_t *>(smem + L.stage); // [slot][PK_MAXC]
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 15, g = lane >> 4;
  const int pidx = blockIdx.x - p.NC, j0 = pidx * PK_PU, s = p.s, nks = p.e >> 5;
  const int b = p.b, M = p.M, D = p.D;
  uint32_t *myflag = p.flags + (size_t)(p.NC + pidx) * 64;
  uint4 wr[PK_KSW][2];
#pragma unroll
  for (int i = 0; i < PK_KSW; ++i) {
    const int ks = wave + PK_WAVES * i;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int gate = mt * 2 + (lr >> 3);
      wr[i][mt] = make_uint4(0u, 0u, 0u, 0u);
      if (ks < nks && gate < 3)
        wr[i][mt] = *reinterpret_cast<const uint4 *>(
            p.W_ih + (size_t)(gate * s + j0 + (lr & 7)) * p.e + ks * 32 + g * 8);
    }
  }
  if (tid < 3 * PK_PU) bih[tid] = p.b_ih ? p.b_ih[(tid / PK_PU) * s + j0 + tid % PK_PU] : 0.f;
  for (int i = tid; i < D * PK_MAXC; i += PK_THREADS) {
    const int slot = i / PK_MAXC, row = i - slot * PK_MAXC;
    int tk = 0;
    if (slot == 0) {
      if (row < b) tk = min(max(p.root[row], 0), p.V - 1);
    } else if (row < b * M) {
      tk = max(p.C[((size_t)(row / M) * D + slot - 1) * M + (row % M)], 0);
    }
    toks[i] = tk;
  }
  __syncthreads();
  for (int slot = 0; slot < D; ++slot) {
    const int nrow = slot == 0 ? b : b * M;
    const int nnt = nrow > 16 ? 2 : 1;
    uint4 xb[2][PK_KSW];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int xr = min(nt * 16 + lr, nrow - 1);
      const uint16_t *xrow = p.Emb + (size_t)toks[slot * PK_MAXC + xr] * p.e + g * 8;
#pragma unroll
      for (int i = 0; i < PK_KSW; ++i) {
        const int ks = wave + PK_WAVES * i;
        xb[nt][i] = make_uint4(0u, 0u, 0u, 0u);
        if (ks < nks && nt < nnt) xb[nt][i] = *reinterpret_cast<const uint4 *>(xrow + ks * 32);
      }
    }
    f32x4 acc[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) { acc[mt][0] = f32x4{0.f, 0.f, 0.f, 0.f}; acc[mt][1] = acc[mt][0]; }
#pragma unroll
    for (int i = 0; i < PK_KSW; ++i) {
      const int ks = wave + PK_WAVES * i;
      if (ks < nks) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          acc[mt][0] = mfma(wr[i][mt], xb[0][i], acc[mt][0]);
          acc[mt][1] = mfma(wr[i][mt], xb[1][i], acc[mt][1]);
        }
      }
    }
    // lane holds D[arow 4g + t][col lr]; stored as one 16-byte run per lane
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
        *reinterpret_cast<f32x4 *>(red + ((((wave * 2 + mt) * 2 + nt) * 16 + lr) * 16 + 4 * g)) =
            acc[mt][nt];
    __syncthreads();
    float *out = p.gitab + (size_t)slot * PK_MAXC * 3 * s;
    for (int i = tid; i < nrow * 3 * PK_PU; i += PK_THREADS) {
      const int row = i / (3 * PK_PU), gr = i - row * 3 * PK_PU;
      const int m = gr / PK_PU, u = gr - m * PK_PU;
      const int mt = m >> 1, arow = (m & 1) * 8 + u, nt = row >> 4, col = row & 15;
      float v = bih[gr];
#pragma unroll
      for (int wv = 0; wv < PK_WAVES; ++wv)
        v += red[(((wv * 2 + mt) * 2 + nt) * 16 + col) * 16 + arow];
      pk_put(out + (size_t)row * 3 * s + m * s + j0 + u, v);
    }
    pk_raise(myflag, p.epoch0 + slot + 1);
  }
}

// ---- consumer: the depth loop
__device__ void pk_consumer(const PKParams &p, uint8_t *smem) {
  const PKLayout L = pk_layout();
  float *red = reinterpret_cast<float *>(smem + L.red);      // [8][PK_NMT mt][16 row][16 unit]
  const uint16_t *sfr = reinterpret_cast<const uint16_t *>(red);   // state fragments, before red
  float *stage = reinterpret_cast<float *>(smem + L.stage);  // [group][entries]
  float *gis = reinterpret_cast<float *>(smem + L.gis);      // [cand][3][PK_CU]
  float *gsl = reinterpret_cast<float *>(smem + L.gsl);      // [request][PK_CU units][M]
  float *ghs = reinterpret_cast<float *>(smem + L.ghs);      // [PK_NMT mt][16 rows][16 units]
  float *bhh = reinterpret_cast<float *>(smem + L.bhh);      // [gate][PK_CU units]
  float *ell = reinterpret_cast<float *>(smem + L.ell);
  float *ex = reinterpret_cast<float *>(smem + L.ex);
  uint64_t *lpkey = reinterpret_cast<uint64_t *>(smem + L.lpkey);
  float *snew = reinterpret_cast<float *>(smem + L.snew);    // [2][16 rows][PK_CU units]
  uint64_t *ckey = reinterpret_cast<uint64_t *>(smem + L.ckey);
  uint32_t *clex = reinterpret_cast<uint32_t *>(smem + L.clex);
  int32_t *cmeta = reinterpret_cast<int32_t *>(smem + L.cmeta);
  int32_t *cpar = reinterpret_cast<int32_t *>(smem + L.cpar);   // children's parent node ids
  int32_t *ctok = reinterpret_cast<int32_t *>(smem + L.ctok);
  int32_t *sinfo = reinterpret_cast<int32_t *>(smem + L.sinfo);
  int32_t *finfo = reinterpret_cast<int32_t *>(smem + L.finfo);
  int *misc = reinterpret_cast<int *>(smem + L.misc);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 15, g = lane >> 4;
  const int c = blockIdx.x, j0 = c * PK_CU;
  const int s = p.s, M = p.M, b = p.b, D = p.D, K = p.K, bM = b * M, nks = s >> 5;
  uint32_t *cflags = p.flags;
  const uint32_t *pflags = p.flags + (size_t)(p.NC + PK_PPC * c) * 64;   // this consumer's producers

  // W_hh rows of this workgroup's units, as MFMA A fragments: tile mt =
  // gate * PK_HALF + half covers gate rows gate*s + j0 + half*16 + (0..15)
  uint4 wh[PK_HKS][PK_NMT];
#pragma unroll
  for (int i = 0; i < PK_HKS; ++i) {
    const int ks = wave + PK_WAVES * i;
#pragma unroll
    for (int mt = 0; mt < PK_NMT; ++mt) {
      wh[i][mt] = make_uint4(0u, 0u, 0u, 0u);
      if (ks < nks)
        wh[i][mt] = *reinterpret_cast<const uint4 *>(
            p.W_hh + (size_t)((mt / PK_HALF) * s + j0 + (mt % PK_HALF) * 16 + lr) * s + ks * 32 + g * 8);
    }
  }
  uint16_t *Tcur = p.T0, *Tnext = p.T1;
  float *sn_cur = snew, *sn_nxt = snew + PK_ROWS * PK_CU;
  if (tid < 3 * PK_CU) bhh[tid] = p.b_hh ? p.b_hh[(tid / PK_CU) * s + j0 + tid % PK_CU] : 0.f;
  for (int i = tid; i < b * PK_CU * M; i += PK_THREADS) {
    const int q = i / (PK_CU * M), rem = i - q * PK_CU * M;
    gsl[i] = p.G[((size_t)(q * D + 0) * s + j0) * M + rem];
  }
  for (int q = tid; q < b; q += PK_THREADS) {
    finfo[q * 4 + 0] = 0;                       // node id
    finfo[q * 4 + 1] = 0;                       // lexicographic rank
    finfo[q * 4 + 2] = __float_as_int(0.f);     // score
  }
  // root state from slot 0 (h = 0, so the state part is b_hh)
  if (!pk_wait(cflags, 0, 0u, pflags, PK_PPC, p.epoch0 + 1, p.t.status, p.host_fail, p.spin, misc)) return;
  for (int i = tid; i < b * PK_CU; i += PK_THREADS) {
    const int q = i / PK_CU, u = i - q * PK_CU;
    const float *a = p.gitab + (size_t)q * 3 * s + j0 + u;
    const float ar = pk_get(a), az = pk_get(a + s), an = pk_get(a + 2 * s);
    const float r = 1.f / (1.f + expf(-(ar + bhh[u])));
    const float z = 1.f / (1.f + expf(-(az + bhh[PK_CU + u])));
    const float n = tanhf(an + r * bhh[2 * PK_CU + u]);
    const float h = (1.f - z) * n;
    sn_cur[q * PK_CU + u] = h;
    pk_put_state(Tcur, c, b, q, u, h);
  }
  __syncthreads();
  for (int i = tid; i < bM; i += PK_THREADS) {
    const int q = i / M, j = i - q * M;
    float acc = 0.f;
#pragma unroll
    for (int u = 0; u < PK_CU; ++u) acc += gsl[(q * PK_CU + u) * M + j] * sn_cur[q * PK_CU + u];
    pk_put(p.part + (size_t)c * PK_MAXELL + i, acc);
  }
  pk_raise(cflags + c * 64, p.epoch0 + 1);
  // (the producers' next slot is waited for only where depth 0 first needs it)
  if (!pk_wait(cflags, p.NC, p.epoch0 + 1, pflags, 0, 0u, p.t.status, p.host_fail, p.spin, misc)) return;

  // input projections of table slot `slot` (this workgroup's units) into LDS
  auto load_gis = [&](int slot) {
    const float *gtab = p.gitab + (size_t)slot * PK_MAXC * 3 * s + j0;
    constexpr int CPR = PK_CU / 4;   // 16-byte chunks per gate row of this workgroup's units
    pk_dma<PK_COHERENT>(gis, bM * 3 * CPR, [&](int ci) {
      const int rw = ci / CPR, cj = rw / 3;
      return gtab + (size_t)cj * 3 * s + (rw - 3 * cj) * s + (ci % CPR) * 4;
    });
  };
  // (branch row, candidate) of this thread's entry; the entries are row-major
  const int row0 = tid / M, jj0 = tid - row0 * M;
  const PkDiv divK(K), divQC(PK_CU / 4 * M), divNC(p.NC);
  int A = 1, off = 1;   // branches expanded at this depth; node id of its first child
  for (int dd = 0; dd < D; ++dd) {
    const int rows = b * A;
    const int Z = A * K;
    const int An = Z < p.W ? Z : p.W;
    const int E = rows * M;
    const bool more = dd + 1 < D;
    const PkDiv divA(A), divZ(Z), divAn(An);
    const float *pp = p.part + (size_t)(dd & 1) * p.NC * PK_MAXELL;
    // ---- one round trip: partial sums of every consumer into registers; the
    // tables of the next depth and the current branches' states straight into
    // LDS.  Thread (eq, sg) takes consumers PK_XS sg .. PK_XS sg + PK_XS - 1
    // of entries 4 eq .. 4 eq + 3 (entries 256+ in a second pass).
    const __amdgpu_buffer_rsrc_t prs = pk_rsrc(pp, (uint32_t)(p.NC * PK_MAXELL * 4));
    const int eq = tid & 63, sg = tid >> 6;
    float4 xs[PK_XS];
#pragma unroll
    for (int v = 0; v < PK_XS; ++v) {
      xs[v] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (4 * eq < E && PK_XS * sg + v < p.NC)
        xs[v] = pk_get4(prs, (uint32_t)(((PK_XS * sg + v) * PK_MAXELL + 4 * eq) * 4));
    }
    if (more) {
      pk_dma<PK_COHERENT>(red, nks * 3 * pk_rp(rows) * 4,
                          [&](int ci) { return reinterpret_cast<const float *>(Tcur + 8 * ci); });
      if (dd > 0) load_gis(dd + 1);
      const int qc = PK_CU / 4 * M;   // chunks per request: PK_CU units x M candidates
      pk_dma<0>(gsl, b * qc, [&](int ci) {
        const int q = divQC(ci);
        return p.G + ((size_t)(q * D + dd + 1) * s + j0) * M + 4 * (ci - q * qc);
      });
    }
    float gval = 0.f;
    if (tid < E) gval = p.g[((size_t)divA(row0) * D + dd) * M + jj0];
    // raw token, clamped only after the loads above have landed
    const int tq = tid < bM ? row0 : b - 1, tj = tid < bM ? jj0 : M - 1;
    const int tokraw = p.C[((size_t)tq * D + dd) * M + tj];
    for (int half = 0;; ++half) {
      if (4 * eq + 256 * half < E) {
        float4 t = xs[0];
#pragma unroll
        for (int v = 1; v < PK_XS; ++v) { t.x += xs[v].x; t.y += xs[v].y; t.z += xs[v].z; t.w += xs[v].w; }
        *reinterpret_cast<float4 *>(stage + sg * PK_MAXELL + 4 * eq + 256 * half) = t;
      }
      if (half == 1 || E <= 256) break;
#pragma unroll
      for (int v = 0; v < PK_XS; ++v) {
        xs[v] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (4 * eq + 256 < E && PK_XS * sg + v < p.NC)
          xs[v] = pk_get4(prs, (uint32_t)(((PK_XS * sg + v) * PK_MAXELL + 256 + 4 * eq) * 4));
      }
    }
    if (tid < bM) ctok[tid] = max(tokraw, 0);
    __builtin_amdgcn_s_waitcnt(0);   // direct-to-LDS copies have landed
    __syncthreads();
    // ---- state projection of every current branch (MFMA over the published
    // three-term splits; see pk_put_state).  Only issued here: the selection
    // below runs while the matrix cores work, the sums are used after it.
    const int rp = pk_rp(rows);
    f32x4 acc[PK_NMT];
#pragma unroll
    for (int mt = 0; mt < PK_NMT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // (zero-state steps: the product is zero and the state part is b_hh)
    if (more && !p.markov) {
      const int npass = pk_npass(rows);
      // fragments of k-step i + 1 are read while those of k-step i feed the
      // matrix cores; slots past the 3 x rp used ones share their columns
      // with used slots of earlier passes, so they must contribute zero
      auto frags = [&](int i, uint4 (&f)[3]) {
        const int ks = wave + PK_WAVES * i;
#pragma unroll
        for (int ps = 0; ps < 3; ++ps) {
          const bool ok = ks < nks && ps < npass && ps * 16 + lr < 3 * rp;
          const uint4 v = *reinterpret_cast<const uint4 *>(
              sfr + (ok ? (ks * 3 * rp + ps * 16 + lr) * 32 + g * 8 : 0));
          f[ps] = ok ? v : make_uint4(0u, 0u, 0u, 0u);
        }
      };
      uint4 fc[3], fn[3];
      frags(0, fc);
#pragma unroll
      for (int i = 0; i < PK_HKS; ++i) {
        if (i + 1 < PK_HKS) frags(i + 1, fn);
        if (wave + PK_WAVES * i < nks) {
#pragma unroll
          for (int ps = 0; ps < 3; ++ps)
            if (ps < npass) {
#pragma unroll
              for (int mt = 0; mt < PK_NMT; ++mt) acc[mt] = mfma(wh[i][mt], fc[ps], acc[mt]);
            }
        }
#pragma unroll
        for (int ps = 0; ps < 3; ++ps) fc[ps] = fn[ps];
      }
    }
    // ---- selection, one thread per (branch, candidate): log-softmax over M.
    // When M is a power of two a branch's M candidates are M aligned lanes of
    // one wave: max and sum are lane butterflies (every lane of a group gets
    // the same bits), each thread keeps its own logit in a register and the
    // group needs no workgroup barrier.
    const bool act = tid < E;
    const bool lanes = (M & (M - 1)) == 0;
    float ev = 0.f;
    if (act) {
      float v = 0.f;   // consumer groups in a fixed order
      pk_scan<float>(PK_WAVES, [&](int q) { return stage[q * PK_MAXELL + tid]; },
                     [&](float x) { v += x; });
      ev = gval + v;
      if (!lanes) ell[tid] = ev;
    }
    if (!lanes) __syncthreads();
    const int row = row0, jj = jj0;
    const float lval = ev;
    float mx = -INFINITY, sum = 0.f;
    if (lanes) {
      mx = pk_group_reduce(lval, M, [](float a, float b2) { return fmaxf(a, b2); });
      sum = pk_group_reduce(expf(lval - mx), M, [](float a, float b2) { return a + b2; });
    } else {
      if (act) {
        const float *er = ell + row * M;
        pk_scan<float>(M, [&](int j) { return er[j]; }, [&](float x) { mx = fmaxf(mx, x); });
        ex[tid] = expf(lval - mx);
      }
      __syncthreads();
      if (act) {
        const float *xr = ex + row * M;
        pk_scan<float>(M, [&](int j) { return xr[j]; }, [&](float x) { sum += x; });
      }
    }
    uint64_t mykey = 0ull;
    float lp = 0.f;
    if (act) {
      lp = lval - (mx + logf(sum));
      mykey = make_key(lp, (uint32_t)ctok[divA(row) * M + jj]);
      lpkey[tid] = mykey;
    }
    if (lanes) {
      // LDS accesses of one wave take effect in issue order
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
    } else {
      __syncthreads();
    }
    // Top-K children of each branch (log-prob desc, token asc) by rank
    if (act) {
      int rank = 0;
      const uint64_t *kr = lpkey + row * M;
      pk_scan<uint64_t>(M, [&](int j) { return kr[j]; }, [&](uint64_t x) { rank += x > mykey; });
      if (rank < K) {
        const int q = divA(row), a = row - q * A;
        const int cc = q * Z + a * K + rank;
        const float sc = __fadd_rn(__int_as_float(finfo[row * 4 + 2]), lp);
        const uint32_t lex = ((uint32_t)finfo[row * 4 + 1] << 18) | (uint32_t)ctok[q * M + jj];
        ckey[cc] = make_key(sc, lex);
        clex[cc] = lex;
        cmeta[cc] = jj;
        cpar[cc] = finfo[row * 4 + 0];
      }
    }
    __syncthreads();
    // Top-W survivors of each request (score desc, token path asc) by rank
    if (tid < b * Z) {
      const int q = divZ(tid), z = tid - q * Z;
      const uint64_t kc = ckey[tid];
      const uint64_t *kq = ckey + q * Z;
      int rank = 0;
      pk_scan<uint64_t>(Z, [&](int c2) { return kq[c2]; }, [&](uint64_t x) { rank += x > kc; });
      if (rank < An) {
        int32_t *si = sinfo + (q * An + rank) * 8;
        si[0] = off + z;                        // node id
        si[1] = q * A + divK(z);                // parent's row among the current branches
        si[3] = cmeta[tid];                     // candidate index
        si[4] = (int32_t)clex[tid];
        si[5] = __float_as_int(key_val(kc));    // score
      }
    }
    __syncthreads();
    if (tid < b * An) {
      const int q = divAn(tid);
      const uint32_t li = (uint32_t)sinfo[tid * 8 + 4];
      int rank = 0;
      pk_scan<uint32_t>(An, [&](int j) { return (uint32_t)sinfo[(q * An + j) * 8 + 4]; },
                        [&](uint32_t x) { rank += x < li; });
      sinfo[tid * 8 + 6] = rank;
    }
    __syncthreads();
    // node records of this depth, split over the consumers (read by the
    // emission kernel after this one ends); written while waiting for the
    // next hand-off, from LDS that stays put until the next selection
    auto write_records = [&]() {
      const int per = divNC(b * Z + p.NC - 1);
      for (int cc = c * per + tid; cc < min(b * Z, (c + 1) * per); cc += PK_THREADS) {
        const int q = divZ(cc), z = cc - q * Z;
        const size_t id = (size_t)q * p.t.NT + off + z;
        p.t.n_tok[id] = (int32_t)(clex[cc] & 0x3FFFFu);
        p.t.n_par[id] = cpar[cc];
        p.t.n_dep[id] = dd + 1;
        p.t.n_score[id] = key_val(ckey[cc]);
        p.t.n_lex[id] = clex[cc];
      }
      for (int i = c + p.NC * tid; i < b * An; i += p.NC * PK_THREADS) {
        const int q = divAn(i), rk = i - q * An;
        p.t.surv_hist[((size_t)q * (D + 1) + dd + 1) * p.t.Wmax + rk] = sinfo[i * 8 + 0];
      }
    };
    if (!more) {
      write_records();
      break;
    }
    // depth 0: the producers' slot 1 was not needed before the GRU step
    if (dd == 0) {
      if (!pk_wait(cflags, 0, 0u, pflags, PK_PPC, p.epoch0 + 2, p.t.status, p.host_fail, p.spin, misc)) return;
      load_gis(1);
    }
    // the fragment table under red was read before the barriers above
    // lane holds D[unit 4g + t][column lr]; the lanes of columns r, r + rp
    // and r + 2 rp (mod 16) add up row r's terms first, then every row is
    // one 16-byte run per lane
    // (DPP row_ror:n gives lane l the value of lane l - n mod 16)
    auto put_rows = [&](auto variant) {
      constexpr int RV = decltype(variant)::value;
      auto ror = [](float x, auto n) {
        return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x120 + decltype(n)::value,
                                                       0xF, 0xF, false));
      };
#pragma unroll
      for (int mt = 0; mt < PK_NMT; ++mt) {
        f32x4 v = acc[mt];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          if constexpr (RV == 8) v[t] += ror(v[t], std::integral_constant<int, 8>());
          if constexpr (RV == 5)
            v[t] += ror(v[t], std::integral_constant<int, 11>()) + ror(v[t], std::integral_constant<int, 6>());
        }
        if (lr < rows)
          *reinterpret_cast<f32x4 *>(red + ((wave * PK_NMT + mt) * 16 + lr) * 16 + 4 * g) = v;
      }
    };
    if (rp == 8) put_rows(std::integral_constant<int, 8>());
    else if (rp == 5) put_rows(std::integral_constant<int, 5>());
    else put_rows(std::integral_constant<int, 16>());
    __syncthreads();
    const PkDiv div16r(16 * rows);
    for (int i = tid; i < PK_NMT * 16 * rows; i += PK_THREADS) {
      const int mt = div16r(i), rem = i - mt * 16 * rows, row = rem >> 4, u = rem & 15;
      float v = bhh[(mt / PK_HALF) * PK_CU + (mt % PK_HALF) * 16 + u];
      float w8[PK_WAVES];
#pragma unroll
      for (int wv = 0; wv < PK_WAVES; ++wv) w8[wv] = red[((wv * PK_NMT + mt) * 16 + row) * 16 + u];
#pragma unroll
      for (int wv = 0; wv < PK_WAVES; ++wv) v += w8[wv];
      ghs[(mt * 16 + row) * 16 + u] = v;
    }
    if (dd == 0) __builtin_amdgcn_s_waitcnt(0);   // the copy of slot 1 has landed
    __syncthreads();

    // ---- GRU step of the survivors for this workgroup's PK_CU units
    const int nrow = b * An;
    if (tid < nrow * PK_CU) {
      const int i = tid / PK_CU, u = tid - i * PK_CU;
      const int q = divAn(i);
      const int pr = sinfo[i * 8 + 1], jc = sinfo[i * 8 + 3];
      const float *a = gis + (q * M + jc) * 3 * PK_CU;
      const int half = u >> 4, ul = u & 15;
      const float h = p.markov ? 0.f : sn_cur[pr * PK_CU + u];
      const float *gh = ghs + (half * 16 + pr) * 16 + ul;   // gate g at + g * PK_HALF * 256
      const float r = 1.f / (1.f + expf(-(a[u] + gh[0])));
      const float z = 1.f / (1.f + expf(-(a[PK_CU + u] + gh[PK_HALF * 256])));
      const float n = tanhf(a[2 * PK_CU + u] + r * gh[2 * PK_HALF * 256]);
      const float hn = (1.f - z) * n + z * h;
      sn_nxt[i * PK_CU + u] = hn;
      pk_put_state(Tnext, c, nrow, i, u, hn);
    }
    for (int i = tid; i < nrow; i += PK_THREADS) {
      finfo[i * 4 + 0] = sinfo[i * 8 + 0];
      finfo[i * 4 + 1] = sinfo[i * 8 + 6];
      finfo[i * 4 + 2] = sinfo[i * 8 + 5];
    }
    __syncthreads();
    // partial corrected logits of depth dd+1 over this workgroup's units
    float *pn = p.part + ((size_t)((dd + 1) & 1) * p.NC + c) * PK_MAXELL;
    if (tid < nrow * M) {
      const int i = row0, j = jj0, q = divAn(i);
      const float *gq = gsl + q * PK_CU * M + j;
      const float *sq = sn_nxt + i * PK_CU;
      float acc = 0.f;
#pragma unroll
      for (int u0 = 0; u0 < PK_CU; u0 += 8) {
        float gv[8], sv[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) { gv[k] = gq[(u0 + k) * M]; sv[k] = sq[u0 + k]; }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < 8; ++k) acc += gv[k] * sv[k];
      }
      pk_put(pn + tid, acc);
    }
    pk_raise(cflags + c * 64, p.epoch0 + dd + 2);
    write_records();
    // producer slot dd + 2 holds the candidates of depth dd + 1
    const uint32_t pe = p.epoch0 + (dd + 2 < D ? dd + 3 : D);
    if (!pk_wait(cflags, p.NC, p.epoch0 + dd + 2, pflags, PK_PPC, pe, p.t.status, p.host_fail, p.spin, misc)) return;
    uint16_t *tmp = Tcur; Tcur = Tnext; Tnext = tmp;
    float *tn = sn_cur; sn_cur = sn_nxt; sn_nxt = tn;
    off += Z;
    A = An;
  }
}

__global__ __launch_bounds__(PK_THREADS) void k_depth_persistent(PKParams p) {
  extern __shared__ __align__(16) uint8_t smem[];
  if ((int)blockIdx.x < p.NC) pk_consumer(p, smem);
  else pk_producer(p, smem);
}

// ---------------------------------------------------------------- host side
bool persist_eligible(int b, int D, int M, int K, int W, int s, int e, int r, int wtype,
                      size_t lds_max) {
  if (wtype != WT_BF16 || s % 128 || e % 128) return false;
  if (s > 32 * PK_HKS * PK_WAVES || e > 32 * PK_KSW * PK_WAVES || D > PK_MAXD) return false;
  if (b * W > PK_ROWS || b * M > PK_MAXC || (long long)b * W * M > PK_MAXELL) return false;
  if ((long long)b * W * K > PK_MAXZ) return false;
  if (r > 32 * CT_MAXKS || r % 8) return false;   // correction-table fragments
  return pk_layout().total <= lds_max;
}

size_t persist_flag_words(int s) { return (size_t)(s / PK_CU + s / PK_PU) * 64; }
size_t persist_part_floats(int s) { return (size_t)2 * (s / PK_CU) * PK_MAXELL; }
size_t persist_gitab_floats(int s, int D) { return (size_t)D * PK_MAXC * 3 * s; }
size_t persist_terms_floats(int s) { return (size_t)(s / 32) * PK_SLOTS * 32 / 2; }

hipError_t persist_prepare(int s) {
  (void)s;
  return hipFuncSetAttribute(reinterpret_cast<const void *>(&k_depth_persistent),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)pk_layout().total);
}

size_t corr_w1t_elems(int s, int r) { return (size_t)s * ((r + 31) & ~31); }

hipError_t launch_transpose_w1s(const void *W1, int r, int s, int d, int ldw1, void *W1t,
                                hipStream_t st) {
  const size_t n = corr_w1t_elems(s, r);
  hipLaunchKernelGGL(k_transpose_w1s, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                     static_cast<const uint16_t *>(W1), r, s, d, ldw1,
                     static_cast<uint16_t *>(W1t));
  return hipGetLastError();
}

hipError_t launch_corr_tables(int rows, int M, int r, int s, const void *W2, const void *W1t,
                              const int32_t *C, const float *Cl, const float *uH, float *G,
                              float *g, hipStream_t st) {
  dim3 grid((s + CT_NB - 1) / CT_NB, (rows + 15) / 16);
  hipLaunchKernelGGL(k_corr_tables, grid, dim3(CT_THREADS), 0, st, rows, M, r, s,
                     static_cast<const uint16_t *>(W2), static_cast<const uint16_t *>(W1t), C, Cl,
                     uH, G, g);
  return hipGetLastError();
}

hipError_t launch_depth_persistent(const PersistArgs &a, bool cooperative, hipStream_t st) {
  if (a.s % 128 || a.D < 1 || a.D > PK_MAXD) return hipErrorInvalidValue;
  PKParams p{};
  p.b = a.b; p.D = a.D; p.M = a.M; p.K = a.K; p.W = a.W; p.s = a.s; p.e = a.e; p.V = a.V;
  p.NC = a.s / PK_CU;
  p.NP = a.s / PK_PU;
  p.W_ih = static_cast<const uint16_t *>(a.W_ih);
  p.W_hh = static_cast<const uint16_t *>(a.W_hh);
  p.Emb = static_cast<const uint16_t *>(a.Emb);
  p.b_ih = a.b_ih; p.b_hh = a.b_hh; p.C = a.C; p.root = a.root; p.G = a.G; p.g = a.g;
  p.T0 = reinterpret_cast<uint16_t *>(a.T0);
  p.T1 = reinterpret_cast<uint16_t *>(a.T1);
  p.part = a.part; p.gitab = a.gitab; p.flags = a.flags;
  p.epoch0 = a.epoch0;
  p.markov = a.markov;
  p.host_fail = a.host_fail;
  p.spin = a.spin ? a.spin : PK_SPIN;
  p.t = a.t;
  // Every workgroup needs a whole CU (LDS) and all of them must run at once.
  // A plain launch onto an otherwise idle device places them all; the flag
  // waits detect the case where they could not be (see pk_wait), and the
  // caller then switches to cooperative launches, which guarantee it at a
  // higher launch cost.
  if (!cooperative) {
    hipLaunchKernelGGL(k_depth_persistent, dim3(p.NC + p.NP), dim3(PK_THREADS), pk_layout().total,
                       st, p);
    return hipGetLastError();
  }
  void *args[] = {&p};
  return hipLaunchCooperativeKernel(reinterpret_cast<const void *>(&k_depth_persistent),
                                    dim3(p.NC + p.NP), dim3(PK_THREADS), args, pk_layout().total, st);
}

}  // namespace dtree
