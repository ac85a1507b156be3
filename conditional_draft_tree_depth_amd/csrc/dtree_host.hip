// Host runtime of libdtree.so: argument checks, workspace, launch sequence.
//
// One round (dtree_build_round) enqueues, on the caller's stream and with no
// host synchronisation:
//   K1  base logits + fused per-slice Top-M      (k_lmhead.hip)
//   K1b merge of the slices -> C, Cl             (k_lmhead.hip)
//   K2  uH = W1[:, :d] Hq, root GRU state        (k_gemm.hip)
//   for each depth: u = uH + W1[:, d:] S, corrected logits of the M
//       candidates, selection, GRU step of the survivors  (k_gemm/k_depth)
//   K4  global Top-B, canonical order, mask      (k_topb.hip)
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <type_traits>

#include "dtree.h"
#include "kernels.hpp"

using namespace dtree;

namespace {
thread_local std::string g_create_err;

struct Ws {
  uint64_t *part = nullptr;
  int32_t *C = nullptr;
  float *Cl = nullptr, *uH = nullptr, *S[2] = {nullptr, nullptr};
  // per depth: [u | W_hh S + b_hh] of every expanded branch, [b * W, r + 3s]
  float *uh = nullptr;
  float *ell = nullptr, *gi = nullptr;
  uint64_t *ckey = nullptr;   // per depth: children's selection keys [b * W * K]
  int32_t *ccand = nullptr;   //   and candidate indices
  uint32_t *selflag = nullptr; // [b, 64] arrival flags of the batched selection
  float *sscore[2] = {nullptr, nullptr};   // survivors' scores (batched selection)
  void *wcat = nullptr;      // [W1[:, d:] ; W_hh], [r + 3s, s] in the weight dtype
  int32_t *n_tok = nullptr, *n_par = nullptr, *n_dep = nullptr;
  float *n_score = nullptr;
  uint32_t *n_lex = nullptr;
  int32_t *surv[2] = {nullptr, nullptr}, *rank[2] = {nullptr, nullptr};
  int32_t *surv_hist = nullptr, *gidx_tok = nullptr, *gidx_par = nullptr, *sel = nullptr;
  // GRU input projections of the round's candidates, made before the
  // multi-kernel depth loop: one row per distinct token (or per candidate
  // when few), [min(b D M, V), 3s]; each survivor's candidate row; the
  // distinct-token tables (first row per token [V], representatives' positions,
  // distinct tokens, candidate row -> distinct position, count)
  float *gi_all = nullptr;
  int32_t *gidx_cand = nullptr;
  uint64_t *first_row = nullptr;
  int32_t *cidx_tmp = nullptr, *uniq = nullptr, *rowmap = nullptr, *ucount = nullptr,
          *lpos = nullptr, *btot = nullptr;
  size_t gi_rows = 0;
  uint32_t *status = nullptr;
  // persistent depth loop: correction tables, partial sums, arrival flags
  float *G = nullptr, *g = nullptr, *pk_part = nullptr, *gitab = nullptr, *pk_terms = nullptr;
  uint16_t *w1t = nullptr;   // W1[:, d:]^T, padded (correction tables)
  uint16_t *hb = nullptr;    // bf16 hidden rows of the round (LM-head kernel)
  float *logits = nullptr;   // [b * D, V] base logits when 32 or more rows (tiled product)
  uint32_t *gmax = nullptr;  //   with it: [b * D, lmhead_groups(V)] column-group maxima
  uint32_t *rbound = nullptr;  //   and [b * D] the rows' list bounds
  int32_t *ovf = nullptr;      //   and [ceil(b * D / 8), P] overflow flags
  uint16_t *S3[2] = {nullptr, nullptr};   // states as bf16 planes (many branches)
  uint32_t *flags = nullptr;
  HeapBufs hp;               // sequential best-first builder (allocated on first use)
};

int superarbol_nodes(int D, int K, int W) {
  long long A = 1, NT = 1;
  for (int dd = 0; dd < D; ++dd) {
    NT += A * K;
    A = A * K < W ? A * K : W;
    if (NT > (1 << 30)) return -1;
  }
  return (int)NT;
}
}  // namespace

struct dtree_ctx {
  int device = 0;
  dtree_weights w{};
  dtree_caps caps{};
  int P = 0, NTcap = 0;
  size_t k1_smem = 0, lds_max = 0;
  int k1_ring = 0;
  Ws ws;
  std::string err;
  bool has_round = false;
  bool last_heap = false;   // the last round ran the sequential best-first builder
  dtree_params last{};
  int last_batch = 0, last_NT = 0;
  // persistent depth loop: available for this context, and the arrival
  // epoch of the next round (flags only ever grow, so they need no reset)
  bool pk = false;
  bool sel_batch = false;  // selection over many workgroups (correction logits inside)
  int scoring = DTREE_SCORE_CONDITIONAL;
  int builder = DTREE_BUILD_DEPTHWISE;
  uint32_t tok_epoch = 0;   // distinct-token tables: grows by one per round that uses them
  int pk_rows = 0;
  // persistent depth loop: plain launches until one of its waits runs out
  // (it then stores 1 to *pk_fail, host memory the kernel writes through
  // pk_fail_dev); from then on cooperative launches
  bool pk_coop = false;
  uint32_t *pk_fail = nullptr, *pk_fail_dev = nullptr;
  uint32_t pk_spin = 0;   // 0: the kernel's default limit
  uint32_t epoch = 0;
  // stage timing: kProfRounds rounds x (DTREE_NSTAGES + 1) events
  bool prof = false;
  int prof_n = 0;
  hipEvent_t *prof_ev = nullptr;
  // errors go here instead of err when set (a context on the stack of the
  // allocation-free entry point: no host allocation for the message)
  char *err_buf = nullptr;
  size_t err_cap = 0;
};

static constexpr int kProfRounds = 4096;
static const char *g_static_err_text();

static dtree_status fail(dtree_ctx *c, dtree_status s, const std::string &m) {
  if (c && c->err_buf) std::snprintf(c->err_buf, c->err_cap, "%s", m.c_str());
  else if (c) c->err = m;
  else g_create_err = m;
  return s;
}
static dtree_status fail(dtree_ctx *c, dtree_status s, const char *m) {
  if (c && c->err_buf) std::snprintf(c->err_buf, c->err_cap, "%s", m);
  else if (c) c->err = m;
  else g_create_err = m;
  return s;
}

#define HIPCHK(ctx, expr)                                                                \
  do {                                                                                 \
    hipError_t e_ = (expr);                                                            \
    if (e_ != hipSuccess)                                                              \
      return fail(ctx, DTREE_E_HIP, std::string(#expr) + ": " + hipGetErrorString(e_)); \
  } while (0)

namespace {
struct DeviceGuard {
  int prev = -1;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    if (prev != dev) (void)hipSetDevice(dev);
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

template <typename T>
hipError_t alloc(T **p, size_t n) {
  return hipMalloc(reinterpret_cast<void **>(p), (n ? n : 1) * sizeof(T));
}

void free_ws(Ws &ws) {
  void *ptrs[] = {ws.part, ws.hb, ws.C, ws.Cl, ws.uH, ws.S[0], ws.S[1], ws.uh, ws.ell, ws.ckey,
                  ws.ccand, ws.selflag, ws.sscore[0], ws.sscore[1], ws.gi, ws.wcat, ws.n_tok, ws.n_par, ws.n_dep,
                  ws.n_score, ws.n_lex, ws.surv[0], ws.surv[1], ws.rank[0], ws.rank[1], ws.surv_hist, ws.gidx_tok, ws.gidx_par, ws.sel,
                  ws.status, ws.G, ws.g, ws.pk_part, ws.gitab, ws.pk_terms, ws.w1t, ws.flags,
                  ws.logits, ws.gmax, ws.rbound, ws.ovf, ws.S3[0], ws.S3[1], ws.gi_all, ws.gidx_cand, ws.first_row,
                  ws.cidx_tmp, ws.uniq, ws.rowmap, ws.ucount, ws.lpos, ws.btot,
                  ws.hp.tok, ws.hp.par, ws.hp.dep, ws.hp.score, ws.hp.gref, ws.hp.pv,
                  ws.hp.nnodes, ws.hp.pops, ws.hp.ex, ws.hp.S, ws.hp.UH, ws.hp.gi};
  for (void *p : ptrs)
    if (p) (void)hipFree(p);
  ws = Ws();
}
}  // namespace

static void prof_mark(dtree_ctx *ctx, int stage, hipStream_t st) {
  if (ctx->prof && ctx->prof_n < kProfRounds)
    (void)hipEventRecord(ctx->prof_ev[ctx->prof_n * (DTREE_NSTAGES + 1) + stage], st);
}

extern "C" int32_t dtree_superarbol_nodes(const dtree_params *p) {
  if (!p || p->D < 1 || p->K < 1 || p->W < 1) return -1;
  return superarbol_nodes(p->D, p->K, p->W);
}

extern "C" int32_t dtree_heap_nodes(const dtree_params *p) {
  if (!p || p->K < 1 || p->B < 1) return -1;
  const long long n = (long long)p->K * (p->B + 1) + 1;
  return n > (1 << 30) ? -1 : (int32_t)n;
}

extern "C" dtree_status dtree_create(const dtree_weights *w, const dtree_caps *caps, int device,
                                     dtree_ctx **out) {
  g_create_err.clear();
  if (!w || !caps || !out) return fail(nullptr, DTREE_E_ARG, "null argument");
  *out = nullptr;
  if (w->wtype != DTREE_F32 && w->wtype != DTREE_BF16)
    return fail(nullptr, DTREE_E_DTYPE, "wtype must be DTREE_F32 or DTREE_BF16");
  if (w->d < 1 || w->V < 1 || w->e < 1 || w->s < 1 || w->r < 1)
    return fail(nullptr, DTREE_E_ARG, "d, V, e, s, r must be >= 1");
  if (w->V > (1 << 18)) return fail(nullptr, DTREE_E_SHAPE, "V must be <= 262144");
  if (!w->W_lm || !w->Emb || !w->W_ih || !w->W_hh || !w->W1 || !w->W2)
    return fail(nullptr, DTREE_E_ARG, "null weight pointer");
  if (w->wtype == DTREE_BF16) {
    if (w->d % 128) return fail(nullptr, DTREE_E_SHAPE, "bf16 weights need d % 128 == 0");
    if (reinterpret_cast<uintptr_t>(w->W_lm) % 16)
      return fail(nullptr, DTREE_E_ARG, "W_lm must be 16-byte aligned");
  }
  const dtree_caps &c = *caps;
  if (c.max_batch < 1 || c.max_D < 1 || c.max_M < 1 || c.max_K < 1 || c.max_W < 1 || c.max_B < 1)
    return fail(nullptr, DTREE_E_ARG, "caps must be >= 1");
  if (c.max_D > 31) return fail(nullptr, DTREE_E_SHAPE, "max_D must be <= 31");
  if (c.max_M > 128) return fail(nullptr, DTREE_E_SHAPE, "max_M must be <= 128");
  if (c.max_W > 512) return fail(nullptr, DTREE_E_SHAPE, "max_W must be <= 512");
  if ((long long)c.max_W * c.max_K > 1024)
    return fail(nullptr, DTREE_E_SHAPE, "max_W * max_K must be <= 1024");
  const int NTcap = superarbol_nodes(c.max_D, c.max_K, c.max_W);
  if (NTcap < 0 || NTcap > 8192)
    return fail(nullptr, DTREE_E_SHAPE, "superarbol of the caps exceeds 8192 nodes");

  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || device < 0 || device >= ndev)
    return fail(nullptr, DTREE_E_DEVICE, "no such HIP device");
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device) != hipSuccess)
    return fail(nullptr, DTREE_E_DEVICE, "device query failed");
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(nullptr, DTREE_E_DEVICE, std::string("needs gfx950, found ") + prop.gcnArchName);

  dtree_ctx *ctx = new (std::nothrow) dtree_ctx();
  if (!ctx) return fail(nullptr, DTREE_E_NOMEM, "host allocation failed");
  ctx->device = device;
  ctx->w = *w;
  ctx->caps = c;
  ctx->NTcap = NTcap;
  ctx->lds_max = prop.sharedMemPerBlock;
  ctx->P = lmhead_partitions(w->V, w->wtype, (w->r + 15) / 16);
  ctx->k1_ring = lmhead_ring(w->d, w->wtype, ctx->lds_max);
  ctx->k1_smem = lmhead_smem(w->d, w->wtype, ctx->k1_ring);
  const size_t cl_smem = corr_logits_smem(c.max_W, c.max_M, w->r, w->wtype);
  const size_t tb_smem = topb_smem(NTcap, c.max_B);
  auto reject = [&](dtree_status s, const std::string &m) {
    delete ctx;
    return fail(nullptr, s, m);
  };
  if (ctx->k1_smem > ctx->lds_max) return reject(DTREE_E_SHAPE, "d too large for the LM-head LDS tile");
  if (topm_merge_smem(ctx->P) > 131072) return reject(DTREE_E_SHAPE, "vocabulary too large for the Top-M merge");
  if (cl_smem > ctx->lds_max) return reject(DTREE_E_SHAPE, "max_M * r too large for the correction LDS tile");
  if (tb_smem > ctx->lds_max) return reject(DTREE_E_SHAPE, "superarbol too large for the Top-B LDS sort");

  DeviceGuard dg(device);
  Ws &ws = ctx->ws;
  const size_t rows = (size_t)c.max_batch * c.max_D;
  const size_t bw = (size_t)c.max_batch * c.max_W;
  const int s = w->s, r = w->r;
  hipError_t e = hipSuccess;
  auto A = [&](hipError_t x) { if (e == hipSuccess) e = x; };
  A(alloc(&ws.part, rows * ctx->P * K1_LSTRIDE));
  // counters of the merge fused into the LM-head kernel: only ever grow
  A(alloc(&ws.C, rows * c.max_M));
  A(alloc(&ws.Cl, rows * c.max_M));
  A(alloc(&ws.uH, rows * r));
  A(alloc(&ws.hb, (size_t)((rows + 15) / 16 * 16) * w->d));
  if (lmhead_tiled_ok((int)rows, w->d, w->wtype == DTREE_BF16 ? WT_BF16 : WT_F32)) {
    A(alloc(&ws.logits, rows * (size_t)w->V));
    A(alloc(&ws.gmax, rows * (size_t)lmhead_groups(w->V)));
    A(alloc(&ws.rbound, rows));
    A(alloc(&ws.ovf, (rows + 7) / 8 * (size_t)ctx->P));
  }
  A(alloc(&ws.S[0], bw * s));
  A(alloc(&ws.S[1], bw * s));
  A(alloc(&ws.uh, bw * (r + 3 * s)));
  // 256 or more branches: the state products run as tiled bf16 products over
  // the bf16 plane split of the states
  if (w->wtype == DTREE_BF16 && s % 64 == 0 && bw >= 256)
    for (int i = 0; i < 2; ++i) A(alloc(&ws.S3[i], bw * STATE_PLANES * s));
  A(alloc(&ws.ell, bw * c.max_M));
  A(alloc(&ws.ckey, bw * c.max_K));
  A(alloc(&ws.ccand, bw * c.max_K));
  A(alloc(&ws.selflag, (size_t)c.max_batch * 64));
  for (int i = 0; i < 2; ++i) A(alloc(&ws.sscore[i], bw));
  A(alloc(&ws.gi, bw * 3 * s));
  const size_t esz_w = w->wtype == DTREE_BF16 ? 2 : 4;
  A(alloc(reinterpret_cast<uint8_t **>(&ws.wcat), (size_t)(r + 3 * s) * s * esz_w));
  if (e == hipSuccess)
    A(launch_concat_state_weights(w->W1, w->W_hh, r, s, w->d,
                                  w->wtype == DTREE_BF16 ? WT_BF16 : WT_F32, ws.wcat, nullptr));
  if (e == hipSuccess) A(hipDeviceSynchronize());   // rounds may run on any stream
  const size_t nt = (size_t)c.max_batch * NTcap;
  A(alloc(&ws.n_tok, nt));
  A(alloc(&ws.n_par, nt));
  A(alloc(&ws.n_dep, nt));
  A(alloc(&ws.n_score, nt));
  A(alloc(&ws.n_lex, nt));
  for (int i = 0; i < 2; ++i) { A(alloc(&ws.surv[i], bw)); A(alloc(&ws.rank[i], bw)); }
  A(alloc(&ws.surv_hist, (size_t)c.max_batch * (c.max_D + 1) * c.max_W));
  A(alloc(&ws.gidx_tok, bw));
  A(alloc(&ws.gidx_par, bw));
  if (w->wtype == DTREE_BF16) {
    const size_t ncand = rows * c.max_M;
    ws.gi_rows = ncand < (size_t)w->V ? ncand : (size_t)w->V;
    A(alloc(&ws.gi_all, ws.gi_rows * 3 * s));
    A(alloc(&ws.gidx_cand, bw));
    A(alloc(&ws.first_row, (size_t)w->V));
    A(alloc(&ws.cidx_tmp, ncand));
    A(alloc(&ws.uniq, ws.gi_rows));
    A(alloc(&ws.rowmap, ncand));
    A(alloc(&ws.ucount, 1));
    A(alloc(&ws.lpos, ncand));
    A(alloc(&ws.btot, ncand / 256 + 1));
    if (e == hipSuccess) A(hipMemset(ws.first_row, 0, (size_t)w->V * 8));
  }
  A(alloc(&ws.sel, (size_t)c.max_batch * c.max_B));
  A(alloc(&ws.status, 1));
  // the persistent depth loop needs bf16 weights and MFMA-friendly GRU sizes
  auto al16 = [](const void *p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; };
  ctx->pk = w->wtype == DTREE_BF16 && s % 128 == 0 && w->e % 128 == 0 && al16(w->Emb) &&
            al16(w->W_ih) && al16(w->W_hh) && al16(w->W2) &&
            persist_eligible(1, c.max_D, 1, 1, 1, s, w->e, r, WT_BF16, ctx->lds_max);
  if (ctx->pk) {
    const int cand = c.max_batch * c.max_M < 64 ? c.max_batch * c.max_M : 64;
    ctx->pk_rows = cand * c.max_D;
    A(alloc(&ws.G, (size_t)ctx->pk_rows * s));
    A(alloc(&ws.g, (size_t)ctx->pk_rows));
    A(alloc(&ws.pk_part, persist_part_floats(s)));
    A(alloc(&ws.gitab, persist_gitab_floats(s, c.max_D)));
    A(alloc(&ws.pk_terms, 2 * persist_terms_floats(s)));
    A(alloc(&ws.w1t, corr_w1t_elems(s, r)));
    if (e == hipSuccess) A(launch_transpose_w1s(w->W1, r, s, w->d, w->d + s, ws.w1t, nullptr));
    A(alloc(&ws.flags, persist_flag_words(s)));
    if (e == hipSuccess) A(hipMemset(ws.flags, 0, persist_flag_words(s) * 4));
    if (e == hipSuccess) A(hipHostMalloc(reinterpret_cast<void **>(&ctx->pk_fail), sizeof(uint32_t),
                                         hipHostMallocMapped));
    if (e == hipSuccess) {
      *ctx->pk_fail = 0u;
      A(hipHostGetDevicePointer(reinterpret_cast<void **>(&ctx->pk_fail_dev), ctx->pk_fail, 0));
    }
    if (e == hipSuccess) A(hipDeviceSynchronize());
  }
  if (e != hipSuccess) {
    free_ws(ws);
    if (ctx->pk_fail) (void)hipHostFree(ctx->pk_fail);
    return reject(DTREE_E_NOMEM, std::string("workspace: ") + hipGetErrorString(e));
  }
  // (every kernel may use up to the device's LDS per workgroup: contexts and
  // allocation-free calls of other sizes never lower each other's limits)
  hipError_t pe = lmhead_prepare(w->wtype, ctx->k1_ring, ctx->lds_max);
  if (pe == hipSuccess) pe = corr_logits_prepare(w->wtype, ctx->lds_max);
  if (pe == hipSuccess) pe = topb_prepare(ctx->lds_max);
  if (pe == hipSuccess) pe = gemm_prepare();
  // correction logits inside the (batched) selection kernel: bf16 W2 rows
  // of 16-byte pieces
  ctx->sel_batch = w->wtype == DTREE_BF16 && r % 8 == 0 && r <= 512 &&
                   reinterpret_cast<uintptr_t>(w->W2) % 16 == 0 &&
                   branch_select_smem(r) + 32768 <= ctx->lds_max;
  if (pe == hipSuccess && ctx->sel_batch) pe = branch_select_prepare(ctx->lds_max);
  if (pe == hipSuccess && ctx->pk) pe = persist_prepare(s);
  if (pe != hipSuccess) {
    free_ws(ws);
    return reject(DTREE_E_HIP, std::string("kernel attributes: ") + hipGetErrorString(pe));
  }
  *out = ctx;
  return DTREE_OK;
}

static dtree_status enqueue_round(dtree_ctx *ctx, const dtree_params *p, int32_t batch,
                                  const float *H, const int32_t *root, int32_t *tok,
                                  int32_t *parent, int32_t *depth, float *score, uint8_t *mask,
                                  int32_t *n_nodes, hipStream_t st);

extern "C" dtree_status dtree_build_round(dtree_ctx *ctx, const dtree_params *p, int32_t batch,
                                          const float *H, const int32_t *root, int32_t *tok,
                                          int32_t *parent, int32_t *depth, float *score,
                                          uint8_t *mask, int32_t *n_nodes, void *stream) {
  if (!ctx) return DTREE_E_ARG;
  ctx->err.clear();
  if (!p) return fail(ctx, DTREE_E_ARG, "null params");
  if (!H || !root || !tok || !parent || !depth || !score || !mask || !n_nodes)
    return fail(ctx, DTREE_E_ARG, "null input or output pointer");
  const dtree_caps &c = ctx->caps;
  const int D = p->D, M = p->M, K = p->K, W = p->W, B = p->B;
  if (batch < 1 || batch > c.max_batch) return fail(ctx, DTREE_E_ARG, "batch outside [1, max_batch]");
  if (D < 1 || D > c.max_D) return fail(ctx, DTREE_E_ARG, "D outside [1, max_D]");
  if (M < 1 || M > c.max_M || M > ctx->w.V) return fail(ctx, DTREE_E_ARG, "M outside [1, min(max_M, V)]");
  if (K < 1 || K > M || K > c.max_K) return fail(ctx, DTREE_E_ARG, "K outside [1, min(M, max_K)]");
  if (W < 1 || W > c.max_W) return fail(ctx, DTREE_E_ARG, "W outside [1, max_W]");
  if (B < 1 || B > c.max_B) return fail(ctx, DTREE_E_ARG, "B outside [1, max_B]");
  if (!(p->beta <= 0.0f)) return fail(ctx, DTREE_E_ARG, "beta must be <= 0 (and not NaN)");
  if (std::isinf(p->beta)) return fail(ctx, DTREE_E_ARG, "beta must be finite");
  if (ctx->builder == DTREE_BUILD_HEAP && ctx->scoring == DTREE_SCORE_MARGINAL)
    return fail(ctx, DTREE_E_ARG, "the heap builder scores conditionally or with the Markov head");

  // an earlier round's depth-loop kernel could not have all its workgroups
  // resident at once (the device was shared): that round failed (status bit
  // 1); report it here, loudly, and use cooperative launches from now on
  if (ctx->pk_fail && __atomic_load_n(ctx->pk_fail, __ATOMIC_ACQUIRE)) {
    __atomic_store_n(ctx->pk_fail, 0u, __ATOMIC_RELEASE);
    ctx->pk_coop = true;
    return fail(ctx, DTREE_E_HIP,
                "an earlier round's depth loop could not run all its workgroups at once; its "
                "outputs are invalid; later rounds use cooperative launches");
  }

  DeviceGuard dg(ctx->device);
  return enqueue_round(ctx, p, batch, H, root, tok, parent, depth, score, mask, n_nodes,
                       static_cast<hipStream_t>(stream));
}

// The kernels of one round, enqueued on st (arguments already checked).
static dtree_status enqueue_round(dtree_ctx *ctx, const dtree_params *p, int32_t batch,
                                  const float *H, const int32_t *root, int32_t *tok,
                                  int32_t *parent, int32_t *depth, float *score, uint8_t *mask,
                                  int32_t *n_nodes, hipStream_t st) {
  const dtree_caps &c = ctx->caps;
  const int D = p->D, M = p->M, K = p->K, W = p->W, B = p->B;
  const dtree_weights &w = ctx->w;
  Ws &ws = ctx->ws;
  const int rows = batch * D;
  const int d = w.d, s = w.s, r = w.r;
  const int wt = w.wtype == DTREE_BF16 ? WT_BF16 : WT_F32;
  const size_t esz = wt == WT_BF16 ? 2 : 4;
  ctx->has_round = false;

  // round start (done by the first kernel of the round)
  TreeBufs tb{};
  tb.NT = ctx->NTcap;
  tb.V = w.V;
  tb.Wmax = c.max_W;
  tb.n_tok = ws.n_tok; tb.n_par = ws.n_par; tb.n_dep = ws.n_dep;
  tb.n_score = ws.n_score; tb.n_lex = ws.n_lex;
  tb.surv_hist = ws.surv_hist; tb.gidx_tok = ws.gidx_tok; tb.gidx_par = ws.gidx_par;
  tb.sel = ws.sel; tb.status = ws.status; tb.selflag = ws.selflag;
  int cur = 0;
  tb.surv_node = ws.surv[0]; tb.surv_rank = ws.rank[0];
  tb.nsurv_node = ws.surv[1]; tb.nsurv_rank = ws.rank[1];
  tb.surv_score = ws.sscore[0]; tb.nsurv_score = ws.sscore[1];

  // K1 + K1b: candidate tables
  prof_mark(ctx, 0, st);
  // bf16: the LM-head kernel also produces uH = W1[:, :d] . Hq (same operand)
  // 32 or more rows: a tiled product writes the logits, lists from those
  const bool tiled = ws.logits != nullptr && lmhead_tiled_ok(rows, d, wt);
  const bool fuse_uH = !tiled && wt == WT_BF16 && (d + s) % 8 == 0 &&
                       reinterpret_cast<uintptr_t>(w.W1) % 16 == 0;
  LMHeadArgs la{H, rows, d, w.W_lm, wt, w.V, w.lm_bias, M, ctx->P, ws.part,
                fuse_uH ? w.W1 : nullptr, d + s, r, ws.uH,
                root, batch, D + 1, tb, ctx->k1_ring, ws.hb, ws.gmax, ws.rbound, ws.ovf};
  // round start: a kernel of its own ahead of the tiled product (bf16 rows
  // for it); the streaming kernels round the rows and start the round
  // themselves
  if (tiled) HIPCHK(ctx, launch_stage_hidden(la, st));
  // the LM-head stage is timed by the kernel's own start and end (no marker
  // packets around it)
  hipEvent_t k1ev[2] = {nullptr, nullptr};
  if (ctx->prof && ctx->prof_n < kProfRounds)
    for (int i = 0; i < 2; ++i) k1ev[i] = ctx->prof_ev[ctx->prof_n * (DTREE_NSTAGES + 1) + 1 + i];
  if (tiled) HIPCHK(ctx, launch_lmhead_tiled(la, ws.logits, st, k1ev[0], k1ev[1]));
  else HIPCHK(ctx, launch_lmhead(la, st, k1ev[0], k1ev[1]));
  // the persistent depth loop's correction tables come with the merge when
  // the fused kernel fits (decided here, used below)
  const bool marginal = ctx->scoring == DTREE_SCORE_MARGINAL;
  const bool pk = !marginal && ctx->builder != DTREE_BUILD_HEAP && ctx->pk && batch * M <= 64 &&
                  batch * D * M <= ctx->pk_rows &&
                  persist_eligible(batch, D, M, K, W, s, w.e, r, wt, ctx->lds_max);
  const bool pk_fused = pk && fuse_uH && topm_tables_ok(M, r, s, w.W2, ws.w1t);
  if (pk_fused)
    HIPCHK(ctx, launch_topm_tables(ws.part, ctx->P, M, rows, r, s, w.W2, ws.w1t, ws.uH, ws.C,
                                   ws.Cl, ws.G, ws.g, st));
  else
    HIPCHK(ctx, launch_topm_merge(ws.part, ctx->P, M, rows, ws.C, ws.Cl, st));
  prof_mark(ctx, 3, st);
  // K2: uH = W1[:, :d] . Hq for every (request, depth), when not fused above
  GemmArgs g{};
  if (tiled) {   // from the bf16 hidden rows of the round start (= the rounded H)
    g = GemmArgs{rows, r, d, ws.hb, WT_BF16, d, nullptr, 0, w.W1, wt, d + s,
                 nullptr, nullptr, 0, 1, 0, 0, ws.uH, r};
    HIPCHK(ctx, launch_gemm(g, st));
  } else if (!fuse_uH) {
    g = GemmArgs{rows, r, d, H, WT_F32, d, nullptr, wt == WT_BF16 ? 1 : 0, w.W1, wt, d + s,
                 nullptr, nullptr, 0, 1, 0, 0, ws.uH, r};
    HIPCHK(ctx, launch_gemm(g, st));
  }


  // Markov scoring: each survivor's GRU step starts from a zero state, so
  // the W_hh product of the branches is not needed
  const bool markov = ctx->scoring == DTREE_SCORE_MARKOV;
  if (ctx->builder == DTREE_BUILD_HEAP) {
    // sequential best-first builder: one heap step and one state product per pop
    HeapBufs &hp = ws.hp;
    // GRU input projections of every candidate of the round [b D M, 3s]
    g = GemmArgs{rows * M, 3 * s, w.e, w.Emb, wt, w.e, ws.C, 0, w.W_ih, wt, w.e, w.b_ih, nullptr,
                 0, 1, 0, 0, hp.gi, 3 * s};
    HIPCHK(ctx, launch_gemm(g, st));
    // root state: the GRU consumes the last verified token from a zero state
    g = GemmArgs{batch, 3 * s, w.e, w.Emb, wt, w.e, ws.gidx_tok, 0, w.W_ih, wt, w.e,
                 w.b_ih, nullptr, 0, 1, 0, 0, ws.gi, 3 * s};
    HIPCHK(ctx, launch_gemm(g, st));
    HIPCHK(ctx, launch_gru_combine(batch, s, ws.gi, nullptr, nullptr, nullptr, 0, w.b_hh, nullptr,
                                   nullptr, ws.S[0], nullptr, st));
    const int ldu = r + 3 * s;
    const size_t slots = (size_t)hp.Bcap + 1;
    // [u | W_hh S + b_hh] of one state per request into expansion slot Y
    auto product = [&](const float *X, int ldx, float *Y) {
      GemmArgs gp{batch, ldu, s, X, WT_F32, ldx, nullptr, 0, ws.wcat, wt, s, w.b_hh, nullptr,
                  0, 1, 0, 0, Y, (int)(slots * ldu)};
      gp.bias_n0 = r;
      return launch_gemm(gp, st);
    };
    HIPCHK(ctx, product(ws.S[0], s, hp.UH));
    prof_mark(ctx, 4, st);
    HeapStepArgs ha{batch, 0, B, D, M, K, s, r, markov ? 1 : 0, w.V, p->beta, w.W2,
                    wt == WT_BF16 ? 1 : 0, ws.C, ws.Cl, ws.uH, root, ws.S[0], w.b_hh, hp};
    for (int t = 0; t < B; ++t) {
      ha.t = t;
      HIPCHK(ctx, launch_heap_step(ha, st));
      if (t + 1 < B)
        HIPCHK(ctx, product(hp.S + (size_t)(t + 1) * s, (int)(slots * s),
                            hp.UH + (size_t)(t + 1) * ldu));
    }
    prof_mark(ctx, 5, st);
    HIPCHK(ctx, launch_heap_emit(batch, B, D, hp, tok, parent, depth, score, mask, n_nodes, st));
    prof_mark(ctx, 6, st);
    if (ctx->prof && ctx->prof_n < kProfRounds) ++ctx->prof_n;
    ctx->has_round = true;
    ctx->last = *p;
    ctx->last_batch = batch;
    ctx->last_NT = 0;
    ctx->last_heap = true;
    return DTREE_OK;
  }
  ctx->last_heap = false;
  int A = 1, off = 1, sc = 0;
  if (marginal) {
    // every branch of a depth is scored by the depth's base logits Cl
    // (no correction, no GRU state): the whole depth loop is one kernel
    prof_mark(ctx, 4, st);
    HIPCHK(ctx, launch_select_marginal(batch, M, K, W, D, ws.C, ws.Cl, tb, st));
    for (int dd = 0; dd < D; ++dd) {
      off += A * K;
      A = A * K < W ? A * K : W;
    }
  } else if (pk) {
    // correction tables G = W2[C] W1[:, d:], g = Cl + W2[C] uH, then the
    // whole depth loop as one cooperative launch
    if (!pk_fused)
      HIPCHK(ctx, launch_corr_tables(batch * D * M, M, r, s, w.W2, ws.w1t, ws.C, ws.Cl, ws.uH,
                                     ws.G, ws.g, st));
    prof_mark(ctx, 4, st);
    PersistArgs pa{batch, D, M, K, W, s, w.e, w.V, w.W_ih, w.W_hh, w.Emb, w.b_ih, w.b_hh,
                   ws.C, root, ws.G, ws.g, ws.pk_terms, ws.pk_terms + persist_terms_floats(s),
                   ws.pk_part, ws.gitab, ws.flags, ctx->pk_fail_dev, ctx->pk_spin,
                   ctx->epoch, tb, markov ? 1 : 0};
    HIPCHK(ctx, launch_depth_persistent(pa, ctx->pk_coop, st));
    ctx->epoch += (uint32_t)D + 1u;
    for (int dd = 0; dd < D; ++dd) {
      off += A * K;
      A = A * K < W ? A * K : W;
    }
  } else {
    // root state: the GRU consumes the last verified token from a zero state
    g = GemmArgs{batch, 3 * s, w.e, w.Emb, wt, w.e, ws.gidx_tok, 0, w.W_ih, wt, w.e,
                 w.b_ih, nullptr, 0, 1, 0, 0, ws.gi, 3 * s};
    HIPCHK(ctx, launch_gemm(g, st));
    HIPCHK(ctx, launch_gru_combine(batch, s, ws.gi, nullptr, nullptr, nullptr, 0, w.b_hh, nullptr,
                                   nullptr, ws.S[0], ws.S3[0], st));
    // the GRU input projection depends on the token only: it is made once
    // per distinct token of the round's candidates (a tiled product whose row
    // count is read on the device), or once per candidate when they are few,
    // and each survivor's GRU step reads its token's row
    const int ncand = batch * D * M;
    int precomp = 0;   // 0: per depth, 1: per candidate, 2: per distinct token
    GemmArgs gu{};
    if (ws.gi_all) {
      gu = GemmArgs{(int)std::min((size_t)ncand, ws.gi_rows), 3 * s, w.e, w.Emb, wt, w.e, ws.uniq,
                    0, w.W_ih, wt, w.e, w.b_ih, nullptr, 0, 1, 0, 0, ws.gi_all, 3 * s};
      gu.Rdev = ws.ucount;
      // (finding the distinct tokens costs five small launches: worth it
      // with many candidates, whose tokens repeat across depths and requests)
      if (ncand > 2048 && ncand <= 262144 && gemm_rdev_ok(gu)) precomp = 2;
      else if ((size_t)ncand <= ws.gi_rows && ncand <= 4096) precomp = 1;
    }
    if (precomp == 2) {
      // the epoch runs 1 .. 2^32 - 1, then starts again at 1 (which clears the table)
      if (++ctx->tok_epoch == 0u) ctx->tok_epoch = 1u;
      HIPCHK(ctx, launch_token_dedupe(ncand, ws.C, ws.first_row, w.V, ctx->tok_epoch, ws.lpos,
                                      ws.btot, ws.cidx_tmp, ws.uniq, ws.rowmap, ws.ucount, st));
      HIPCHK(ctx, launch_gemm(gu, st));
    } else if (precomp == 1) {
      g = GemmArgs{ncand, 3 * s, w.e, w.Emb, wt, w.e, ws.C, 0, w.W_ih, wt, w.e,
                   w.b_ih, nullptr, 0, 1, 0, 0, ws.gi_all, 3 * s};
      HIPCHK(ctx, launch_gemm(g, st));
    }
    if (precomp) tb.gidx_cand = ws.gidx_cand;
    prof_mark(ctx, 4, st);
    for (int dd = 0; dd < D; ++dd) {
      // for every expanded branch, one product over its state S:
      //   u = uH[req, dd] + W1[:, d:] . S   (outputs 0 .. r-1)
      //   W_hh . S + b_hh                  (outputs r .. r+3s-1, the GRU state
      //                                      part of all of the branch's children)
      const int ldu = r + 3 * s;
      if (ws.wcat && !markov) {
        g = GemmArgs{batch * A, ldu, s, ws.S[sc], WT_F32, s, nullptr, 0, ws.wcat, wt, s, w.b_hh,
                     ws.uH, r, A, D, dd, ws.uh, ldu};
        g.add_n = r;
        g.bias_n0 = r;
        if (ws.S3[sc]) {   // the state as bf16 planes, if a tiled product takes it
          GemmArgs g3 = g;
          g3.X = ws.S3[sc];
          g3.xtype = WT_BF16;
          g3.ldx = STATE_PLANES * s;
          g3.Kd = STATE_PLANES * s;
          g3.kw = s;
          if (gemm_tiled_ok(g3)) g = g3;
        }
        HIPCHK(ctx, launch_gemm(g, st));
      } else {
        // no concatenated copy (allocation-free calls): the same two
        // products straight from W1[:, d:] and W_hh
        g = GemmArgs{batch * A, r, s, ws.S[sc], WT_F32, s, nullptr, 0,
                     static_cast<const uint8_t *>(w.W1) + (size_t)d * esz, wt, d + s, nullptr,
                     ws.uH, r, A, D, dd, ws.uh, ldu};
        HIPCHK(ctx, launch_gemm(g, st));
        if (!markov) {
          g = GemmArgs{batch * A, 3 * s, s, ws.S[sc], WT_F32, s, nullptr, 0, w.W_hh, wt, s,
                       w.b_hh, nullptr, 0, 1, 0, 0, ws.uh + r, ldu};
          HIPCHK(ctx, launch_gemm(g, st));
        }
      }
      // correction logits, log-softmax, Top-K and Top-W: one kernel over 8
      // branches per workgroup (bf16 W2), else the logits and the selection
      // as two kernels
      if (ctx->sel_batch) {
        HIPCHK(ctx, launch_branch_select(batch, A, M, K, W, D, dd, off, r, w.W2, ws.C, ws.Cl,
                                         ws.uh, ldu, tb, ws.ckey, ws.ccand, st));
      } else {
        HIPCHK(ctx, launch_corr_logits(batch, A, M, r, D, dd, w.W2, wt, ws.C, ws.Cl, ws.uh, ldu,
                                       ws.ell, st));
        HIPCHK(ctx, launch_select(batch, A, M, K, W, D, dd, off, ws.C, ws.ell, (long)A * M, M, tb,
                                  st));
      }
      const int An = A * K < W ? A * K : W;
      if (dd + 1 < D) {
        if (!precomp) {
          g = GemmArgs{batch * An, 3 * s, w.e, w.Emb, wt, w.e, ws.gidx_tok, 0, w.W_ih, wt, w.e,
                       w.b_ih, nullptr, 0, 1, 0, 0, ws.gi, 3 * s};
          HIPCHK(ctx, launch_gemm(g, st));
        }
        HIPCHK(ctx, launch_gru_combine(batch * An, s, precomp ? ws.gi_all : ws.gi,
                                       precomp ? ws.gidx_cand : nullptr,
                                       precomp == 2 ? ws.rowmap : nullptr,
                                       markov ? nullptr : ws.uh + r, ldu,
                                       markov ? w.b_hh : nullptr, markov ? nullptr : ws.S[sc],
                                       ws.gidx_par, ws.S[1 - sc], ws.S3[1 - sc], st));
        sc = 1 - sc;
      }
      cur = 1 - cur;
      tb.surv_node = ws.surv[cur]; tb.surv_rank = ws.rank[cur];
      tb.nsurv_node = ws.surv[1 - cur]; tb.nsurv_rank = ws.rank[1 - cur];
      tb.surv_score = ws.sscore[cur]; tb.nsurv_score = ws.sscore[1 - cur];
      off += A * K;
      A = An;
    }
  }
  const int NT = off;
  prof_mark(ctx, 5, st);
  HIPCHK(ctx, launch_topb_emit(batch, NT, B, p->beta, c.max_B, tb, tok, parent, depth, score,
                               mask, n_nodes, st));
  prof_mark(ctx, 6, st);
  if (ctx->prof && ctx->prof_n < kProfRounds) ++ctx->prof_n;
  ctx->has_round = true;
  ctx->last = *p;
  ctx->last_batch = batch;
  ctx->last_NT = NT;
  return DTREE_OK;
}

static dtree_status heap_trace(dtree_ctx *ctx, int32_t req, dtree_trace *o);

extern "C" dtree_status dtree_get_trace(dtree_ctx *ctx, int32_t req, dtree_trace *o) {
  if (!ctx) return DTREE_E_ARG;
  ctx->err.clear();
  if (!o) return fail(ctx, DTREE_E_ARG, "null trace");
  if (!ctx->has_round) return fail(ctx, DTREE_E_STATE, "no round has been built");
  if (req < 0 || req >= ctx->last_batch) return fail(ctx, DTREE_E_ARG, "req out of range");
  DeviceGuard dg(ctx->device);
  HIPCHK(ctx, hipDeviceSynchronize());
  if (ctx->last_heap) return heap_trace(ctx, req, o);
  const dtree_params &p = ctx->last;
  const Ws &ws = ctx->ws;
  const size_t cm = (size_t)p.D * p.M;
  const size_t nb = (size_t)req * ctx->NTcap;
  const int NT = ctx->last_NT, Wm = ctx->caps.max_W;
  if (o->C) HIPCHK(ctx, hipMemcpy(o->C, ws.C + req * cm, cm * 4, hipMemcpyDeviceToHost));
  if (o->Cl) HIPCHK(ctx, hipMemcpy(o->Cl, ws.Cl + req * cm, cm * 4, hipMemcpyDeviceToHost));
  if (o->node_tok) HIPCHK(ctx, hipMemcpy(o->node_tok, ws.n_tok + nb, NT * 4, hipMemcpyDeviceToHost));
  if (o->node_parent) HIPCHK(ctx, hipMemcpy(o->node_parent, ws.n_par + nb, NT * 4, hipMemcpyDeviceToHost));
  if (o->node_score) HIPCHK(ctx, hipMemcpy(o->node_score, ws.n_score + nb, NT * 4, hipMemcpyDeviceToHost));
  if (o->surv)
    HIPCHK(ctx, hipMemcpy2D(o->surv, (size_t)p.W * 4, ws.surv_hist + (size_t)req * (p.D + 1) * Wm,
                            (size_t)Wm * 4, (size_t)p.W * 4, p.D + 1, hipMemcpyDeviceToHost));
  if (o->sel)
    HIPCHK(ctx, hipMemcpy(o->sel, ws.sel + (size_t)req * ctx->caps.max_B, (size_t)p.B * 4,
                          hipMemcpyDeviceToHost));
  uint32_t st = 0;
  HIPCHK(ctx, hipMemcpy(&st, ws.status, 4, hipMemcpyDeviceToHost));
  o->n_sa = NT;
  o->status = (int32_t)st;
  return DTREE_OK;
}

// The heap builder's trace: candidates, every pushed node (push order), the
// pops in pop order (-1 past the last); no per-depth survivors (-1).
static dtree_status heap_trace(dtree_ctx *ctx, int32_t req, dtree_trace *o) {
  const dtree_params &p = ctx->last;
  const Ws &ws = ctx->ws;
  const HeapBufs &hp = ws.hp;
  const size_t cm = (size_t)p.D * p.M;
  const size_t nb = (size_t)req * hp.NH;
  int32_t nn = 0;
  HIPCHK(ctx, hipMemcpy(&nn, hp.nnodes + req, 4, hipMemcpyDeviceToHost));
  if (o->C) HIPCHK(ctx, hipMemcpy(o->C, ws.C + req * cm, cm * 4, hipMemcpyDeviceToHost));
  if (o->Cl) HIPCHK(ctx, hipMemcpy(o->Cl, ws.Cl + req * cm, cm * 4, hipMemcpyDeviceToHost));
  if (o->node_tok) HIPCHK(ctx, hipMemcpy(o->node_tok, hp.tok + nb, (size_t)nn * 4, hipMemcpyDeviceToHost));
  if (o->node_parent) HIPCHK(ctx, hipMemcpy(o->node_parent, hp.par + nb, (size_t)nn * 4, hipMemcpyDeviceToHost));
  if (o->node_score) HIPCHK(ctx, hipMemcpy(o->node_score, hp.score + nb, (size_t)nn * 4, hipMemcpyDeviceToHost));
  if (o->surv) std::fill(o->surv, o->surv + (size_t)(p.D + 1) * p.W, -1);
  if (o->sel)
    HIPCHK(ctx, hipMemcpy(o->sel, hp.pops + (size_t)req * hp.Bcap, (size_t)p.B * 4,
                          hipMemcpyDeviceToHost));
  o->n_sa = nn;
  o->status = 0;
  return DTREE_OK;
}

extern "C" dtree_status dtree_profile_enable(dtree_ctx *ctx, int enable) {
  if (!ctx) return DTREE_E_ARG;
  ctx->err.clear();
  DeviceGuard dg(ctx->device);
  if (enable && !ctx->prof_ev) {
    const int n = kProfRounds * (DTREE_NSTAGES + 1);
    ctx->prof_ev = new (std::nothrow) hipEvent_t[n];
    if (!ctx->prof_ev) return fail(ctx, DTREE_E_NOMEM, "event table");
    for (int i = 0; i < n; ++i) {
      if (hipEventCreate(&ctx->prof_ev[i]) != hipSuccess) {
        for (int j = 0; j < i; ++j) (void)hipEventDestroy(ctx->prof_ev[j]);
        delete[] ctx->prof_ev;
        ctx->prof_ev = nullptr;
        return fail(ctx, DTREE_E_HIP, "hipEventCreate failed");
      }
    }
  }
  ctx->prof = enable != 0;
  ctx->prof_n = 0;
  return DTREE_OK;
}

extern "C" dtree_status dtree_profile_read(dtree_ctx *ctx, float *ms, int32_t *rounds) {
  if (!ctx) return DTREE_E_ARG;
  ctx->err.clear();
  if (!ms || !rounds) return fail(ctx, DTREE_E_ARG, "null output");
  for (int k = 0; k < DTREE_NSTAGES; ++k) ms[k] = 0.f;
  *rounds = 0;
  if (!ctx->prof_ev) return DTREE_OK;
  DeviceGuard dg(ctx->device);
  for (int rr = 0; rr < ctx->prof_n; ++rr) {
    hipEvent_t *e = ctx->prof_ev + rr * (DTREE_NSTAGES + 1);
    HIPCHK(ctx, hipEventSynchronize(e[DTREE_NSTAGES]));
    for (int k = 0; k < DTREE_NSTAGES; ++k) {
      float t = 0.f;
      HIPCHK(ctx, hipEventElapsedTime(&t, e[k], e[k + 1]));
      ms[k] += t;
    }
  }
  *rounds = ctx->prof_n;
  ctx->prof_n = 0;
  return DTREE_OK;
}

extern "C" dtree_status dtree_set_persistent_launch(dtree_ctx *ctx, int32_t cooperative,
                                                    int32_t spin_limit) {
  if (!ctx) return DTREE_E_ARG;
  ctx->err.clear();
  if (cooperative != 0 && cooperative != 1) return fail(ctx, DTREE_E_ARG, "cooperative must be 0 or 1");
  if (spin_limit < 0) return fail(ctx, DTREE_E_ARG, "spin_limit must be >= 0");
  ctx->pk_coop = cooperative == 1;
  ctx->pk_spin = (uint32_t)spin_limit;
  return DTREE_OK;
}

extern "C" dtree_status dtree_set_builder(dtree_ctx *ctx, int32_t builder) {
  if (!ctx) return DTREE_E_ARG;
  ctx->err.clear();
  if (builder != DTREE_BUILD_DEPTHWISE && builder != DTREE_BUILD_HEAP)
    return fail(ctx, DTREE_E_ARG, "builder must be DTREE_BUILD_DEPTHWISE or DTREE_BUILD_HEAP");
  if (builder == DTREE_BUILD_HEAP && !ctx->ws.hp.tok) {
    const dtree_caps &c = ctx->caps;
    const int s = ctx->w.s, r = ctx->w.r;
    const long long NH = (long long)c.max_K * (c.max_B + 1) + 1;
    if (NH > (1 << 24)) return fail(ctx, DTREE_E_SHAPE, "max_K * (max_B + 1) too large for the heap");
    if (heap_emit_smem((int)NH, c.max_B) > ctx->lds_max ||
        heap_step_smem((int)NH, c.max_D, c.max_M, ctx->w.r) > ctx->lds_max)
      return fail(ctx, DTREE_E_SHAPE, "max_K * max_B too large for the heap builder's LDS");
    DeviceGuard dg(ctx->device);
    HeapBufs &hp = ctx->ws.hp;
    hp.NH = (int)NH;
    hp.Bcap = c.max_B;
    const size_t nodes = (size_t)c.max_batch * NH, slots = (size_t)c.max_batch * (c.max_B + 1);
    hipError_t e = hipSuccess;
    auto A = [&](hipError_t x) { if (e == hipSuccess) e = x; };
    A(alloc(&hp.tok, nodes));
    A(alloc(&hp.par, nodes));
    A(alloc(&hp.dep, nodes));
    A(alloc(&hp.score, nodes));
    A(alloc(&hp.gref, nodes * 2));
    A(alloc(&hp.pv, nodes));
    A(alloc(&hp.nnodes, (size_t)c.max_batch));
    A(alloc(&hp.pops, (size_t)c.max_batch * c.max_B));
    A(alloc(&hp.ex, (size_t)c.max_batch * 4));
    A(alloc(&hp.S, slots * s));
    A(alloc(&hp.UH, slots * (size_t)(r + 3 * s)));
    A(alloc(&hp.gi, (size_t)c.max_batch * c.max_D * c.max_M * 3 * s));
    if (e == hipSuccess) e = heap_prepare(ctx->lds_max);
    if (e != hipSuccess) {
      void *ptrs[] = {hp.tok, hp.par, hp.dep, hp.score, hp.gref, hp.pv, hp.nnodes, hp.pops,
                      hp.ex, hp.S, hp.UH, hp.gi};
      for (void *q : ptrs)
        if (q) (void)hipFree(q);
      hp = HeapBufs();
      return fail(ctx, e == hipErrorOutOfMemory ? DTREE_E_NOMEM : DTREE_E_HIP,
                  std::string("heap builder tables: ") + hipGetErrorString(e));
    }
  }
  ctx->builder = builder;
  return DTREE_OK;
}

extern "C" dtree_status dtree_set_scoring(dtree_ctx *ctx, int32_t scoring) {
  if (!ctx) return DTREE_E_ARG;
  ctx->err.clear();
  if (scoring != DTREE_SCORE_CONDITIONAL && scoring != DTREE_SCORE_MARGINAL &&
      scoring != DTREE_SCORE_MARKOV)
    return fail(ctx, DTREE_E_ARG,
                "scoring must be DTREE_SCORE_CONDITIONAL, DTREE_SCORE_MARGINAL or DTREE_SCORE_MARKOV");
  ctx->scoring = scoring;
  return DTREE_OK;
}

extern "C" const char *dtree_last_error(const dtree_ctx *ctx) {
  if (ctx) return ctx->err.c_str();
  return g_create_err.empty() ? g_static_err_text() : g_create_err.c_str();
}

extern "C" dtree_status dtree_destroy(dtree_ctx *ctx) {
  if (!ctx) return DTREE_OK;
  {
    DeviceGuard dg(ctx->device);
    free_ws(ctx->ws);
    if (ctx->pk_fail) (void)hipHostFree(ctx->pk_fail);
    if (ctx->prof_ev) {
      for (int i = 0; i < kProfRounds * (DTREE_NSTAGES + 1); ++i) (void)hipEventDestroy(ctx->prof_ev[i]);
      delete[] ctx->prof_ev;
    }
  }
  delete ctx;
  return DTREE_OK;
}

// ---------------------------------------------------------------- allocation-free rounds
//
// dtree_build_round_static: one round with no context.  Its whole workspace
// lives in `scratch`, a file-scope device array of kStaticScratch bytes (each
// device the library runs on holds its own copy until the process ends).  In
// host code `scratch` names a host-side stand-in, so the array's device
// address is taken once per device with hipGetSymbolAddress and only that
// address is used.  Calls on one device share the array: calls whose work
// overlaps on the device race (one stream, or synchronised streams, per
// device); every buffer a round reads is written earlier in the same round
// (the round-start kernel clears the survivor history and the status word).
static constexpr size_t kStaticScratch = (size_t)16 << 20;
static __device__ __align__(256) uint8_t scratch[kStaticScratch];

namespace {
constexpr int kMaxDevices = 64;
struct StaticDevice {
  bool ready = false;
  bool gfx950 = false;
  size_t lds_max = 0;
  void *scratch = nullptr;   // device address of this device's `scratch`
};
StaticDevice g_static_dev[kMaxDevices];
std::mutex g_static_mu;
thread_local char g_static_err[256];

dtree_status static_fail(dtree_status s, const char *m) {
  std::snprintf(g_static_err, sizeof g_static_err, "%s", m);
  g_create_err.clear();
  return s;
}
}  // namespace

// The workspace of a round sized exactly for p and batch, carved from base
// (256-byte aligned pieces); returns the bytes it needs (nothing is written
// when base is null).
static size_t static_layout(const dtree_weights &w, const dtree_params &p, int batch, int P,
                            int NT, uint8_t *base, Ws &ws) {
  size_t off = 0;
  auto take = [&](auto **ptr, size_t n) {
    using T = std::remove_pointer_t<std::remove_reference_t<decltype(*ptr)>>;
    const size_t at = (off + 255) & ~(size_t)255;
    off = at + (n ? n : 1) * sizeof(T);
    if (base) *ptr = reinterpret_cast<T *>(base + at);
  };
  const size_t rows = (size_t)batch * p.D, bw = (size_t)batch * p.W;
  const int s = w.s, r = w.r;
  take(&ws.part, rows * P * K1_LSTRIDE);
  take(&ws.C, rows * p.M);
  take(&ws.Cl, rows * p.M);
  take(&ws.uH, rows * r);
  take(&ws.hb, (rows + 15) / 16 * 16 * (size_t)w.d);
  take(&ws.S[0], bw * s);
  take(&ws.S[1], bw * s);
  take(&ws.uh, bw * (r + 3 * s));
  take(&ws.ell, bw * p.M);
  take(&ws.ckey, bw * p.K);
  take(&ws.ccand, bw * p.K);
  take(&ws.selflag, (size_t)batch * 64);
  for (int i = 0; i < 2; ++i) take(&ws.sscore[i], bw);
  take(&ws.gi, bw * 3 * s);
  const size_t nt = (size_t)batch * NT;
  take(&ws.n_tok, nt);
  take(&ws.n_par, nt);
  take(&ws.n_dep, nt);
  take(&ws.n_score, nt);
  take(&ws.n_lex, nt);
  for (int i = 0; i < 2; ++i) { take(&ws.surv[i], bw); take(&ws.rank[i], bw); }
  take(&ws.surv_hist, (size_t)batch * (p.D + 1) * p.W);
  take(&ws.gidx_tok, bw);
  take(&ws.gidx_par, bw);
  take(&ws.sel, (size_t)batch * p.B);
  take(&ws.status, 1);
  return off;
}

extern "C" dtree_status dtree_build_round_static(const dtree_weights *w, const dtree_params *p,
                                                 int32_t batch, const float *H,
                                                 const int32_t *root, int32_t *tok,
                                                 int32_t *parent, int32_t *depth, float *score,
                                                 uint8_t *mask, int32_t *n_nodes, void *stream) {
  g_static_err[0] = '\0';
  if (!w || !p) return static_fail(DTREE_E_ARG, "null weights or params");
  if (!H || !root || !tok || !parent || !depth || !score || !mask || !n_nodes)
    return static_fail(DTREE_E_ARG, "null input or output pointer");
  if (w->wtype != DTREE_F32 && w->wtype != DTREE_BF16)
    return static_fail(DTREE_E_DTYPE, "wtype must be DTREE_F32 or DTREE_BF16");
  if (w->d < 1 || w->V < 1 || w->e < 1 || w->s < 1 || w->r < 1)
    return static_fail(DTREE_E_ARG, "d, V, e, s, r must be >= 1");
  if (w->V > (1 << 18)) return static_fail(DTREE_E_SHAPE, "V must be <= 262144");
  if (!w->W_lm || !w->Emb || !w->W_ih || !w->W_hh || !w->W1 || !w->W2)
    return static_fail(DTREE_E_ARG, "null weight pointer");
  if (w->wtype == DTREE_BF16) {
    if (w->d % 128) return static_fail(DTREE_E_SHAPE, "bf16 weights need d % 128 == 0");
    if (reinterpret_cast<uintptr_t>(w->W_lm) % 16)
      return static_fail(DTREE_E_ARG, "W_lm must be 16-byte aligned");
  }
  const int D = p->D, M = p->M, K = p->K, W = p->W, B = p->B;
  if (batch < 1) return static_fail(DTREE_E_ARG, "batch must be >= 1");
  if (D < 1 || D > 31) return static_fail(DTREE_E_ARG, "D outside [1, 31]");
  if (M < 1 || M > 128 || M > w->V) return static_fail(DTREE_E_ARG, "M outside [1, min(128, V)]");
  if (K < 1 || K > M) return static_fail(DTREE_E_ARG, "K outside [1, M]");
  if (W < 1 || W > 512 || (long long)W * K > 1024)
    return static_fail(DTREE_E_ARG, "W outside [1, 512] or W * K > 1024");
  if (B < 1) return static_fail(DTREE_E_ARG, "B must be >= 1");
  if (!(p->beta <= 0.0f)) return static_fail(DTREE_E_ARG, "beta must be <= 0 (and not NaN)");
  if (std::isinf(p->beta)) return static_fail(DTREE_E_ARG, "beta must be finite");
  const int NT = superarbol_nodes(D, K, W);
  if (NT < 0 || NT > 8192) return static_fail(DTREE_E_SHAPE, "superarbol exceeds 8192 nodes");
  const int P = lmhead_partitions(w->V, w->wtype, (w->r + 15) / 16);
  Ws ws;
  const size_t need = static_layout(*w, *p, batch, P, NT, nullptr, ws);
  if (need > kStaticScratch) {
    char m[160];
    std::snprintf(m, sizeof m, "round workspace of %zu bytes exceeds the %zu-byte static scratch",
                  need, kStaticScratch);
    return static_fail(DTREE_E_SHAPE, m);
  }

  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return static_fail(DTREE_E_DEVICE, "no current HIP device");
  StaticDevice &sd = g_static_dev[dev];
  {
    std::lock_guard<std::mutex> lk(g_static_mu);
    if (!sd.ready) {
      hipDeviceProp_t prop;
      if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
        return static_fail(DTREE_E_DEVICE, "device query failed");
      sd.gfx950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
      sd.lds_max = prop.sharedMemPerBlock;
      if (sd.gfx950) {
        void *ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) {
          char m[128];
          std::snprintf(m, sizeof m, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
          return static_fail(DTREE_E_HIP, m);
        }
        sd.scratch = ptr;
        hipError_t pe = hipSuccess;
        for (int ring = 0; ring <= 2 && pe == hipSuccess; ++ring)
          pe = lmhead_prepare(WT_BF16, ring, sd.lds_max);
        if (pe == hipSuccess) pe = corr_logits_prepare(WT_BF16, sd.lds_max);
        if (pe == hipSuccess) pe = corr_logits_prepare(WT_F32, sd.lds_max);
        if (pe == hipSuccess) pe = topb_prepare(sd.lds_max);
        if (pe == hipSuccess) pe = gemm_prepare();
        if (pe == hipSuccess) pe = branch_select_prepare(sd.lds_max);
        if (pe != hipSuccess) {
          char m[128];
          std::snprintf(m, sizeof m, "kernel attributes: %s", hipGetErrorString(pe));
          return static_fail(DTREE_E_HIP, m);
        }
      }
      sd.ready = true;
    }
  }
  if (!sd.gfx950) return static_fail(DTREE_E_DEVICE, "needs a gfx950 device");

  // the kernels' own limits, as dtree_create checks them
  const int ring = lmhead_ring(w->d, w->wtype, sd.lds_max);
  const size_t k1_smem = lmhead_smem(w->d, w->wtype, ring);
  if (k1_smem > sd.lds_max) return static_fail(DTREE_E_SHAPE, "d too large for the LM-head LDS tile");
  if (topm_merge_smem(P) > 131072)
    return static_fail(DTREE_E_SHAPE, "vocabulary too large for the Top-M merge");
  if (corr_logits_smem(W, M, w->r, w->wtype) > sd.lds_max)
    return static_fail(DTREE_E_SHAPE, "M * r too large for the correction LDS tile");
  if (topb_smem(NT, B) > sd.lds_max)
    return static_fail(DTREE_E_SHAPE, "superarbol too large for the Top-B LDS sort");

  // a context on the stack: workspace in scratch, no persistent depth loop,
  // no derived weight copies, no stage events
  dtree_ctx ctx;
  ctx.device = dev;
  ctx.w = *w;
  ctx.caps = dtree_caps{batch, D, M, K, W, B};
  ctx.P = P;
  ctx.NTcap = NT;
  ctx.k1_ring = ring;
  ctx.k1_smem = k1_smem;
  ctx.lds_max = sd.lds_max;
  static_layout(*w, *p, batch, P, NT, static_cast<uint8_t *>(sd.scratch), ctx.ws);
  ctx.sel_batch = w->wtype == DTREE_BF16 && w->r % 8 == 0 && w->r <= 512 &&
                  reinterpret_cast<uintptr_t>(w->W2) % 16 == 0 &&
                  branch_select_smem(w->r) + 32768 <= sd.lds_max;
  ctx.err_buf = g_static_err;
  ctx.err_cap = sizeof g_static_err;
  return enqueue_round(&ctx, p, batch, H, root, tok, parent, depth, score, mask, n_nodes,
                       static_cast<hipStream_t>(stream));
}

static const char *g_static_err_text() { return g_static_err; }

// ---------------------------------------------------------------------------
// tree-attention verification

static dtree_status attn_check(const dtree_attn_args *a, int *splits) {
  if (!a) return static_fail(DTREE_E_ARG, "null arguments");
  if (a->batch < 1 || a->n_max < 1) return static_fail(DTREE_E_ARG, "batch and n_max must be >= 1");
  if (a->n_max > 4096) return static_fail(DTREE_E_SHAPE, "n_max must be <= 4096");
  if (a->dh != 64 && a->dh != 128) return static_fail(DTREE_E_SHAPE, "dh must be 64 or 128");
  if (a->Hkv < 1 || a->Hq < 1 || a->Hq % a->Hkv)
    return static_fail(DTREE_E_SHAPE, "Hq must be a positive multiple of Hkv");
  if (a->Hq / a->Hkv > 64) return static_fail(DTREE_E_SHAPE, "Hq / Hkv must be <= 64");
  if (a->L_cap < a->n_max) return static_fail(DTREE_E_SHAPE, "L_cap must be >= n_max");
  if ((long long)a->L_cap * a->dh >= (1LL << 30))
    return static_fail(DTREE_E_SHAPE, "L_cap * dh must be < 2^30 (32-bit byte offsets)");
  if ((long long)a->batch * a->Hkv * a->L_cap * a->dh >= (1LL << 40) ||
      (long long)a->batch * a->n_max * a->Hq * a->dh >= (1LL << 31))
    return static_fail(DTREE_E_SHAPE, "tensors too large");
  if (!(std::isfinite(a->scale) && a->scale > 0.f))
    return static_fail(DTREE_E_ARG, "scale must be finite and > 0");
  if (a->splits < 0 || a->splits > 256) return static_fail(DTREE_E_ARG, "splits outside [0, 256]");
  const long long rb = ((long long)a->n_max * (a->Hq / a->Hkv) + 63) / 64;
  const int S = dtree::tree_attn_splits(a->batch, a->n_max, a->Hq, a->Hkv, a->L_cap, a->splits);
  if (rb * a->Hkv * a->batch * S >= (1LL << 31))
    return static_fail(DTREE_E_SHAPE, "grid too large");
  *splits = S;
  return DTREE_OK;
}

extern "C" dtree_status dtree_tree_attention_workspace(const dtree_attn_args *a, size_t *bytes) {
  g_static_err[0] = '\0';
  if (!bytes) return static_fail(DTREE_E_ARG, "null output pointer");
  int S = 1;
  const dtree_status st = attn_check(a, &S);
  if (st != DTREE_OK) return st;
  *bytes = dtree::tree_attn_workspace(a->batch, a->n_max, a->Hq, a->Hkv, a->dh, S);
  return DTREE_OK;
}

namespace {
int g_attn_arch[kMaxDevices];   // 0 unknown, 1 gfx950, -1 other
}

extern "C" dtree_status dtree_tree_attention(const dtree_attn_args *a, void *stream) {
  g_static_err[0] = '\0';
  int S = 1;
  const dtree_status st = attn_check(a, &S);
  if (st != DTREE_OK) return st;
  if (!a->Q || !a->K || !a->V || !a->prefix_len || !a->n_nodes || !a->mask || !a->O)
    return static_fail(DTREE_E_ARG, "null input or output pointer");
  if (reinterpret_cast<uintptr_t>(a->Q) % 16 || reinterpret_cast<uintptr_t>(a->K) % 16 ||
      reinterpret_cast<uintptr_t>(a->V) % 16 || reinterpret_cast<uintptr_t>(a->O) % 16)
    return static_fail(DTREE_E_ARG, "Q, K, V and O must be 16-byte aligned");
  const size_t need = dtree::tree_attn_workspace(a->batch, a->n_max, a->Hq, a->Hkv, a->dh, S);
  if (need && (!a->workspace || a->workspace_bytes < need ||
               reinterpret_cast<uintptr_t>(a->workspace) % 256)) {
    char m[160];
    std::snprintf(m, sizeof m, "needs a 256-byte aligned workspace of %zu bytes", need);
    return static_fail(DTREE_E_ARG, m);
  }
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return static_fail(DTREE_E_DEVICE, "no current HIP device");
  int arch = 0;
  {
    std::lock_guard<std::mutex> lk(g_static_mu);
    if (!g_attn_arch[dev]) {
      hipDeviceProp_t prop;
      if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
        return static_fail(DTREE_E_DEVICE, "device query failed");
      g_attn_arch[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    }
    arch = g_attn_arch[dev];
  }
  if (arch < 0) return static_fail(DTREE_E_DEVICE, "needs a gfx950 device");
  dtree::TreeAttnArgs t{a->batch, a->n_max, a->Hq, a->Hkv, a->dh, a->L_cap, S,
                        a->Q, a->K, a->V, a->prefix_len, a->n_nodes, a->mask,
                        a->scale, a->O, a->workspace};
  const hipError_t e = dtree::launch_tree_attn(t, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    char m[160];
    std::snprintf(m, sizeof m, "tree attention launch: %s", hipGetErrorString(e));
    return static_fail(DTREE_E_HIP, m);
  }
  return DTREE_OK;
}
