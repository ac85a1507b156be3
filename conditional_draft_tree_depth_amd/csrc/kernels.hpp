// Host-side launchers of the draft-tree kernels (one translation unit each).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dtree {

enum { WT_F32 = 0, WT_BF16 = 1 };

// Lets kernel fn use up to lds_bytes of LDS per workgroup in all: its limit
// for dynamic LDS is lds_bytes less the kernel's own static LDS.
inline hipError_t set_lds_limit(const void *fn, size_t lds_bytes) {
  hipFuncAttributes fa;
  hipError_t e = hipFuncGetAttributes(&fa, fn);
  if (e != hipSuccess) return e;
  const size_t st = fa.sharedSizeBytes;
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)(lds_bytes > st ? lds_bytes - st : 0));
}

struct TreeBufs {
  int NT;              // superarbol nodes per request (root included)
  int V;               // vocabulary size (root tokens are clamped into [0, V))
  int Wmax;            // survivor slots per request
  int32_t *n_tok, *n_par, *n_dep;   // [b, NT]
  float *n_score;                   // [b, NT]
  uint32_t *n_lex;                  // [b, NT] (parent lexrank << 18) | token
  int32_t *surv_node, *surv_rank;   // [b, Wmax] current expanded nodes
  int32_t *nsurv_node, *nsurv_rank; // [b, Wmax] next depth
  float *surv_score, *nsurv_score;  // [b, Wmax] their scores (batched selection only, or null)
  int32_t *surv_hist;               // [b, D+1, Wmax]
  int32_t *gidx_tok, *gidx_par;     // [b * Wmax] gathers for the GRU step
  int32_t *gidx_cand;               // [b * Wmax] survivor's candidate row (q D + depth) M + j,
                                    // written when not null
  int32_t *sel;                     // [b, Bmax]
  uint32_t *status;                 // device status bits
  uint32_t *selflag;                // [b, 64] arrival flags of the batched selection (or null)
};

// Start of a round for request q (called by one workgroup per request before
// anything reads the tree buffers): empty survivor history, the root node
// (its token clamped into [0, V)) as the only expanded branch.
__device__ inline void init_round_request(int q, const int32_t *root, const TreeBufs &t, int Dp1,
                                          int tid, int nt) {
  for (int i = tid; i < Dp1 * t.Wmax; i += nt)
    t.surv_hist[(size_t)q * Dp1 * t.Wmax + i] = i == 0 ? 0 : -1;
  if (t.selflag)
    for (int i = tid; i < 64; i += nt) t.selflag[(size_t)q * 64 + i] = 0u;
  if (tid == 0) {
    const size_t n0 = (size_t)q * t.NT;
    const int32_t rt = root[q] < 0 ? 0 : (root[q] >= t.V ? t.V - 1 : root[q]);
    t.n_tok[n0] = rt;
    t.n_par[n0] = -1;
    t.n_dep[n0] = 0;
    t.n_score[n0] = 0.f;
    t.n_lex[n0] = 0u;
    t.surv_node[(size_t)q * t.Wmax] = 0;
    t.surv_rank[(size_t)q * t.Wmax] = 0;
    if (t.surv_score) t.surv_score[(size_t)q * t.Wmax] = 0.f;
    t.gidx_tok[q] = rt;
    if (q == 0) *t.status = 0u;
  }
}

// ---- K1: base logits Hq . W_lm^T + bias with a fused per-workgroup Top-M
// pre-selection.  For every row and vocabulary slice p (P slices per row)
// it writes the list part[row][p][0 .. K1_LSTRIDE): up to K1_LCAP keys (any
// order) that include the slice's M best, then tau, head and count: every
// slice key >= tau is among the `count` keys, at least min(M, slice size)
// slice keys are >= tau, head is the slice's best key.
constexpr int K1_LCAP = 128;
constexpr int K1_LSTRIDE = K1_LCAP + 4;
struct LMHeadArgs {
  const float *H;      // [rows, d] fp32
  int rows, d;
  const void *W;       // [V, d]
  int wtype, V;
  const float *bias;   // [V] or null
  int M, P;
  uint64_t *part;      // [rows, P, K1_LSTRIDE]
  const void *W1;      // bf16 only: W1[:, :d] rows ride along -> uH (or null)
  int ldw1, r;
  float *uH;           // [rows, r]
  // round start (init_round_request for q < b): done by the first workgroups
  // of the streaming kernels, by k1_stage_hidden ahead of the tiled product
  const int32_t *root;
  int b, Dp1;
  TreeBufs t;
  int ring;            // bf16: LDS ring depth from lmhead_ring (0 = register path)
  uint16_t *Hb;        // bf16, tiled product: [rows rounded up to 16, d] rounded hidden rows
  // tiled product (or null): [rows, lmhead_groups(V)] ordered maxima of column
  // groups of the logits, and [rows] the row-wide list bound found from them
  uint32_t *gmax = nullptr, *rbound = nullptr;
  int32_t *ovf = nullptr;   // [ceil(rows / 8), P] flags: lists that overflowed the bound
};
// column groups of the tiled product's per-group logit maxima (the most any
// of its tile shapes makes)
inline int lmhead_groups(int V) { return (V + 63) / 64; }
int lmhead_partitions(int V, int wtype, int extra_tiles);
// LDS ring depth of the bf16 kernel that fits lds_max (0: register path)
int lmhead_ring(int d, int wtype, size_t lds_max);
size_t lmhead_smem(int d, int wtype, int ring);
// every prepare call lets its kernels use up to lds_bytes of LDS in all
hipError_t lmhead_prepare(int wtype, int ring, size_t lds_bytes);
// bf16, tiled product: round start (k1_stage_hidden: Hb, init_round_request)
// before launch_lmhead_tiled; the streaming kernels (launch_lmhead) round the
// hidden rows and start the round themselves
hipError_t launch_stage_hidden(const LMHeadArgs &a, hipStream_t st);
// ev0 / ev1 (or null): events that take the kernel's own start and end times
hipError_t launch_lmhead(const LMHeadArgs &a, hipStream_t st, hipEvent_t ev0 = nullptr,
                         hipEvent_t ev1 = nullptr);
// ---- K1b: the M best keys of each row from its P lists -> C (tokens), Cl (logits)
size_t topm_merge_smem(int P);
// 32 or more hidden rows (bf16): logits [rows, V] fp32 by a tiled MFMA
// product, then the same per-slice candidate lists (uH is not produced)
bool lmhead_tiled_ok(int rows, int d, int wtype);
hipError_t launch_lmhead_tiled(const LMHeadArgs &a, float *logits, hipStream_t st,
                               hipEvent_t ev0, hipEvent_t ev1);
// the merge fused with the correction tables of the persistent depth loop
// (G [rows][s][M], g [rows][M]; W1t as launch_corr_tables takes it)
bool topm_tables_ok(int M, int r, int s, const void *W2, const void *W1t);
hipError_t launch_topm_tables(const uint64_t *part, int P, int M, int rows, int r, int s,
                              const void *W2, const void *W1t, const float *uH, int32_t *C,
                              float *Cl, float *G, float *g, hipStream_t st);
hipError_t launch_topm_merge(const uint64_t *part, int P, int M, int rows,
                             int32_t *C, float *Cl, hipStream_t st);

// ---- generic fp32-activation x weight^T product with gathers and epilogue
// Y[i][n] = sum_k X[xrow(i)][k] * W[n][k] + bias[n - bias_n0] (n >= bias_n0)
//           + addend[arow(i)][n] (n < add_n)
// xrow(i) = xidx ? xidx[i] : i ; arow(i) = (i / adiv) * amul + aoff
struct GemmArgs {
  int R, N, Kd;
  const void *X; int xtype; int ldx; const int32_t *xidx; int xround;
  const void *W; int wtype; int ldw;
  const float *bias;
  const float *addend; int lda, adiv, amul, aoff;
  float *Y; int ldy;
  int add_n = 1 << 30;   // the addend covers outputs n < add_n
  int bias_n0 = 0;       // the bias covers outputs n >= bias_n0
  const int32_t *Rdev = nullptr;   // tiled product only: the row count read on the
                                   // device (R is then its upper bound)
  int kw = 0;            // bf16 X only: W's k index is k mod kw (0: kw = Kd); a
                         // state split into bf16 planes [hi | lo]
                         // is multiplied by the same weights once per plane
  // LM-head product only (or null): gmax[row * ldg + n / GW] = largest
  // ordered output (f32_ord) of row over the columns n of its group of GW
  // (the tile's columns per wave: 64 or 80)
  uint32_t *gmax = nullptr;
  int ldg = 0;
};
hipError_t launch_gemm(const GemmArgs &a, hipStream_t st);
// GRU gates: gi, gh = input/state projections incl. biases ([R, 3s]); if gh
// is null the previous state is zero and the state part equals b_hh.
// Row i takes gi row gidx[i] (i if gidx is null; mapped through gmap when
// given), gh row pidx[i] (stride ldgh) and previous state row pidx[i].
// S3 (or null): the new state also as STATE_PLANES bf16 planes, row i =
// [hi | lo] ([R, STATE_PLANES s]): hi = bf16(x), lo = bf16(x - hi), so
// |x - hi - lo| <= 2^-18 |x| for every fp32 value x.
constexpr int STATE_PLANES = 2;
hipError_t launch_gru_combine(int R, int s, const float *gi, const int32_t *gidx,
                              const int32_t *gmap, const float *gh, int ldgh,
                              const float *b_hh, const float *Sprev,
                              const int32_t *pidx, float *Snew, uint16_t *S3, hipStream_t st);
hipError_t gemm_prepare();
// Distinct tokens of tok[0..n) (n <= 262144): uniq[0..*count) in order of
// first occurrence, rowmap[i] = position of tok[i] in uniq.  first [V] u64;
// epoch must grow by one from round to round, starting at 1 (and again at 1
// after it wraps: epoch 1 clears first); lpos, cidx [n] and btot
// [n / 256 + 1] are scratch.
hipError_t launch_token_dedupe(int n, const int32_t *tok, void *first, int V, uint32_t epoch,
                               int32_t *lpos, int32_t *btot, int32_t *cidx, int32_t *uniq,
                               int32_t *rowmap, int32_t *count, hipStream_t st);
// true when launch_gemm runs a as a tiled product (many rows, bf16 operands)
bool gemm_tiled_ok(const GemmArgs &a);
// tiled product (bf16 operands, k and kw multiples of 64): tile bm x bn in
// {256 x 128, 128 x 128} (chosen for R x N by mm_tile) or 128 x 320 (the
// LM head with one row tile); ev0/ev1 (or null) are recorded at the
// kernel's start and end
bool mm_ok(const GemmArgs &a);
void mm_tile(int R, int N, int *bm, int *bn);
hipError_t launch_mm(const GemmArgs &a, int bm, int bn, hipStream_t st, hipEvent_t ev0,
                     hipEvent_t ev1);
// the LM-head product (no row gather, no planes, bias from n = 0): tiles of
// bm x bn in {128 x 256, 128 x 320, 256 x 256} with a ring per operand
hipError_t launch_mm_lm(const GemmArgs &a, int bm, int bn, hipStream_t st, hipEvent_t ev0,
                        hipEvent_t ev1);
// true when launch_gemm accepts a device row count (a.Rdev) for a
bool gemm_rdev_ok(const GemmArgs &a);
// Wcat = [W1[:, d:] ; W_hh] as [r + 3s, s] rows in the weight dtype
hipError_t launch_concat_state_weights(const void *W1, const void *W_hh, int r, int s, int d,
                                       int wtype, void *Wcat, hipStream_t st);

// ---- per-depth kernels
hipError_t launch_corr_logits(int b, int A, int M, int r, int D, int delta,
                              const void *W2, int wtype, const int32_t *C,
                              const float *Cl, const float *u, int ldu, float *ell,
                              hipStream_t st);
size_t corr_logits_smem(int A, int M, int r, int wtype);
// marginal scoring: the whole depth loop, one workgroup per request
hipError_t launch_select_marginal(int b, int M, int K, int W, int D, const int32_t *C,
                                  const float *Cl, const TreeBufs &t, hipStream_t st);
// branch a of request q reads its M logits at ell + q * ldq + a * lda
hipError_t launch_select(int b, int A, int M, int K, int W, int D, int delta,
                         int off, const int32_t *C, const float *ell, long ldq, int lda,
                         const TreeBufs &t, hipStream_t st);
// selection spread over many workgroups (bf16 W2, 16-byte aligned, r % 8 ==
// 0, r <= 512, M <= 128): correction logits and Top-K per branch, then Top-W
// per request; ckey / ccand hold b * A * K child keys and candidate indices,
// t.selflag b * 64 arrival flags (cleared at the round start)
size_t branch_select_smem(int r);   // dynamic LDS (beside about 30 KB of static LDS)
hipError_t branch_select_prepare(size_t lds_bytes);
hipError_t launch_branch_select(int b, int A, int M, int K, int W, int D, int delta, int off,
                                int r, const void *W2, const int32_t *C, const float *Cl,
                                const float *u, int ldu, const TreeBufs &t, uint64_t *ckey,
                                int32_t *ccand, hipStream_t st);
hipError_t launch_topb_emit(int b, int NT, int B, float beta, int Bmax,
                            const TreeBufs &t, int32_t *tok, int32_t *parent,
                            int32_t *depth, float *score, uint8_t *mask,
                            int32_t *n_nodes, hipStream_t st);
size_t topb_smem(int NT, int B);
hipError_t topb_prepare(size_t lds_bytes);

// ---- persistent depth loop (small batches) and its correction tables
struct PersistArgs {
  int b, D, M, K, W, s, e, V;
  const void *W_ih, *W_hh, *Emb;
  const float *b_ih, *b_hh;
  const int32_t *C, *root;
  const float *G, *g;
  float *T0, *T1;        // published states (persist_terms_floats each)
  float *part, *gitab;
  uint32_t *flags;
  uint32_t *host_fail;   // device address of a host-visible word (or null)
  uint32_t spin;         // polls before a wait gives up (0: the default)
  uint32_t epoch0;
  TreeBufs t;
  int markov;            // nonzero: zero-state GRU steps (no W_hh product)
};
bool persist_eligible(int b, int D, int M, int K, int W, int s, int e, int r, int wtype,
                      size_t lds_max);
size_t persist_flag_words(int s);
size_t persist_part_floats(int s);
size_t persist_gitab_floats(int s, int D);
size_t persist_terms_floats(int s);
hipError_t persist_prepare(int s);
// W1t = W1[:, d:]^T zero-padded to [s, (r + 31) & ~31] bf16 (made once)
size_t corr_w1t_elems(int s, int r);
hipError_t launch_transpose_w1s(const void *W1, int r, int s, int d, int ldw1, void *W1t,
                                hipStream_t st);
hipError_t launch_corr_tables(int rows, int M, int r, int s, const void *W2, const void *W1t,
                              const int32_t *C, const float *Cl, const float *uH, float *G,
                              float *g, hipStream_t st);
hipError_t launch_depth_persistent(const PersistArgs &a, bool cooperative, hipStream_t st);
hipError_t corr_logits_prepare(int wtype, size_t lds_bytes);

// ---- sequential best-first builder (k_heap.hip)
// Per request: a node table of NH entries (push order, node 0 = the root),
// the pop sequence and expansion flags of Bcap steps, the GRU state and the
// state product [u | W_hh S + b_hh] of every expansion slot (Bcap + 1), and
// the GRU input projections of all candidates [b D M, 3s].
// Node table of the best-first builder, NH nodes per request in push order.
struct HeapBufs {
  int NH = 0, Bcap = 0;
  int32_t *tok = nullptr, *par = nullptr, *dep = nullptr;
  float *score = nullptr;
  int32_t *gref = nullptr;    // [NH][2]: candidate index at its depth, parent's expansion slot
  uint64_t *pv = nullptr;     // packed pop value; 0 once popped (and for the root)
  int32_t *nnodes = nullptr;  // [batch] nodes pushed so far
  int32_t *pops = nullptr;    // [batch][Bcap] node popped at each step
  int32_t *ex = nullptr;      // [batch][4] node the next step expands (-1: none), its depth
                              // and score bits
  float *S = nullptr, *UH = nullptr, *gi = nullptr;
};
struct HeapStepArgs {
  int batch, t, B, D, M, K, s, r, markov, V;
  float beta;
  const void *W2;
  int w2_bf16;
  const int32_t *C;
  const float *Cl, *uH;
  const int32_t *root;
  const float *S_root, *b_hh;
  HeapBufs h;
};
size_t heap_step_smem(int NH, int D, int M, int r);
size_t heap_emit_smem(int NH, int B);
hipError_t launch_heap_step(const HeapStepArgs &a, hipStream_t st);
hipError_t launch_heap_emit(int batch, int B, int D, const HeapBufs &h, int32_t *tok,
                            int32_t *parent, int32_t *depth, float *score, uint8_t *mask,
                            int32_t *n_nodes, hipStream_t st);
hipError_t heap_prepare(size_t lds_bytes);

// ---- tree-attention verification (k_attn.hip)
struct TreeAttnArgs {
  int batch, n_max, Hq, Hkv, dh, L_cap, splits;
  const void *Q, *K, *V;
  const int32_t *prefix_len, *n_nodes;
  const uint8_t *mask;
  float scale;
  float *O;
  void *workspace;
};
// key splits per row block (requested > 0 is taken as is)
int tree_attn_splits(int batch, int n_max, int Hq, int Hkv, int L_cap, int requested);
size_t tree_attn_workspace(int batch, int n_max, int Hq, int Hkv, int dh, int splits);
hipError_t launch_tree_attn(const TreeAttnArgs &a, hipStream_t st);

}  // namespace dtree
