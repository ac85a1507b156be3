/*
 * dtree.h -- C ABI of libdtree.so: one round of conditional draft-tree
 * construction on an AMD Instinct MI355X (gfx950).
 *
 * The operation (pages cited by title and section):
 *   * "Resumen Técnico: Domino", Metodología 1 and 2: base logits
 *     L_base = H . W_lm (+ bias) from the shared hidden states H of the draft
 *     block; a GRU folds the embeddings of the preceding draft tokens into a
 *     causal state S; a low-rank head maps [H_i ; S_{i-1}] to rank r (W1) and
 *     back to vocabulary space (W2) giving Delta L_i; L = L_base + Delta L.
 *   * "Resumen Técnico: DominoTree", Componentes Principales 1, 2 and 5: children are
 *     scored by the path's own correction; the correction is restricted to
 *     the Top-M marginal candidates of each depth (an r x M slice of W2)
 *     before the Top-k children are kept; verification uses tree attention
 *     with an ancestor-only mask.
 *   * "DARTree: Speculative Diffusion Decoding with Autoregressive Draft
 *     Trees", Metodología 1 and 2: the tree grows depth by depth; every
 *     active branch of a depth is corrected in one batch with its own prefix
 *     state; extensions are scored by corrected cumulative log-probability;
 *     the W best branches are kept and their states carried forward; the
 *     fixed-width superarbol so built is pruned by ONE global Top-B with a
 *     non-positive depth bonus beta, which Lemma 1 shows selects the same
 *     set as the sequential best-first max-heap.
 *
 * Conventions fixed by this library where the pages leave them open:
 *   * log-probabilities are normalised over the M candidates of the depth;
 *   * H row delta (0-based) scores the children at depth delta+1; the GRU
 *     starts from a zero state and first consumes the root token (the last
 *     verified token), so the depth-1 children use S = GRU(Emb[root], 0);
 *   * GRU = the PyTorch GRUCell equations, gate blocks (r, z, n);
 *   * the low-rank head is linear: u = W1 [Hq_delta ; S], Delta L = W2 u;
 *   * every scored child enters the superarbol; only the top W per depth
 *     are expanded; B counts selected nodes excluding the root;
 *   * selection key = score + beta * depth (fp32), order: key descending,
 *     then depth ascending, then token path lexicographically ascending;
 *     Top-M and Top-K ties go to the smaller token id, Top-W ties to the
 *     lexicographically smaller token path;
 *   * bf16 weights: the only bf16 values are the stored weights and
 *     Hq = bf16_rne(H); the GRU state, gate pre-activations, u, the
 *     corrected logits, log-probs and scores are fp32.
 *
 * Memory: every pointer named "device" is device memory of the device the
 * context was created on.  Weights are BORROWED (the caller keeps them alive
 * and unchanged for the context's life); the context owns its workspace;
 * outputs are caller-allocated.  All calls return a dtree_status; nothing
 * throws across the ABI.  On error dtree_last_error() describes it.
 */
#ifndef DTREE_H
#define DTREE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct dtree_ctx dtree_ctx;

typedef enum {
  DTREE_OK = 0,
  DTREE_E_ARG = 1,     /* bad argument value (K > M, beta > 0, NULL, ...)   */
  DTREE_E_SHAPE = 2,   /* a size the kernels do not support                  */
  DTREE_E_DTYPE = 3,   /* unknown weight type                                */
  DTREE_E_DEVICE = 4,  /* not a gfx950 device, or device query failed        */
  DTREE_E_NOMEM = 5,   /* workspace allocation failed                        */
  DTREE_E_HIP = 6,     /* a HIP runtime call or kernel launch failed         */
  DTREE_E_STATE = 7    /* call out of order (e.g. trace before any round)    */
} dtree_status;

typedef enum { DTREE_F32 = 0, DTREE_BF16 = 1 } dtree_dtype;

/* Shared drafter weights, PyTorch module layouts, row-major, device memory.
 * Matrices are stored as `wtype` (bf16 = raw 16-bit patterns).  Biases are
 * fp32 and may be NULL (read as zeros).  The context borrows the weights:
 * they must stay valid and unchanged while it exists (it also keeps a
 * transposed copy of W1[:, d:] made by dtree_create).  With bf16 weights,
 * 16-byte aligned W_ih, W_hh, Emb and W2 let the depth loop run as a single
 * persistent kernel when the shapes allow it.                                */
typedef struct {
  int32_t d;   /* hidden size of H                                          */
  int32_t V;   /* vocabulary size, <= 262144                                 */
  int32_t e;   /* embedding size fed to the GRU                              */
  int32_t s;   /* GRU state size                                             */
  int32_t r;   /* rank of the correction bottleneck                          */
  int32_t wtype;                /* dtree_dtype                              */
  const void *W_lm;             /* [V, d]   LM head (nn.Linear(d, V).weight) */
  const float *lm_bias;         /* [V]      added to the base logits or NULL */
  const void *Emb;              /* [V, e]   token embedding table            */
  const void *W_ih;             /* [3s, e]  GRUCell.weight_ih, blocks r,z,n  */
  const void *W_hh;             /* [3s, s]  GRUCell.weight_hh                */
  const float *b_ih, *b_hh;     /* [3s]     GRUCell biases or NULL           */
  const void *W1;               /* [r, d+s] columns [0,d) act on H, [d,d+s) on S */
  const void *W2;               /* [V, r]   row v maps u to token v's logit   */
} dtree_weights;

/* Upper bounds the workspace is sized for (dtree_create).                   */
typedef struct {
  int32_t max_batch;  /* requests per round                                  */
  int32_t max_D;      /* depth, <= 31                                        */
  int32_t max_M;      /* candidates per depth, <= 128                        */
  int32_t max_K;      /* children per branch                                 */
  int32_t max_W;      /* branches per depth, <= 512                          */
  int32_t max_B;      /* node budget                                         */
} dtree_caps;

/* Per-round tree parameters.  Need 1 <= K <= M <= V, W >= 1, B >= 1,
 * 1 <= D, each within the caps, and beta <= 0 (Lemma 1's precondition:
 * beta > 0 returns DTREE_E_ARG).  The superarbol (root included) must hold
 * at most 8192 nodes and A*K <= 1024 children per depth.                    */
typedef struct {
  int32_t D, M, K, W, B;
  float beta;
} dtree_params;

/* Create a context on HIP device `device`: validates the weights and caps,
 * checks the device is gfx950 and allocates the workspace (hipMalloc).
 * bf16 weights need d % 128 == 0.  On success *out owns the workspace.      */
dtree_status dtree_create(const dtree_weights *w, const dtree_caps *caps,
                          int device, dtree_ctx **out);

/* Enqueue one round on `stream` (a hipStream_t; NULL = default stream).
 * Asynchronous: returns after enqueueing; nothing is synchronised inside.
 * Argument errors are found before anything is enqueued.
 *   H       device, [batch, D, d] fp32 hidden states (row delta scores
 *           depth delta+1)
 *   root    device, [batch] int32, last verified token of each request
 * Outputs, device, caller-owned, N = B + 1 slots per request:
 *   tok     [batch, N] int32  token of each node (row 0 = root)
 *   parent  [batch, N] int32  index of the parent node, -1 for the root
 *   depth   [batch, N] int32  depth, root 0
 *   score   [batch, N] fp32   cumulative log-prob (beta not included)
 *   mask    [batch, N, N] u8  mask[i][j] = 1 iff node j is node i or an
 *                             ancestor of it (query row, key column)
 *   n_nodes [batch] int32     min(B, superarbol size) + 1
 * Nodes are in canonical order: root, then depth ascending, then token path
 * lexicographically ascending, so parent[i] < i.  Slots past n_nodes hold
 * tok/parent/depth = -1, score = -inf and zero mask rows and columns.
 * H and root must stay valid until the stream work completes.  A context is
 * not reentrant: calls on one context must not overlap.
 * With bf16 weights and small batches the depth loop runs as one persistent
 * kernel whose workgroups wait on each other (each needs a whole CU).  It is
 * launched like any other kernel; should its workgroups not all become
 * resident together (another stream holding CUs for a long time), its waits
 * run out after a bounded time and that round fails: its n_nodes are 0 (a
 * valid round has n_nodes >= 1, so a failed round marks itself in its own
 * outputs even when rounds are queued back to back), its status gets bit 1,
 * the next dtree_build_round on the context returns DTREE_E_HIP without
 * enqueueing anything (once the failed round has run: the flag is read
 * without synchronising), and every later round uses cooperative launches,
 * which guarantee co-residency at a higher launch cost (about 18 us on
 * MI355X).                                                                  */
dtree_status dtree_build_round(dtree_ctx *ctx, const dtree_params *p,
                               int32_t batch, const float *H,
                               const int32_t *root, int32_t *tok,
                               int32_t *parent, int32_t *depth, float *score,
                               uint8_t *mask, int32_t *n_nodes, void *stream);

/* dtree_build_round for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): one round with no context, with the same arguments and
 * outputs as dtree_build_round (weights as for dtree_create; the params are
 * their own caps).  The round's whole workspace comes from one fixed array
 * inside the library, 16 MiB on each device the library runs on (held from
 * the first call until the process ends); nothing is allocated: no
 * hipMalloc, hipFree or allocating library routine.  A round whose
 * workspace exceeds 16 MiB returns DTREE_E_SHAPE before anything is
 * enqueued (the Qwen3-4B shape with one request needs about 5 MiB: the
 * per-slice candidate lists of the LM head dominate).  The depth loop runs
 * as one product, correction, selection and GRU step per depth (never the
 * persistent kernel), with no distinct-token or tiled paths.  All calls on
 * one device share that array, which keeps the last call's contents: calls
 * whose work overlaps on the device race (use one stream per device, or
 * order the streams).  Asynchronous on `stream`; argument errors return
 * before anything is enqueued; dtree_last_error(NULL) describes the last
 * failure of this call on the calling thread.                              */
dtree_status dtree_build_round_static(const dtree_weights *w, const dtree_params *p,
                                      int32_t batch, const float *H, const int32_t *root,
                                      int32_t *tok, int32_t *parent, int32_t *depth,
                                      float *score, uint8_t *mask, int32_t *n_nodes,
                                      void *stream);

/* Launch of the persistent depth loop (see dtree_build_round).
 *   cooperative  0: plain launches (the default; a context switches itself to
 *                cooperative launches after a round whose waits ran out),
 *                1: cooperative launches from now on
 *   spin_limit   polls before a wait between its workgroups gives up and the
 *                round fails with status bit 1; 0 restores the default
 *                (about a second); tests use a tiny value to exercise the
 *                failure report without a stalled GPU
 * Takes effect from the next round; DTREE_E_ARG for other values.          */
dtree_status dtree_set_persistent_launch(dtree_ctx *ctx, int32_t cooperative,
                                         int32_t spin_limit);

/* How the children of every expanded branch are scored (for the context's
 * later rounds):
 *   DTREE_SCORE_CONDITIONAL (0, the default): corrected logits
 *       L_base + Delta L, Delta L from the low-rank head over [H_i ; S] with
 *       the branch's own GRU state S ("Resumen Técnico: Domino",
 *       Metodología 2; DARTree page, Metodología 1);
 *   DTREE_SCORE_MARGINAL (1): the path-independent base logits alone
 *       (Delta L = 0, no GRU state), the uncorrected DDTree-style scoring the
 *       pages compare against with the same drafter and tree construction
 *       ("Resumen Técnico: DominoTree", Contribuciones Clave, the ablation of
 *       conditionality).  Everything else in the round is unchanged: Top-M
 *       per depth, log-softmax over M, Top-K, Top-W, global Top-B, mask;
 *   DTREE_SCORE_MARKOV (2): a first-order correction that conditions on the
 *       parent token only (DARTree page, Resultados Experimentales,
 *       Ablación: the method also helps the DSpark drafter, whose
 *       correction head is Markov).  Reading taken: a branch's causal state
 *       is the GRU applied to its last token from a zero state,
 *       S = GRU(Emb[token], 0) (the root's state is the same as in
 *       conditional scoring); the low-rank head and the rest of the round
 *       are unchanged.
 * DTREE_E_ARG for other values.                                            */
#define DTREE_SCORE_CONDITIONAL 0
#define DTREE_SCORE_MARGINAL 1
#define DTREE_SCORE_MARKOV 2
dtree_status dtree_set_scoring(dtree_ctx *ctx, int32_t scoring);

/* Which builder grows the tree (for the context's later rounds):
 *   DTREE_BUILD_DEPTHWISE (0, the default): the depth-wise batched build with
 *       a fixed-width superarbol and one global Top-B (DARTree page,
 *       Metodología 1 and 2);
 *   DTREE_BUILD_HEAP (1): the sequential best-first builder the pages
 *       compare it with ("Resumen Técnico: DominoTree", Componentes
 *       Principales 1 and 2; DARTree page, Planteamiento del Problema 3 and
 *       Resultados Experimentales, Ablación: latency): a max-priority queue
 *       of nodes keyed like the global Top-B (key = score + beta * depth
 *       descending, then depth ascending, then token path ascending), seeded
 *       with the root's Top-K children; each of the B pops runs the GRU one
 *       step along the popped node's own path and, below depth D, corrects
 *       the next depth's Top-M candidates with that state and pushes the
 *       node's Top-K children.  The popped nodes are the tree (emitted in the
 *       same canonical order, with the same mask).  Candidates per depth,
 *       log-softmax over M and the tie rules are those of the depth-wise
 *       build; W is not used.  Every pop is one heap-step kernel and one
 *       state product on the stream (2 B launches per round, no host
 *       synchronisation).  Conditional or Markov scoring (a round with
 *       marginal scoring returns DTREE_E_ARG).
 * The first switch to the heap builder allocates its tables, sized by the
 * caps (nodes max_K (max_B + 1) + 1 per request, max_B + 1 states and state
 * products, the input projections of max_batch max_D max_M candidates):
 * DTREE_E_NOMEM / DTREE_E_SHAPE if they do not fit.  DTREE_E_ARG for other
 * values.                                                                  */
#define DTREE_BUILD_DEPTHWISE 0
#define DTREE_BUILD_HEAP 1
dtree_status dtree_set_builder(dtree_ctx *ctx, int32_t builder);

/* Number of superarbol nodes (root included) a round with `p` builds per
 * request, or -1 if p is invalid.  Pure host arithmetic.                     */
int32_t dtree_superarbol_nodes(const dtree_params *p);

/* Upper bound on the nodes (root included) the heap builder pushes per
 * request with `p`: K (B + 1) + 1, or -1 if p is invalid.  Pure host
 * arithmetic.                                                               */
int32_t dtree_heap_nodes(const dtree_params *p);

/* Debug copy of request `req`'s intermediates of the LAST round, host memory,
 * caller-allocated with the sizes noted (for that round's params).  Any
 * pointer may be NULL to skip that part.  Synchronises the device.          */
typedef struct {
  int32_t *C;          /* [D*M]  candidate tokens per depth, value desc     */
  float *Cl;           /* [D*M]  their base logits                           */
  int32_t *node_tok;   /* [n_sa] superarbol, node 0 = root                   */
  int32_t *node_parent;/* [n_sa] parent node id, -1 for the root            */
  float *node_score;   /* [n_sa]                                             */
  int32_t *surv;       /* [(D+1)*W] expanded node ids per depth, -1 padded   */
  int32_t *sel;        /* [B]    selected node ids in selection order, -1 pad */
  int32_t n_sa;        /* out: superarbol nodes incl. root                   */
  int32_t status;      /* out: device status bits (0 = fine; bit 0: the
                          selection was not closed under parents; bit 1:
                          the persistent depth loop could not run all its
                          workgroups at once, the round's outputs are
                          invalid)                                          */
} dtree_trace;
/* After a heap-builder round the node arrays hold every pushed node in push
 * order (up to dtree_heap_nodes(p) entries: size them for that), sel the
 * popped node ids in pop order (-1 past the last pop), surv is all -1.      */
dtree_status dtree_get_trace(dtree_ctx *ctx, int32_t req, dtree_trace *out);

/* Stage timing with HIP events recorded on the round's own stream.  When
 * enabled, every round records events between its stages:
 *   0 round start (bf16: hidden rows rounded once; empty with fp32 weights)
 *   1 base-logit GEMM with fused per-slice Top-M (32 or more hidden rows:
 *     the logits product alone, timed by the kernel's own start and end)
 *   2 Top-M merge (32 or more hidden rows: the per-slice lists built from
 *     the logits, then the merge)
 *   3 path-independent prologue (uH, correction tables or root GRU state)
 *   4 depth loop (correction, selection, GRU, all depths; heap builder:
 *     all pops)
 *   5 global Top-B, canonical order and mask (heap builder: emission)
 * dtree_profile_read synchronises, writes the summed milliseconds of each
 * stage over the rounds recorded since dtree_profile_enable(ctx, 1) to
 * ms[0..DTREE_NSTAGES) and the round count to *rounds, and clears them.
 * At most 4096 rounds are recorded; later rounds are not timed.            */
#define DTREE_NSTAGES 6
dtree_status dtree_profile_enable(dtree_ctx *ctx, int enable);
dtree_status dtree_profile_read(dtree_ctx *ctx, float *ms, int32_t *rounds);

/* ---- tree-attention verification ------------------------------------------
 * One layer's attention of the target model's verification pass over an
 * emitted draft tree ("Resumen Técnico: DominoTree", Componentes Principales
 * 5: tree attention with an ancestor-only mask; "DARTree: Speculative
 * Diffusion Decoding with Autoregressive Draft Trees", Metodología 2,
 * verification).  Tree token i of request q attends to the request's
 * verified prefix and to the tree tokens j with mask[q][i][j] = 1 (its
 * root-to-node path, itself included, in the round's emitted convention):
 *
 *   O[q,i,h] = sum_k softmax_k(scale * Q[q,i,h] . K[q,h/G,k]) V[q,h/G,k]
 *
 * over the visible cache positions k: [0, prefix_len[q]) and
 * prefix_len[q] + j for the visible nodes j.  G = Hq / Hkv query heads share
 * one KV head (query head h reads KV head h / G).  bf16 inputs, fp32
 * scores and sums; the softmax weights enter the weighted sum of V rounded
 * to bf16 (so |O - exact| <= 2^-8 sum_k w_k |V_k| plus fp32 rounding).
 *
 * Layouts (all device memory, row-major):
 *   Q           [batch, n_max, Hq, dh] bf16 (tree token i, head h);
 *   K, V        [batch, Hkv, L_cap, dh] bf16: the KV cache, prefix at
 *               positions [0, prefix_len[q]), tree token j at prefix_len[q] + j;
 *   prefix_len  [batch] int32, n_nodes [batch] int32 (the round's n_nodes);
 *   mask        [batch, n_max, n_max] uint8 (the round's mask, n_max = B + 1);
 *   O           [batch, n_max, Hq, dh] fp32, caller-owned; rows i >= n_nodes[q]
 *               are written as 0.
 * Only positions below prefix_len[q] + n_nodes[q] are read.  The tree must be
 * in the round's canonical order (every ancestor before its descendants).
 * Limits: dh 64 or 128, Hq a multiple of Hkv with Hq / Hkv <= 64,
 * n_max <= 4096 and <= L_cap; Q, K, V, O 16-byte aligned.
 * splits: key ranges per block of 64 query rows whose partial results are
 * merged by a second kernel (0: chosen from the shape to fill the device);
 * with more than one, a workspace of dtree_tree_attention_workspace() bytes,
 * 256-byte aligned, caller-owned, is needed (NULL when that size is 0).
 * Errors: shapes and pointers are checked before anything is enqueued
 * (DTREE_E_ARG / DTREE_E_SHAPE, DTREE_E_DEVICE off gfx950); text from
 * dtree_last_error(NULL).  Per-request lengths live on the device and are
 * checked there: a request with prefix_len < 0, n_nodes outside
 * [1, n_max] or prefix_len + n_nodes > L_cap reads nothing and gets NaN in
 * every row of O.  Asynchronous on `stream`; no host synchronisation; no
 * state kept between calls (calls on different streams are independent if
 * their workspaces differ).                                                 */
typedef struct {
  int32_t batch, n_max, Hq, Hkv, dh, L_cap;
  const void *Q, *K, *V;
  const int32_t *prefix_len, *n_nodes;
  const uint8_t *mask;
  float scale;        /* > 0, e.g. 1 / sqrt(dh) */
  float *O;
  int32_t splits;     /* 0 = automatic */
  void *workspace;
  size_t workspace_bytes;
} dtree_attn_args;

dtree_status dtree_tree_attention_workspace(const dtree_attn_args *a, size_t *bytes);
dtree_status dtree_tree_attention(const dtree_attn_args *a, void *stream);

/* Text of the last error on this context ("" if none); ctx may be NULL for
 * errors of dtree_create, of the allocation-free round and of the attention
 * calls.  Valid until the next call on the context.                         */
const char *dtree_last_error(const dtree_ctx *ctx);

/* Free the workspace.  NULL-safe.  The caller must ensure no enqueued round
 * still runs (synchronise the stream first).                                */
dtree_status dtree_destroy(dtree_ctx *ctx);

#ifdef __cplusplus
}
#endif
#endif /* DTREE_H */
