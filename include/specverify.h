/*
 * specverify.h -- C ABI of the target-side verification step of speculative
 * decoding, for AMD Instinct MI355X (gfx950).
 *
 * What the step computes (per sequence b of B; R = B*(gamma+1) rows in all):
 *
 *   1. logits[r][v] = sum_k hidden[r][k] * W[v][k] for the gamma drafted
 *      positions plus one, all rows in one pass over W.  W is the tied
 *      embedding table, [V][d] row-major.  ("多詞元預測視覺化指南", section
 *      高效嵌入器: the LM head multiplies the hidden state by the embedding
 *      matrix; "推测解码", section 先让小模型猜: one weight read scores all
 *      gamma+1 positions.)
 *   2. p = softmax(logits) per row, temperature 1.
 *   3. For each draft i < gamma with token x = draft[b][i]: keep it iff
 *      uniforms[b][i] * q[b][i][x] <= p[row i][x]; i.e. keep outright when
 *      q <= p, else with probability p/q.  ("推测解码", section 通过的规则.)
 *   4. n = number of leading kept drafts; checking stops at the first
 *      rejection.  ("推测解码", section 留下对的，换掉错的.)
 *   5. If n < gamma the replacement is drawn from max(0, p - q) at row n,
 *      renormalised; if n == gamma the bonus token is drawn from p at row
 *      gamma.  The draw is an inverse CDF over ascending token id with
 *      u = uniforms[b][gamma]: the smallest y whose running weight sum
 *      reaches u * (total weight).  ("推测解码", sections 通过的规则 and
 *      留下对的，换掉错的.)
 *   6. out_tokens[b] = draft[b][0..n-1], y, then -1 up to gamma+1 entries.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are device pointers owned by the caller.  The
 *     library allocates nothing and keeps no state between calls (apart
 *     from the static device array of spec_verify_static).
 *   - Work is enqueued on `hip_stream` (a hipStream_t passed as void*, NULL
 *     for the null stream) and is asynchronous: outputs are valid once the
 *     stream reaches that point.  No host synchronisation, no copies.
 *   - Argument errors are returned before anything is enqueued.  A failed
 *     kernel launch returns SV_ERR_DEVICE.  Data errors are not trapped: an
 *     out-of-range draft id is treated as rejected (p = 0) and recorded in
 *     the per-sequence device status word (see sv_debug_views).
 *   - Results are bitwise deterministic for identical inputs and dims.
 *     Calls that use distinct workspaces may run concurrently.
 *   - Shapes: B in [1, 2^20], gamma in [1, 32], d in [8, 65536] and a
 *     multiple of 8, V in [1, 2^28], and B * ceil(V / 4096) < 2^31.  `hidden`, `W`, `q` and `workspace`
 *     must be 16-byte aligned (workspace: 256-byte aligned).
 *
 * Precision (what a caller may rely on, and when it holds)
 *   - Each logit is an fp32 sum of bf16 x bf16 products; the products are
 *     exact in fp32, so a logit's error is summation rounding only:
 *     |dl_j| <= gamma_{d-1} * sum_k |hidden[k] * W[j][k]|, with
 *     gamma_n = n u / (1 - n u) and u = 2^-24, whatever the order of the
 *     sum.  Rounding errors of random sign make the usual error far
 *     smaller, about a quarter of 2^-24 * sqrt(d) * max_j |l_j| (measured
 *     at d = 1536 with logits up to 90).
 *   - With eps the largest |dl_j| of a row, every probability of that row
 *     obeys |dp_j| <= p_j * (2 eps + 4e-6): the normaliser moves all p_j by
 *     the p-weighted mean of the dl, and the exp2 and reciprocal steps add
 *     under 2e-6 each.
 *   - Hence |dp_j| <= 1e-5 for every entry whenever eps <= 3e-6, and for
 *     every row whose largest p stays below 1e-5 / (2 eps + 4e-6) whatever
 *     eps is.  On the usual error above, eps <= 3e-6 holds while
 *     max_j |l_j| <= 200 / sqrt(d): logits up to about 3 at d = 4096 and 5
 *     at d = 1536.  The guaranteed condition is the worst case:
 *     gamma_{d-1} * max_j sum_k |hidden[k] W[j][k]| <= 3e-6.
 *   - Decisions are taken on these fp32 values.  An accept test agrees with
 *     the exact one unless its uniform lies within (2 eps + 4e-6) p/q of
 *     p/q; a draw agrees unless u lies within 2 (2 eps + 4e-6) / S of an
 *     edge of the normalised running sum (S the sum of the drawn weights).
 *     Logits far beyond the scale above (say |l| ~ 100 at d = 4096) only
 *     widen these bands; the results stay valid draws of fp32 arithmetic.
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__) || defined(__clang__)
#define SV_API __attribute__((visibility("default")))
#else
#define SV_API
#endif

#define SV_ABI_VERSION 5
#define SV_MAX_GAMMA 32

typedef struct {
    int32_t B;         /* sequences */
    int32_t gamma;     /* drafted tokens per sequence */
    int32_t d;         /* hidden size */
    int32_t V;         /* vocabulary size */
    int32_t w_layout;  /* how W_lmhead is laid out: SV_W_ROWS (0) or SV_W_TILED */
} sv_dims;

/* Layouts of the LM-head matrix W (sv_dims.w_layout).
 *   SV_W_ROWS   [V][d] row-major bf16: the embedding table as the model has it.
 *   SV_W_TILED  the same values in 1 KB tiles of 16 vocab rows x 32 hidden
 *               columns, written by sv_tile_w.  With nt = ceil(d / 32), entry
 *               W[v][k] sits at element ((v / 16) * nt + k / 32) * 512 +
 *               (v % 16) * 32 + k % 32; rows V .. 16 ceil(V / 16) - 1 and
 *               columns d .. 32 nt - 1 are zero.  Each k step of the GEMM then
 *               reads whole 1 KB runs of memory instead of 64 bytes from each
 *               of 16 rows 2d bytes apart.  Results are bitwise identical to
 *               SV_W_ROWS (same products, same summation order); only the
 *               speed differs: measured at d = 1536 and 4096, the LM head
 *               runs 4-12% faster tiled from 26 to 1280 rows, and from 4%
 *               slower to 2% faster below 26 rows.
 * The entry points that take sv_dims accept either; sv_sparse_head reads
 * W_lmhead as SV_W_ROWS only. */
#define SV_W_ROWS 0
#define SV_W_TILED 1

typedef enum {
    SV_OK = 0,
    SV_ERR_NULL = 1,       /* a required pointer is NULL */
    SV_ERR_DIMS = 2,       /* a dimension is outside the limits above */
    SV_ERR_WORKSPACE = 3,  /* workspace smaller than sv_workspace_bytes(dims) */
    SV_ERR_ALIGN = 4,      /* a pointer is not aligned as required */
    SV_ERR_DEVICE = 5      /* a HIP launch failed */
} sv_status;

/* Per-sequence device status bits (int32, one word per sequence). */
#define SV_DEV_BAD_DRAFT 1  /* a draft id outside [0, V) was seen (treated as rejected) */
#define SV_DEV_FALLBACK 2   /* the residual summed to <= 0; the replacement was drawn from p */
#define SV_DEV_NONFINITE 4  /* no finite positive weights at all (greedy: no logit above
                               -inf in the emitting row); token 0 was emitted */
#define SV_DEV_BAD_QID 8    /* a sparse q row listed an id >= V (the entry was ignored) */

/* ABI version of the loaded library (SV_ABI_VERSION). */
SV_API int32_t sv_abi_version(void);

/* Human-readable name of a status code (static string, never NULL). */
SV_API const char *sv_status_string(sv_status status);

/* Bytes of the SV_W_TILED form of a [V][d] matrix (2 * 16 ceil(V / 16) *
 * 32 ceil(d / 32)); 0 if V or d is outside the limits of sv_dims. */
SV_API size_t sv_tiled_w_bytes(int32_t V, int32_t d);

/* Writes the SV_W_TILED form of the row-major bf16 matrix W [V][d] into
 * W_tiled (a layout change: the bits are copied unchanged, padding is zero).
 * Both device pointers 16-byte aligned and not overlapping; tiled_bytes at
 * least sv_tiled_w_bytes(V, d) (else SV_ERR_WORKSPACE).  Enqueued on
 * hip_stream like every entry point.  A model's W is tiled once, when it is
 * loaded; the verification calls then take the tiled copy. */
SV_API sv_status sv_tile_w(const uint16_t *W, int32_t V, int32_t d, uint16_t *W_tiled,
                           size_t tiled_bytes, void *hip_stream);

/* Bytes of device workspace one call needs for `dims`; 0 if dims are invalid.
 * The workspace holds the fp32 logits [R][V], the per-row softmax
 * normalisers and argmax candidates, the draw's partial sums and, for
 * R > 64 rows, the hidden rows copied into the tiled layout of SV_W_TILED
 * (the many-row LM-head GEMM reads them so).  Its contents need no
 * initialisation and are overwritten by every call. */
SV_API size_t sv_workspace_bytes(sv_dims dims);

/* The whole verification step: stage 1 then stage 2 below.
 *   hidden       bf16 bits [B][gamma+1][d]   target final hidden states
 *   W_lmhead     bf16 bits [V][d]            LM-head (tied embedding) weights, in the
 *                                            layout dims.w_layout names
 *   draft_tokens int32 [B][gamma]            drafted token ids
 *   q            fp32 [B][gamma][V]          drafter probabilities, used as given
 *   uniforms     fp32 [B][gamma+1] in (0,1]  [:, :gamma] accept tests, [:, gamma] the draw
 *   out_tokens   int32 [B][gamma+1]          emitted tokens, -1 after the last
 *   n_accepted   int32 [B]                   leading kept drafts, 0..gamma       */
SV_API sv_status spec_verify(const uint16_t *hidden, const uint16_t *W_lmhead,
                      const int32_t *draft_tokens, const float *q, const float *uniforms,
                      sv_dims dims, int32_t *out_tokens, int32_t *n_accepted,
                      void *workspace, size_t workspace_bytes, void *hip_stream);

/* spec_verify for callers that cannot allocate device memory (code under HIP
 * graph capture, serving loops and harnesses that forbid hipMalloc): no
 * workspace argument; the workspace is a static device array of the library,
 * SV_STATIC_SCRATCH_BYTES on every device it runs on, kept until the process
 * ends.  Other arguments, results and conventions as for spec_verify.
 *   - Returns SV_ERR_WORKSPACE, before anything is enqueued, when
 *     sv_workspace_bytes(dims) exceeds SV_STATIC_SCRATCH_BYTES (49 MiB: up
 *     to 45 rows at V = 262144, 95 rows at V = 128256).
 *   - Allocates nothing.  The first call on a device looks the array's
 *     address up on the current device (hipGetSymbolAddress); `hip_stream`
 *     must belong to that device.  SV_ERR_DEVICE if the lookup fails.
 *   - Every call on one device uses the same array, which keeps the last
 *     call's contents (no clearing is needed: the step resets what it uses).
 *     Calls that can overlap on one device (different streams or host
 *     threads) race on it; the caller must serialise them. */
#define SV_STATIC_SCRATCH_BYTES ((size_t)49 << 20)
SV_API sv_status spec_verify_static(const uint16_t *hidden, const uint16_t *W_lmhead,
                             const int32_t *draft_tokens, const float *q, const float *uniforms,
                             sv_dims dims, int32_t *out_tokens, int32_t *n_accepted,
                             void *hip_stream);

/* Stage 1 alone: the LM-head GEMM for all R rows in one pass over W, writing
 * the fp32 logits and per-tile softmax and argmax partials into the workspace.
 * (Steps 1-2 above.) */
SV_API sv_status sv_lmhead(const uint16_t *hidden, const uint16_t *W_lmhead, sv_dims dims,
                    void *workspace, size_t workspace_bytes, void *hip_stream);

/* Stage 1 with a choice of what it stores: flags is a bitwise OR of
 *   SV_LMHEAD_LOGITS  the fp32 logits, which sv_accept_and_draw, its sparse-q
 *                     form and sv_debug_views read
 *   SV_LMHEAD_ARGMAX  the argmax partials, which sv_accept_greedy reads
 * (the softmax partials are always stored).  sv_lmhead is
 * flags = SV_LMHEAD_LOGITS | SV_LMHEAD_ARGMAX; spec_verify, spec_verify_static,
 * spec_verify_sparse_q and spec_verify_tree launch SV_LMHEAD_LOGITS; spec_verify_greedy
 * SV_LMHEAD_ARGMAX.  Other bits: SV_ERR_DIMS.  Arguments otherwise as for sv_lmhead. */
#define SV_LMHEAD_LOGITS 1
#define SV_LMHEAD_ARGMAX 2
SV_API sv_status sv_lmhead_ex(const uint16_t *hidden, const uint16_t *W_lmhead, sv_dims dims,
                       int32_t flags, void *workspace, size_t workspace_bytes, void *hip_stream);

/* Stage 2 alone: softmax normalisers, accept tests, first rejection and the
 * replacement/bonus draw, from the logits and partials stage 1 left in the
 * same workspace, with the same dims, on the same device (stage 1 also
 * resets the per-sequence counters stage 2 uses).  (Steps 2-6 above.) */
SV_API sv_status sv_accept_and_draw(const int32_t *draft_tokens, const float *q, const float *uniforms,
                             sv_dims dims, int32_t *out_tokens, int32_t *n_accepted,
                             void *workspace, size_t workspace_bytes, void *hip_stream);

/* Greedy (match) verification -- the deterministic form of the same step.
 * The target's prediction at row i is its greedy token t_i: the largest
 * logit of the row, the lowest id among equal maxima (NaN never wins).
 * Draft i is kept while draft[b][i] == t_i; at the first mismatch n (or n =
 * gamma when all match) t_n is emitted, so out_tokens[b] = t_0..t_n, -1 after:
 * exactly the target's own greedy continuation.  (The maxstudionews.com
 * article 1664 on multi-token prediction for Gemini Nano, paragraphs on the
 * draft / verify split and on bit-identical output; "推测解码", section
 * 先让小模型猜: guess-then-check in its greedy form.)
 *   hidden, W_lmhead, draft_tokens, out_tokens, n_accepted  as for spec_verify
 *   target_tokens int32 [B][gamma+1] or NULL  t_i of every row (-1 where a row
 *                 has no logit above -inf)
 * No q and no uniforms.  The logits are not stored (only per-workgroup
 * argmax and softmax partials): after this call the workspace's logits,
 * row_max and row_sumexp views are stale; status is valid. */
SV_API sv_status spec_verify_greedy(const uint16_t *hidden, const uint16_t *W_lmhead,
                             const int32_t *draft_tokens, sv_dims dims, int32_t *out_tokens,
                             int32_t *n_accepted, int32_t *target_tokens, void *workspace,
                             size_t workspace_bytes, void *hip_stream);

/* Stage 2 of greedy verification alone, after sv_lmhead (or a previous
 * spec_verify_greedy) on the same workspace, dims and device.  Arguments as
 * for spec_verify_greedy. */
SV_API sv_status sv_accept_greedy(const int32_t *draft_tokens, sv_dims dims, int32_t *out_tokens,
                           int32_t *n_accepted, int32_t *target_tokens, void *workspace,
                           size_t workspace_bytes, void *hip_stream);

/* Verification with the drafter's q given sparsely: K (id, value) entries
 * per drafted position instead of a dense [V] row.  The result is that of
 * spec_verify on the dense row holding those values at those ids and 0
 * elsewhere -- the form a clustered drafter head produces, whose q is exactly
 * 0 outside its chosen clusters ("多詞元預測視覺化指南", section 高效嵌入器;
 * the rule itself: "推测解码", section 通过的规则).  Only the K entries of a
 * row are read, never V floats.
 *   q_ids   int32 [B][gamma][K]  token ids, in any order; ids < 0 are padding
 *                                (a row with fewer entries pads with -1);
 *                                ids >= V are ignored and set SV_DEV_BAD_QID
 *   q_vals  fp32  [B][gamma][K]  q at those ids; negative and NaN values count
 *                                as 0; an id listed twice takes the larger value
 *   K       entries per row, 1 <= K <= 2^24
 * Other arguments and the workspace as for spec_verify.  q_ids and q_vals
 * must be 16-byte aligned. */
SV_API sv_status spec_verify_sparse_q(const uint16_t *hidden, const uint16_t *W_lmhead,
                               const int32_t *draft_tokens, const int32_t *q_ids,
                               const float *q_vals, int32_t K, const float *uniforms,
                               sv_dims dims, int32_t *out_tokens, int32_t *n_accepted,
                               void *workspace, size_t workspace_bytes, void *hip_stream);

/* Stage 2 of spec_verify_sparse_q alone, after sv_lmhead on the same
 * workspace, dims and device. */
SV_API sv_status sv_accept_and_draw_sparse_q(const int32_t *draft_tokens, const int32_t *q_ids,
                                      const float *q_vals, int32_t K, const float *uniforms,
                                      sv_dims dims, int32_t *out_tokens, int32_t *n_accepted,
                                      void *workspace, size_t workspace_bytes,
                                      void *hip_stream);

/* ------------------------------------------------------------------------
 * Tree verification: several drafted candidates per position, laid out as a
 * static tree, all scored by the same single pass over W, and checked with
 * the rule of spec_verify at every fork ("推测解码", section on later
 * methods: EAGLE checks its guess tree with the same rule at every fork,
 * which keeps the distribution; sections 通过的规则 and 留下对的，换掉错的 for
 * the rule).  At a node, its children are tested in increasing node index:
 * the first with r * q(x) <= p(x) against p of the node's row, each later
 * one against the renormalised residual max(0, cur - q) / sum the previous
 * rejection left.  A kept child is emitted and checking continues at its
 * row with its own children; when every child is rejected the token is
 * drawn from the last residual, and at a node without children the bonus
 * token is drawn from p of its row (inverse CDF over ascending id, u =
 * uniforms[b][T]).  A path topology (parent[t] = t - 1) is spec_verify.
 *
 *   parent       HOST int32 [T]: parent[t] < t, -1 for the root's children
 *   hidden       bf16 bits [B][T+1][d]: row 0 the root (last context
 *                position), row t+1 node t
 *   tree_tokens  int32 [B][T]: the candidate token of every node
 *   q            fp32 [B][P][V]: the drafter's q at every row that has
 *                children, in row order (P such rows; sv_tree_shape)
 *   uniforms     fp32 [B][T+1] in (0,1]: [:, t] node t's test, [:, T] the draw
 *   dims         B, gamma = T, d, V
 *   out_tokens   int32 [B][D+1]: the kept tokens root to leaf, the drawn
 *                token, -1 after (D = depth of the deepest node)
 *   n_accepted   int32 [B]: kept tokens
 *   path_nodes   int32 [B][D] or NULL: node index of every kept token, -1 after
 * The workspace is sv_tree_workspace_bytes(dims).  Work on the stream: the
 * LM head, then 1 + 2 * rounds launches (rounds from sv_tree_shape). */
#define SV_MAX_TREE_NODES 64

/* Depth D, q rows P and launch rounds of a topology; SV_ERR_DIMS if parent
 * is not a valid tree (1 <= T <= SV_MAX_TREE_NODES, -1 <= parent[t] < t).
 * Host only; any output may be NULL. */
SV_API sv_status sv_tree_shape(const int32_t *parent, int32_t T, int32_t *depth, int32_t *q_rows,
                        int32_t *rounds);

/* Workspace bytes of spec_verify_tree (dims.gamma = T); 0 if dims are invalid. */
SV_API size_t sv_tree_workspace_bytes(sv_dims dims);

SV_API sv_status spec_verify_tree(const uint16_t *hidden, const uint16_t *W_lmhead,
                           const int32_t *parent, const int32_t *tree_tokens, const float *q,
                           const float *uniforms, sv_dims dims, int32_t *out_tokens,
                           int32_t *n_accepted, int32_t *path_nodes, void *workspace,
                           size_t workspace_bytes, void *hip_stream);

/* ------------------------------------------------------------------------
 * The drafter's clustered sparse LM head, which produces that sparse q
 * ("多詞元預測視覺化指南", section 高效嵌入器): the vocabulary is grouped into C
 * clusters of M tokens, each cluster with an embedding of its own.  For each
 * of N hidden rows h:
 *   1. score[c] = h . centroids[c] for every cluster (fp32);
 *   2. the k clusters with the largest scores are chosen (ties to the lower
 *      cluster id), listed in ascending cluster id;
 *   3. the row's K = k*M token ids are the chosen clusters' members, cluster
 *      by cluster in that order, each cluster's in the members table's order;
 *   4. logit[j] = h . W[id_j] and q = softmax over those K logits (fp32).
 * Members outside [0, V) are dropped: their slots get id -1 and q = 0. */
#define SV_HEAD_MAX_CLUSTERS 8192

typedef struct {
    int32_t N;   /* hidden rows, 1..65535 */
    int32_t d;   /* hidden size, 8..65536, a multiple of 8 */
    int32_t V;   /* vocabulary size (rows of W), 1..2^28 */
    int32_t C;   /* clusters, 1..SV_HEAD_MAX_CLUSTERS */
    int32_t M;   /* tokens per cluster (width of the members table), >= 1 */
    int32_t k;   /* clusters chosen per row, 1..C; k*M <= 2^24 */
} sv_head_dims;

/* Device workspace bytes of sv_sparse_head (0 if dims are invalid). */
SV_API size_t sv_sparse_head_workspace_bytes(sv_head_dims dims);

/*   h          bf16 bits [N][d]   drafter hidden states
 *   W_lmhead   bf16 bits [V][d]   the tied embedding table, row-major (SV_W_ROWS)
 *   centroids  bf16 bits [C][d]   one embedding per cluster
 *   members    int32 [C][M]       token ids of each cluster
 *   q_ids      int32 [N][k*M]     out: the row's token ids (step 3)
 *   q_vals     fp32  [N][k*M]     out: q at those ids
 *   clusters   int32 [N][k]       out, may be NULL: the chosen clusters
 * h, W_lmhead and centroids must be 16-byte aligned, the workspace 256-byte
 * aligned.  Conventions as for the entry points above.  The outputs feed
 * spec_verify_sparse_q directly (N = B*gamma rows, K = k*M). */
SV_API sv_status sv_sparse_head(const uint16_t *h, const uint16_t *W_lmhead,
                         const uint16_t *centroids, const int32_t *members, sv_head_dims dims,
                         int32_t *q_ids, float *q_vals, int32_t *clusters, void *workspace,
                         size_t workspace_bytes, void *hip_stream);

/* Device pointers into `workspace` for inspection after a call completes,
 * for the dims that call was given (for spec_verify_tree: gamma = T, so R =
 * B*(T+1) rows):
 *   logits      fp32 [R][V]
 *   row_max     fp32 [R]      max_v logits[r][v]
 *   row_sumexp  fp32 [R]      sum_v exp(logits[r][v] - row_max[r])
 *   status      int32 [B]     SV_DEV_* bits of the last call
 * Any output pointer may be NULL.  Pure pointer arithmetic: enqueues nothing. */
SV_API sv_status sv_debug_views(const void *workspace, sv_dims dims, const float **logits,
                         const float **row_max, const float **row_sumexp,
                         const int32_t **status);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */
