/*
 * dflash2.h - C ABI of the MI355X (gfx950) DFlash 2 candidate-selector library (libdflash2.so).
 *
 * What it computes. For every position of a speculative draft block the selector keeps the
 * drafter's top-k candidate tokens, scores every adjacent candidate pair and walks the resulting
 * lattice greedily:
 *   - "DFlash 2: Keep Drafting Parallel" (inco.ai blog), section "A Lightweight Path Selector":
 *     top 16 candidates per position; pair score S_t(a,b) = U_t(b) + <A(a) (.) H(h_t), B(b)>, a
 *     unary term plus a low-rank bilinear match of a predecessor embedding A(a) and a successor
 *     embedding B(b) under a context gate H(h_t); a greedy walk from the last verified token.
 *   - "DFlash2 Lands in llama.cpp: What PR #27342 Actually Changes" (ramgpt.org), section "What
 *     llama.cpp Actually Builds for the Selector": per-position top-k of the logits, the unary
 *     scores of the candidates, the hidden state projected through the selector-hidden weight,
 *     predecessor codebook rows for the previous position's candidates and successor rows for
 *     the current ones; the walk starts from the anchor and follows the best successor.
 * Readings fixed by this library where the pages leave a step open:
 *   unary = logit - logsumexp(all V logits of the row); g = h . W_sel (linear, no bias/scale);
 *   A = pred_cb, B = succ_cb; candidate order = higher logit first, equal logits by lower id,
 *   +0 == -0; the anchor is the single predecessor of position 0; walk ties go to the lowest
 *   candidate index.
 *
 * Conventions for every entry point.
 *   - Tensors are dense, row-major and contiguous. "Device" pointers are GPU memory the caller
 *     owns (e.g. from PyTorch); the library never allocates, frees or keeps them.
 *   - Every pointer argument must be 16-byte aligned (DFLASH2_ERR_ALIGNMENT otherwise).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and the call returns
 *     without synchronising. Outputs are valid once the stream reaches that point.
 *   - Arguments are validated on the host before anything is launched; on any error nothing is
 *     enqueued and outputs are untouched. A failed launch returns DFLASH2_ERR_HIP.
 *   - Device-side preconditions (not checked on the host): logits are finite with |x| < 1e37;
 *     ids in anchor_ids / cand_ids lie in [0, V). A lattice row whose predecessor or candidate
 *     id lies outside [0, V) is written as NaN instead of being read out of bounds.
 *   - Concurrent calls on different streams are safe when each has its own workspace.
 *   - Results are deterministic: the same inputs give bit-identical outputs on every run.
 */
#ifndef DFLASH2_H
#define DFLASH2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DFLASH2_ABI_VERSION 3
#define DFLASH2_MAX_K 64  /* largest top-k */
#define DFLASH2_MAX_R 256 /* largest codebook rank r */
#define DFLASH2_MAX_V (1 << 28) /* largest vocabulary (a row's bytes stay within 32-bit offsets) */
#define DFLASH2_MAX_CONV_TAPS 8 /* largest kernel of dflash2_dynconv */
#define DFLASH2_LMHEAD_MAX_K 16 /* largest k of dflash2_lmhead_topk */
#define DFLASH2_LMHEAD_MAX_ROWS 16 /* largest R of dflash2_lmhead_topk (one 16-row tile) */

typedef enum dflash2_dtype {
    DFLASH2_F32 = 0,  /* IEEE binary32 */
    DFLASH2_BF16 = 1  /* bfloat16: the upper 16 bits of a binary32 */
} dflash2_dtype;

typedef enum dflash2_status {
    DFLASH2_OK = 0,
    DFLASH2_ERR_INVALID_ARG = -1, /* a size or dtype out of range, or a NULL pointer */
    DFLASH2_ERR_UNSUPPORTED = -2, /* a valid request this build does not implement */
    DFLASH2_ERR_ALIGNMENT = -3,   /* a pointer is not 16-byte aligned */
    DFLASH2_ERR_WORKSPACE = -4,   /* workspace missing or smaller than required */
    DFLASH2_ERR_HIP = -5          /* the HIP runtime reported an error at launch */
} dflash2_status;

/* ABI version of the loaded library (DFLASH2_ABI_VERSION). */
int dflash2_version(void);

/* Static description of a status code (never NULL). */
const char *dflash2_status_string(int status);

/*
 * dflash2_select - the whole selector in one call: top-k + logsumexp, gate, lattice, walk.
 *
 *   logits      [B, L, V]  logits_dtype, device. Row (b, p) is the drafter's output at draft
 *                          position p of sequence b (the row of hidden[b][p]).
 *   hidden      [B, L, H]  act_dtype, device. The drafter's final hidden state per position.
 *   W_sel       [H, r]     act_dtype, device. Selector-hidden projection; g = hidden . W_sel.
 *   pred_cb     [V, r]     cb_dtype, device. Predecessor codebook A.
 *   succ_cb     [V, r]     cb_dtype, device. Successor codebook B.
 *   anchor_ids  [B]        int32, device. Last verified token of each sequence.
 *   B, L, V, H, r, k       B, L, H >= 1; 1 <= V <= DFLASH2_MAX_V; 1 <= r <= DFLASH2_MAX_R;
 *                          1 <= k <= min(V, DFLASH2_MAX_K).
 * Outputs (device, written in full):
 *   cand_ids    [B, L, k]     int32. The first k tokens of the candidate order.
 *   unary       [B, L, k]     float. logit - logsumexp(row), in candidate order.
 *   edges       [B, L, k, k]  float. edges[b][p][i][j] = unary[b][p][j]
 *                               + sum_d pred_cb[prev_i][d] * succ_cb[cand_j][d] * g[b][p][d],
 *                             prev_i = cand_ids[b][p-1][i] for p >= 1; for p = 0 every row i
 *                             uses prev = anchor_ids[b], so the k rows are identical.
 *   path        [B, L]        int32 token ids of the greedy walk: j_0 = argmax_j edges[b][0][0][j],
 *                             j_p = argmax_j edges[b][p][j_{p-1}][j] (lowest j on ties),
 *                             path[b][p] = cand_ids[b][p][j_p].
 *   workspace / workspace_bytes: device scratch of at least dflash2_workspace_bytes(...) bytes
 *                             (may be NULL when that is 0); contents need no initialisation and
 *                             are overwritten.
 * Scores accumulate in fp32.
 */
size_t dflash2_workspace_bytes(int B, int L, int V, int H, int r, int k);

int dflash2_select(const void *logits, int logits_dtype, const void *hidden, int act_dtype,
                   const void *W_sel, const void *pred_cb, const void *succ_cb, int cb_dtype,
                   const int32_t *anchor_ids, int B, int L, int V, int H, int r, int k,
                   int32_t *cand_ids, float *unary, float *edges, int32_t *path, void *workspace,
                   size_t workspace_bytes, void *stream);

/*
 * dflash2_select_noalloc - dflash2_select for callers that cannot allocate device memory (code
 *   under HIP graph capture, tight serving loops, harnesses that forbid allocation). Same
 *   arguments, outputs and errors as dflash2_select, without the workspace: the library's own
 *   scratch array of DFLASH2_NOALLOC_SCRATCH_BYTES bytes per GPU serves as the workspace. The
 *   call allocates nothing. The array belongs to the device current at the call (the stream must
 *   be one of that device's); it is found once per device, on the first call made with that
 *   device current, and is held until the process ends.
 *   - A call whose dflash2_workspace_bytes(B, L, V, H, r, k) exceeds
 *     DFLASH2_NOALLOC_SCRATCH_BYTES returns DFLASH2_ERR_WORKSPACE before anything is launched.
 *   - Every call on one GPU shares that GPU's array and leaves its contents behind; nothing in
 *     it needs clearing between calls. Calls that overlap on one GPU (several streams or host
 *     threads) race on the array: the caller must order them.
 *   - Failing to find the array's device address returns DFLASH2_ERR_HIP.
 */
#define DFLASH2_NOALLOC_SCRATCH_BYTES (16u << 20) /* 16 MiB per GPU */

int dflash2_select_noalloc(const void *logits, int logits_dtype, const void *hidden,
                           int act_dtype, const void *W_sel, const void *pred_cb,
                           const void *succ_cb, int cb_dtype, const int32_t *anchor_ids, int B,
                           int L, int V, int H, int r, int k, int32_t *cand_ids, float *unary,
                           float *edges, int32_t *path, void *stream);

/*
 * dflash2_select_ex - dflash2_select with the walk's two further modes (dflash2_select is this
 *   call with temperature = 0, uniforms = NULL, p_min = 0, draft_len = NULL). Same arguments,
 *   workspace and outputs, plus:
 *   temperature   >= 0 (finite). 0: the greedy walk. > 0: sampling, "DFlash 2: Keep Drafting
 *                 Parallel" (inco.ai blog), section "A Lightweight Path Selector" (sampling draws
 *                 from the same scores): at each position, given the chosen predecessor row e,
 *                 j is drawn from softmax(e / T) by inverse CDF: with w_j = exp((e_j - max e) / T)
 *                 and W = sum_j w_j, j is the smallest index whose running sum (in index order)
 *                 exceeds u * W; if rounding leaves none, the last index with w_j > 0.
 *   uniforms      [B, L] float, device, values in [0, 1): u for each position (the caller's
 *                 random numbers; required when temperature > 0, ignored otherwise, may be NULL).
 *   p_min         early stop, "DFlash2 Lands in llama.cpp" (ramgpt.org), section "p_min Means
 *                 Something Different Under DFlash2": the confidence of position p is the softmax
 *                 of its chosen row at the chosen index, exp(e_j - max e) / sum_i exp(e_i - max e)
 *                 (not scaled by T); the drafted block ends before the first position whose
 *                 confidence is below p_min. path is still the walk over all L positions.
 *                 Any non-NaN value (<= 0: never stops).
 *   draft_len     [B] int32, device, may be NULL: the drafted block length (L if nothing
 *                 stopped it).
 * Errors as dflash2_select; a NaN or negative/infinite temperature, a NaN p_min, or
 * temperature > 0 without uniforms is DFLASH2_ERR_INVALID_ARG; a misaligned uniforms or draft_len
 * is DFLASH2_ERR_ALIGNMENT. Sampling runs the lattice and the walk as two kernels.
 */
int dflash2_select_ex(const void *logits, int logits_dtype, const void *hidden, int act_dtype,
                      const void *W_sel, const void *pred_cb, const void *succ_cb, int cb_dtype,
                      const int32_t *anchor_ids, int B, int L, int V, int H, int r, int k,
                      float temperature, const float *uniforms, float p_min, int32_t *cand_ids,
                      float *unary, float *edges, int32_t *path, int32_t *draft_len,
                      void *workspace, size_t workspace_bytes, void *stream);

/*
 * The four stages, callable one by one (same conventions; dflash2_select runs exactly these).
 *
 * dflash2_topk_lse - per row of logits [R, V]: cand_ids [R, k] and unary [R, k] as above, and
 *   (if lse is not NULL) lse [R] = logsumexp of the row. Needs
 *   dflash2_topk_lse_workspace_bytes(R, V, k, logits_dtype) bytes of workspace.
 *   Sources: blog "A Lightweight Path Selector" (top 16 per position, unary term); ramgpt
 *   "What llama.cpp Actually Builds for the Selector" (per-position top-k, gathered unary).
 */
size_t dflash2_topk_lse_workspace_bytes(int R, int V, int k, int logits_dtype);

int dflash2_topk_lse(const void *logits, int logits_dtype, int R, int V, int k, int32_t *cand_ids,
                     float *unary, float *lse, void *workspace, size_t workspace_bytes,
                     void *stream);

/*
 * dflash2_gate - g [R, r] (float) = hidden [R, H] . W_sel [H, r], act_dtype inputs, fp32
 *   accumulation (bf16 inputs run on the matrix cores). Needs dflash2_gate_workspace_bytes(R, H, r)
 *   bytes of workspace. Source: blog "A Lightweight Path Selector" (context gate H(h_t)); ramgpt
 *   "What llama.cpp Actually Builds for the Selector" (hidden state projected through the
 *   selector-hidden weight).
 */
size_t dflash2_gate_workspace_bytes(int R, int H, int r);

int dflash2_gate(const void *hidden, const void *W_sel, int act_dtype, int R, int H, int r,
                 float *g, void *workspace, size_t workspace_bytes, void *stream);

/*
 * dflash2_lattice - edges [B, L, k, k] (float) from cand_ids [B, L, k] (int32), unary [B, L, k]
 *   (float), g [B, L, r] (float), pred_cb / succ_cb [V, r] (cb_dtype) and anchor_ids [B], as in
 *   dflash2_select. No workspace. Source: blog "A Lightweight Path Selector" (eq. S_t(a,b));
 *   ramgpt "What llama.cpp Actually Builds for the Selector" (codebook gathers, anchor).
 */
int dflash2_lattice(const int32_t *cand_ids, const float *unary, const float *g,
                    const void *pred_cb, const void *succ_cb, int cb_dtype,
                    const int32_t *anchor_ids, int B, int L, int V, int r, int k, float *edges,
                    void *stream);

/*
 * dflash2_walk - path [B, L] (int32 token ids) from edges [B, L, k, k] and cand_ids [B, L, k], as
 *   in dflash2_select; path_idx [B, L] (int32, may be NULL) receives the chosen candidate index
 *   j_p. No workspace. Source: blog "A Lightweight Path Selector" (greedy walk from the last
 *   verified token); ramgpt "What llama.cpp Actually Builds for the Selector" (runtime walk).
 */
int dflash2_walk(const float *edges, const int32_t *cand_ids, int B, int L, int k, int32_t *path,
                 int32_t *path_idx, void *stream);

/*
 * dflash2_walk_ex - dflash2_walk with sampling and the p_min early stop, as in dflash2_select_ex
 *   (temperature, uniforms [B, L], p_min, draft_len [B] may be NULL). No workspace.
 */
int dflash2_walk_ex(const float *edges, const int32_t *cand_ids, int B, int L, int k,
                    float temperature, const float *uniforms, float p_min, int32_t *path,
                    int32_t *path_idx, int32_t *draft_len, void *stream);

/*
 * dflash2_dynconv - the grouped dynamic depthwise convolution of the draft blocks, one side of
 *   a sublayer per call. Source: "DFlash 2: Keep Drafting Parallel" (inco.ai blog), section
 *   "A Lightweight Local Convolution" (Conv_k(x)_t = k_{t,0} (.) x_t + k_{t,1} (.) x_{t-1}; each
 *   coefficient a learned base kernel plus a correction from the hidden state, one per 16
 *   channels; the first draft position reads the last verified token); "DFlash2 Lands in
 *   llama.cpp" (ramgpt.org), section "Dynamic Local Convolution" (static weight per tap and
 *   channel plus dynamic weight per position, tap and channel group; block-local, zero padded;
 *   the same dynamic weights on both sides of a sublayer with one base kernel per side).
 *
 *   x      [n_blocks, T, C]          dtype, device. Row 0 of a block is the last verified token,
 *                                    rows 1.. the draft positions.
 *   base   [K, C]                    dtype, device. The side's static kernel.
 *   dyn    [n_blocks, T, K, C/group] dtype, device. The dynamic correction of each output row,
 *                                    tap and channel group (computed upstream from the hidden
 *                                    state).
 *   y      [n_blocks, T, C]          dtype, device, written in full:
 *          y[b][t][c] = sum_{tap < K} (base[tap][c] + dyn[b][t][tap][c / group]) * x[b][t-tap][c],
 *          x[b][t'][c] = 0 for t' < 0 (nothing crosses a block boundary). fp32 arithmetic; bf16
 *          outputs are rounded to nearest even. y must not overlap x.
 *   n_blocks, T, C >= 1; 1 <= K <= DFLASH2_MAX_CONV_TAPS; group >= 1 divides C.
 * No workspace. Errors: DFLASH2_ERR_INVALID_ARG (sizes, dtype, NULL), DFLASH2_ERR_ALIGNMENT.
 */
int dflash2_dynconv(const void *x, const void *base, const void *dyn, int dtype, int n_blocks,
                    int T, int C, int K, int group, void *y, void *stream);

/*
 * dflash2_lmhead_topk - the drafter's LM-head product with the top-k pass folded into it: the
 *   [R, V] logits exist only in registers. Sources: "DFlash2 Lands in llama.cpp" (ramgpt.org),
 *   section "What llama.cpp Actually Builds for the Selector" (the per-position top-k over the
 *   logits of the drafter's full-vocabulary projection) and section "The Most Important
 *   Performance Question Is Now Different" (top-k extraction is one of the draft cycle's costs).
 *   The fusion is this library's design.
 *
 *   hidden   [R, H]  bf16, device, row-major. The drafter's final hidden states.
 *   W_lm     [V, H]  bf16, device, row-major. The LM-head weight (one row per vocabulary token).
 *   x[i][v] = sum_h hidden[i][h] * W_lm[v][h] (bf16 products, fp32 accumulation); then, as
 *   dflash2_topk_lse over x:
 *   cand_ids [R, k]  int32, device, out. The first k tokens of the candidate order.
 *   unary    [R, k]  fp32, device, out. x[i][cand_j] - lse_i.
 *   lse      [R]     fp32, device, out, may be NULL. logsumexp_v x[i][v].
 *   R >= 1; H >= 8 and H % 8 == 0; 1 <= V <= DFLASH2_MAX_V; 1 <= k <= min(V, DFLASH2_LMHEAD_MAX_K).
 *   R <= DFLASH2_LMHEAD_MAX_ROWS (decode: one 16-row tile, where the weight is read once and the
 *   pass is bound by that read); larger R returns DFLASH2_ERR_UNSUPPORTED: the pass would read
 *   the weight once per 16-row tile, and once several row tiles reuse it a library product
 *   followed by dflash2_topk_lse is faster.
 * Workspace: dflash2_lmhead_topk_workspace_bytes(R, H, V, k) bytes (range partials), 16-byte
 * aligned, owned by the caller; contents need not be initialised (0 for sizes the pass refuses).
 * Errors: DFLASH2_ERR_INVALID_ARG, DFLASH2_ERR_UNSUPPORTED (R > DFLASH2_LMHEAD_MAX_ROWS),
 * DFLASH2_ERR_ALIGNMENT (every pointer 16-byte aligned), DFLASH2_ERR_WORKSPACE, DFLASH2_ERR_HIP.
 */
size_t dflash2_lmhead_topk_workspace_bytes(int R, int H, int V, int k);
int dflash2_lmhead_topk(const void *hidden, const void *W_lm, int R, int H, int V, int k,
                        int32_t *cand_ids, float *unary, float *lse, void *workspace,
                        size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* DFLASH2_H */
