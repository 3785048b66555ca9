/*
 * Oracle for the DFlash 2 candidate-selector lattice: plain, slow, fp64, single-threaded C.
 *
 * TEST INFRASTRUCTURE. This file is the correctness reference that the GPU library is checked
 * against. Only the test suite, the smoke check and the benchmark's CPU-baseline leg may load
 * it. The product library never links, calls or includes anything from here, and nothing here
 * includes or calls the product library: the two share no code.
 *
 * What is computed, and where the pages define it:
 *   - "DFlash 2: Keep Drafting Parallel" (inco.ai blog), section "A Lightweight Path Selector":
 *     keep the top 16 candidates per draft position; score every adjacent pair with
 *     S_t(a,b) = U_t(b) + <A(a) (.) H(h_t), B(b)>, a unary term plus a low-rank bilinear match of a
 *     predecessor embedding A and a successor embedding B under a context gate H(h_t); then walk
 *     greedily from the last verified token, following the best successor at each step.
 *   - "DFlash2 Lands in llama.cpp: What PR #27342 Actually Changes" (ramgpt.org), section
 *     "What llama.cpp Actually Builds for the Selector": a per-position top-k of the logits, a
 *     gather of the unary scores of those candidates, a projection of the current hidden state
 *     through the selector-hidden weight, predecessor rows for the previous position's candidates
 *     and successor rows for the current candidates; the runtime walk starts with the anchor as
 *     predecessor and at each position picks the best successor given the chosen predecessor.
 *
 * Readings taken where the pages leave a step open (each listed in the design notes):
 *   - unary = logit - logsumexp over the full vocabulary (log-softmax of the drafter's logits);
 *   - the gate is linear with no bias, activation or scale: g = h . W_sel, W_sel stored [H, r];
 *   - A = pred_cb and B = succ_cb, both materialised [V, r] tables;
 *   - candidate order: higher logit first, equal logits by lower token id (+0 and -0 are equal);
 *   - the anchor is the single predecessor of position 0, so all k rows of that position's
 *     lattice are the same row;
 *   - walk ties go to the lowest candidate index.
 *
 * Precision: every input value (fp32 or bf16) converts to double exactly; all arithmetic is in
 * double. The only library calls are exp and log from libm.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* dtype codes used by the stored inputs: 0 = IEEE binary32, 1 = bfloat16 (upper half of a
 * binary32, stored as uint16). */
enum { ORACLE_F32 = 0, ORACLE_BF16 = 1 };

/* Return codes. */
enum { ORACLE_OK = 0, ORACLE_BAD_ARG = -1 };

/* Read element i of a stored tensor as a double. bf16 -> binary32 is a 16-bit left shift of the
 * stored bits; binary32 -> double is exact. */
static double oracle_value(const void *base, int dtype, size_t i)
{
    if (dtype == ORACLE_F32)
        return (double)((const float *)base)[i];
    uint32_t bits = (uint32_t)((const uint16_t *)base)[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static int dtype_ok(int dtype) { return dtype == ORACLE_F32 || dtype == ORACLE_BF16; }

/* Candidate order: token u (logit xu) comes before token v (logit xv) when its logit is higher,
 * or the logits are equal and its id is lower. Double comparison already treats +0 and -0 as
 * equal. */
static int comes_before(double xu, int32_t u, double xv, int32_t v)
{
    return xu > xv || (xu == xv && u < v);
}

/*
 * Per-row top-k and logsumexp.
 * logits: [R, V] row-major (dtype), cand_ids: [R, k], unary: [R, k], lse: [R] (may be NULL).
 * Row i: m = max_v x_v; lse = m + log(sum_v exp(x_v - m)) with a compensated (Neumaier) sum;
 * cand_ids = the first k tokens of the candidate order, found in one pass that keeps a sorted
 * array of the best k seen so far; unary_j = x_{cand_j} - lse.
 */
int dflash2_ref_topk_lse(const void *logits, int dtype, int R, int V, int k,
                         int32_t *cand_ids, double *unary, double *lse)
{
    if (!logits || !cand_ids || !unary || !dtype_ok(dtype) || R < 0 || V < 1 || k < 1 || k > V)
        return ORACLE_BAD_ARG;
    double *best_x = (double *)malloc((size_t)k * sizeof(double));
    int32_t *best_id = (int32_t *)malloc((size_t)k * sizeof(int32_t));
    if (!best_x || !best_id) {
        free(best_x);
        free(best_id);
        return ORACLE_BAD_ARG;
    }
    for (int row = 0; row < R; ++row) {
        const size_t base = (size_t)row * (size_t)V;

        double m = -INFINITY;
        for (int v = 0; v < V; ++v) {
            double x = oracle_value(logits, dtype, base + v);
            if (x > m)
                m = x;
        }

        double sum = 0.0, comp = 0.0;
        for (int v = 0; v < V; ++v) {
            double t = exp(oracle_value(logits, dtype, base + v) - m);
            double y = sum + t;
            if (fabs(sum) >= fabs(t))
                comp += (sum - y) + t;
            else
                comp += (t - y) + sum;
            sum = y;
        }
        const double row_lse = m + log(sum + comp);

        int n = 0;
        for (int v = 0; v < V; ++v) {
            double x = oracle_value(logits, dtype, base + v);
            if (n == k && !comes_before(x, v, best_x[k - 1], best_id[k - 1]))
                continue;
            int pos = (n < k) ? n : k - 1; /* when full, the current last entry is dropped */
            while (pos > 0 && comes_before(x, v, best_x[pos - 1], best_id[pos - 1])) {
                best_x[pos] = best_x[pos - 1];
                best_id[pos] = best_id[pos - 1];
                --pos;
            }
            best_x[pos] = x;
            best_id[pos] = v;
            if (n < k)
                ++n;
        }

        for (int j = 0; j < k; ++j) {
            cand_ids[(size_t)row * k + j] = best_id[j];
            unary[(size_t)row * k + j] = best_x[j] - row_lse;
        }
        if (lse)
            lse[row] = row_lse;
    }
    free(best_x);
    free(best_id);
    return ORACLE_OK;
}

/*
 * The LM-head product with the top-k pass over it (the drafter's logits, never stored by the GPU
 * path): x[i][v] = sum_h hidden[i][h] * W_lm[v][h], then the per-row top-k and logsumexp of x as
 * defined for dflash2_ref_topk_lse. Sources: "DFlash2 Lands in llama.cpp" (ramgpt.org), section
 * "What llama.cpp Actually Builds for the Selector" (the per-position top-k over the logits of
 * the drafter's full-vocabulary projection).
 * hidden: [R, H], W_lm: [V, H] (both dtype), cand_ids: [R, k], unary: [R, k], lse: [R] (may be
 * NULL), logits: [R, V] (may be NULL; receives x).
 */
int dflash2_ref_lmhead_topk(const void *hidden, const void *W_lm, int dtype, int R, int H, int V,
                            int k, int32_t *cand_ids, double *unary, double *lse, double *logits)
{
    if (!hidden || !W_lm || !cand_ids || !unary || !dtype_ok(dtype) || R < 0 || H < 1 || V < 1 ||
        k < 1 || k > V)
        return ORACLE_BAD_ARG;
    double *x = (double *)malloc((size_t)V * sizeof(double));
    double *top_x = (double *)malloc((size_t)k * sizeof(double));
    int32_t *top_id = (int32_t *)malloc((size_t)k * sizeof(int32_t));
    if (!x || !top_x || !top_id) {
        free(x);
        free(top_x);
        free(top_id);
        return ORACLE_BAD_ARG;
    }
    for (int row = 0; row < R; ++row) {
        /* the product: one dot product per vocabulary row */
        for (int v = 0; v < V; ++v) {
            double dot = 0.0;
            for (int h = 0; h < H; ++h)
                dot += oracle_value(hidden, dtype, (size_t)row * H + h) *
                       oracle_value(W_lm, dtype, (size_t)v * H + h);
            x[v] = dot;
            if (logits)
                logits[(size_t)row * V + v] = dot;
        }

        double mx = -INFINITY;
        for (int v = 0; v < V; ++v)
            if (x[v] > mx)
                mx = x[v];
        double total = 0.0, carry = 0.0;
        for (int v = 0; v < V; ++v) {
            double t = exp(x[v] - mx);
            double y = total + t;
            if (fabs(total) >= fabs(t))
                carry += (total - y) + t;
            else
                carry += (t - y) + total;
            total = y;
        }
        const double x_lse = mx + log(total + carry);

        int n = 0;
        for (int v = 0; v < V; ++v) {
            if (n == k && !comes_before(x[v], v, top_x[k - 1], top_id[k - 1]))
                continue;
            int pos = (n < k) ? n : k - 1;
            while (pos > 0 && comes_before(x[v], v, top_x[pos - 1], top_id[pos - 1])) {
                top_x[pos] = top_x[pos - 1];
                top_id[pos] = top_id[pos - 1];
                --pos;
            }
            top_x[pos] = x[v];
            top_id[pos] = v;
            if (n < k)
                ++n;
        }
        for (int j = 0; j < k; ++j) {
            cand_ids[(size_t)row * k + j] = top_id[j];
            unary[(size_t)row * k + j] = top_x[j] - x_lse;
        }
        if (lse)
            lse[row] = x_lse;
    }
    free(x);
    free(top_x);
    free(top_id);
    return ORACLE_OK;
}

/*
 * Context gate: g[i][d] = sum_h hidden[i][h] * W_sel[h][d].
 * hidden: [R, H], W_sel: [H, r] (both act_dtype), g: [R, r].
 */
int dflash2_ref_gate(const void *hidden, const void *W_sel, int act_dtype, int R, int H, int r,
                     double *g)
{
    if (!hidden || !W_sel || !g || !dtype_ok(act_dtype) || R < 0 || H < 1 || r < 1)
        return ORACLE_BAD_ARG;
    for (int i = 0; i < R; ++i)
        for (int d = 0; d < r; ++d) {
            double acc = 0.0;
            for (int h = 0; h < H; ++h)
                acc += oracle_value(hidden, act_dtype, (size_t)i * H + h) *
                       oracle_value(W_sel, act_dtype, (size_t)h * r + d);
            g[(size_t)i * r + d] = acc;
        }
    return ORACLE_OK;
}

/*
 * Transition lattice.
 * edges[b][p][i][j] = unary[b][p][j] + sum_d pred_cb[prev_i][d] * succ_cb[cand_j][d] * g[b][p][d]
 * with cand_j = cand_ids[b][p][j], prev_i = anchor_ids[b] when p = 0 (every i) and
 * prev_i = cand_ids[b][p-1][i] otherwise.
 * cand_ids, unary: [B, L, k]; g: [B, L, r]; pred_cb, succ_cb: [V, r] (cb_dtype); anchor_ids: [B];
 * edges: [B, L, k, k].
 */
int dflash2_ref_lattice(const int32_t *cand_ids, const double *unary, const double *g,
                        const void *pred_cb, const void *succ_cb, int cb_dtype,
                        const int32_t *anchor_ids, int B, int L, int V, int r, int k,
                        double *edges)
{
    if (!cand_ids || !unary || !g || !pred_cb || !succ_cb || !anchor_ids || !edges ||
        !dtype_ok(cb_dtype) || B < 0 || L < 1 || V < 1 || r < 1 || k < 1)
        return ORACLE_BAD_ARG;
    for (int b = 0; b < B; ++b) {
        if (anchor_ids[b] < 0 || anchor_ids[b] >= V)
            return ORACLE_BAD_ARG;
        for (int p = 0; p < L; ++p) {
            const size_t row = (size_t)b * L + p;
            for (int i = 0; i < k; ++i) {
                const int32_t prev = (p == 0) ? anchor_ids[b] : cand_ids[(row - 1) * k + i];
                if (prev < 0 || prev >= V)
                    return ORACLE_BAD_ARG;
                for (int j = 0; j < k; ++j) {
                    const int32_t cand = cand_ids[row * k + j];
                    if (cand < 0 || cand >= V)
                        return ORACLE_BAD_ARG;
                    double acc = 0.0;
                    for (int d = 0; d < r; ++d)
                        acc += oracle_value(pred_cb, cb_dtype, (size_t)prev * r + d) *
                               oracle_value(succ_cb, cb_dtype, (size_t)cand * r + d) *
                               g[row * r + d];
                    edges[(row * k + i) * k + j] = unary[row * k + j] + acc;
                }
            }
        }
    }
    return ORACLE_OK;
}

/*
 * Greedy walk. For each sequence: the predecessor index starts at 0 (at position 0 every lattice
 * row is the anchor's row); at position p the chosen index is the lowest j with the largest
 * edges[b][p][prev][j]; path = cand_ids[b][p][j]; then prev = j.
 * Diagnostics: path_idx [B, L] (chosen j), margin [B, L] (best edge minus the best other edge
 * in the same row, +inf when k = 1), score [B] (sum of the chosen edges). Any diagnostic
 * pointer may be NULL.
 */
int dflash2_ref_walk(const double *edges, const int32_t *cand_ids, int B, int L, int k,
                     int32_t *path, int32_t *path_idx, double *margin, double *score)
{
    if (!edges || !cand_ids || !path || B < 0 || L < 1 || k < 1)
        return ORACLE_BAD_ARG;
    for (int b = 0; b < B; ++b) {
        int prev = 0;
        double total = 0.0;
        for (int p = 0; p < L; ++p) {
            const size_t row = (size_t)b * L + p;
            const double *e = edges + (row * k + prev) * k;
            int best = 0;
            for (int j = 1; j < k; ++j)
                if (e[j] > e[best])
                    best = j;
            double second = -INFINITY;
            for (int j = 0; j < k; ++j)
                if (j != best && e[j] > second)
                    second = e[j];
            path[row] = cand_ids[row * k + best];
            if (path_idx)
                path_idx[row] = best;
            if (margin)
                margin[row] = (k == 1) ? INFINITY : e[best] - second;
            total += e[best];
            prev = best;
        }
        if (score)
            score[b] = total;
    }
    return ORACLE_OK;
}

/*
 * The walk with its two further modes, on the same lattice.
 *
 * Sampling at temperature T > 0 ("DFlash 2: Keep Drafting Parallel", section "A Lightweight
 * Path Selector": sampling draws from the same scores as greedy): at position p, given the
 * chosen predecessor, index j is drawn from softmax(edges[b][p][prev][.] / T). The draw is by
 * inverse CDF from the caller's uniform u = uniforms[b][p] in [0, 1): with w_j = exp((e_j - m) / T)
 * (m the row maximum) and W = sum_j w_j, j is the smallest index whose running sum
 * w_0 + ... + w_j exceeds u * W (if rounding leaves none, the last index with w_j > 0).
 * T = 0 is the greedy walk (lowest index among the maxima).
 *
 * Early stop ("DFlash2 Lands in llama.cpp", section "p_min Means Something Different Under
 * DFlash2"): the confidence of position p is the softmax of the row's transition scores at the
 * chosen index, conf_p = exp(e_j - m) / sum_i exp(e_i - m) (unscaled by T); the drafted block
 * ends before the first position with conf_p < p_min: draft_len[b] is that position, or L. The
 * walk itself still runs to the end of the block.
 *
 * Diagnostics (each may be NULL): path_idx [B, L]; conf [B, L]; cdf_margin [B, L], the distance
 * of u * W from the nearest running-sum boundary, in units of W (how far the draw was from
 * changing; +inf for greedy steps).
 */
int dflash2_ref_walk_ex(const double *edges, const int32_t *cand_ids, int B, int L, int k,
                        double temperature, const double *uniforms, double p_min,
                        int32_t *path, int32_t *path_idx, int32_t *draft_len, double *conf,
                        double *cdf_margin)
{
    if (!edges || !cand_ids || !path || B < 0 || L < 1 || k < 1 || !(temperature >= 0.0) ||
        (temperature > 0.0 && !uniforms))
        return ORACLE_BAD_ARG;
    double *w = malloc(sizeof(double) * (size_t)k);
    if (!w)
        return ORACLE_BAD_ARG;
    for (int b = 0; b < B; ++b) {
        int prev = 0;
        int stop = L;
        for (int p = 0; p < L; ++p) {
            const size_t row = (size_t)b * L + p;
            const double *e = edges + (row * k + prev) * k;
            double m = e[0];
            for (int j = 1; j < k; ++j)
                if (e[j] > m)
                    m = e[j];
            int pick = 0;
            double margin = INFINITY;
            if (temperature == 0.0) {
                for (int j = 1; j < k; ++j)
                    if (e[j] > e[pick])
                        pick = j;
            } else {
                double total = 0.0;
                for (int j = 0; j < k; ++j) {
                    w[j] = exp((e[j] - m) / temperature);
                    total += w[j];
                }
                const double target = uniforms[row] * total;
                double run = 0.0;
                pick = -1;
                for (int j = 0; j < k; ++j) {
                    run += w[j];
                    const double d = fabs(run - target) / total;
                    if (d < margin)
                        margin = d;
                    if (pick < 0 && run > target)
                        pick = j;
                }
                if (pick < 0) {
                    pick = k - 1;
                    while (pick > 0 && w[pick] == 0.0)
                        --pick;
                }
            }
            double z = 0.0;
            for (int j = 0; j < k; ++j)
                z += exp(e[j] - m);
            const double c = exp(e[pick] - m) / z;
            if (stop == L && c < p_min)
                stop = p;
            path[row] = cand_ids[row * k + pick];
            if (path_idx)
                path_idx[row] = pick;
            if (conf)
                conf[row] = c;
            if (cdf_margin)
                cdf_margin[row] = margin;
            prev = pick;
        }
        if (draft_len)
            draft_len[b] = stop;
    }
    free(w);
    return ORACLE_OK;
}

/*
 * Grouped dynamic depthwise convolution of the draft blocks ("DFlash 2: Keep Drafting Parallel",
 * section "A Lightweight Local Convolution": Conv_k(x)_t = k_{t,0} (.) x_t + k_{t,1} (.) x_{t-1},
 * each coefficient a learned base kernel plus a correction computed from the hidden state, one
 * correction per 16 channels, the first position reading the last verified token; "DFlash2
 * Lands in llama.cpp", section "Dynamic Local Convolution": the sum over taps of (static
 * weight(tap, channel) + dynamic weight(position, tap, group(channel))) * input(position - tap,
 * channel), block-local with zero padding, the same dynamic weights on both sides of a sublayer
 * with a base kernel per side).
 *
 * x [nb, T, C] (block b, row t, channel c; row 0 of a block is the last verified token),
 * base [K, C] (one side's static kernel), dyn [nb, T, K, C / G] (the dynamic corrections of each
 * output row and tap, one per group of G channels), all in `dtype`; out y [nb, T, C] doubles:
 *   y[b][t][c] = sum_{tap < K} (base[tap][c] + dyn[b][t][tap][c / G]) * x[b][t - tap][c],
 * with x[b][t'][c] = 0 for t' < 0 (nothing crosses a block boundary).
 */
int dflash2_ref_dynconv(const void *x, const void *base, const void *dyn, int dtype, int nb, int T,
                        int C, int K, int G, double *y)
{
    if (!x || !base || !dyn || !y || !dtype_ok(dtype) || nb < 0 || T < 1 || C < 1 || K < 1 ||
        G < 1 || C % G != 0)
        return ORACLE_BAD_ARG;
    const int ng = C / G;
    for (int b = 0; b < nb; ++b)
        for (int t = 0; t < T; ++t)
            for (int c = 0; c < C; ++c) {
                double acc = 0.0;
                for (int tap = 0; tap < K; ++tap) {
                    if (t - tap < 0)
                        continue;  /* zero padding at the block start */
                    const double w =
                        oracle_value(base, dtype, (size_t)tap * C + c) +
                        oracle_value(dyn, dtype, (((size_t)b * T + t) * K + tap) * ng + c / G);
                    acc += w * oracle_value(x, dtype, ((size_t)b * T + (t - tap)) * C + c);
                }
                y[((size_t)b * T + t) * C + c] = acc;
            }
    return ORACLE_OK;
}

/*
 * The whole selector: top-k + logsumexp, gate, lattice, walk, in that order, on host buffers.
 * Outputs: cand_ids [B,L,k], unary [B,L,k], edges [B,L,k,k], path [B,L]; optional diagnostics
 * lse [B,L], path_idx [B,L], margin [B,L], score [B] (NULL to skip).
 */
int dflash2_ref_select(const void *logits, int logits_dtype, const void *hidden, int act_dtype,
                       const void *W_sel, const void *pred_cb, const void *succ_cb, int cb_dtype,
                       const int32_t *anchor_ids, int B, int L, int V, int H, int r, int k,
                       int32_t *cand_ids, double *unary, double *edges, int32_t *path,
                       double *lse, int32_t *path_idx, double *margin, double *score)
{
    if (B < 0 || L < 1)
        return ORACLE_BAD_ARG;
    const int R = B * L;
    double *g = (double *)malloc(((size_t)R * r + 1) * sizeof(double));
    if (!g)
        return ORACLE_BAD_ARG;
    int rc = dflash2_ref_topk_lse(logits, logits_dtype, R, V, k, cand_ids, unary, lse);
    if (rc == ORACLE_OK)
        rc = dflash2_ref_gate(hidden, W_sel, act_dtype, R, H, r, g);
    if (rc == ORACLE_OK)
        rc = dflash2_ref_lattice(cand_ids, unary, g, pred_cb, succ_cb, cb_dtype, anchor_ids, B, L,
                                 V, r, k, edges);
    if (rc == ORACLE_OK)
        rc = dflash2_ref_walk(edges, cand_ids, B, L, k, path, path_idx, margin, score);
    free(g);
    return rc;
}
