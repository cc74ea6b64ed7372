/*
 * oracle.c -- plain, slow, fp64 CPU reference for masked causal attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file: only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark use it.  It shares no code, header,
 * table or helper with the GPU library.
 *
 * Every floating-point step runs in double precision.  Inputs arrive as
 * float32 arrays that hold exactly the values the GPU sees (bf16 values
 * widen to float32 without rounding), and are widened to double on read.
 * There is no blocking, fusion or reordering beyond what each cited
 * definition states: scores, maximum, exponentials, sum and weighted sum are
 * formed in that order, keys ascending, channels ascending.
 *
 * Sources (web pages about attention variants):
 *   [VAR]  "Attention Variants Compared" (aiengineeringfromscratch.com
 *          cheatsheet): the swa_mask / strided_mask code, the "Flash style
 *          softmax" tiled_softmax_dot task, the NSA key-count quiz, the
 *          variant/cost table (differential = two maps).
 *   [SSW]  "Learn: Sparse & Sliding-Window Attention" (gunjandhanuka.github.io),
 *          §3 mask equation A = softmax(QK^T/sqrt(d_k) + log M) V, §3a window,
 *          §4 rolling KV window and attention sinks, §6 FLOPs & memory table.
 *   [EXP]  "Exploring Attention Variants: Flash Attention, Sliding-Window, and
 *          Sparse Attention Implementation" (instagit.com): SWA mask range
 *          [i-W+1, i], attention_row(q, K, V, mask_row) -> (out, weights).
 *   [LES]  "Attention Variants — Sliding Window, Sparse, Differential"
 *          (deventureacademy.com): differential attention subtracts one
 *          attention map from another.
 *
 * Where the pages are silent or disagree, the reading taken is stated at the
 * function that depends on it: the window holds W keys (j in [i-W+1, i];
 * with dilation dil, the keys i, i-dil, ..., i-(W-1)*dil), global tokens are
 * the first n_global positions and keep the causal order,
 * the stride is anchored at key 0, the ring slot of position p is p mod W,
 * query head h uses key/value head h / (Hq/Hkv), and differential attention
 * has no normalisation after the subtraction.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Mask                                                                      */
/* ------------------------------------------------------------------------ */

/* [VAR] swa_mask: row i opens keys lo..i with lo = max(0, i - window + 1);
 * a window >= n therefore gives the full causal mask ([SSW] §3 causal case
 * M_ij = 1[j <= i]).  [VAR] strided_mask: start from the window mask, then
 * also open every stride-th key counting from key 0 up to i
 * (range(0, i + 1, stride)).  stride == 0 means no stride pattern.
 * [SSW] §3b Longformer, dilation: gaps inside the window, attending every
 * dilation-th token, so the same budget of `window` keys reaches dilation
 * times further back: keys i - m*dilation for m = 0 .. window-1
 * (dilation == 1 is the plain window).  Global tokens: designated positions
 * that attend to every position and are attended to by every position; here
 * the first n_global positions, and -- this being causal attention -- only
 * pairs with j <= i: row i < n_global opens every key j <= i, and key
 * j < n_global is open to every row i >= j.  (Under the causal order the row
 * half adds nothing: the keys j <= i < n_global of a global row are all
 * global columns.  It is kept to state the definition as the page does.) */
int orc_allowed(int64_t i, int64_t j, int64_t n, int64_t window, int64_t stride,
                int64_t dilation, int64_t n_global)
{
    if (i < 0 || i >= n || j < 0 || j >= n)
        return 0;
    int64_t dist = i - j;
    if (dist >= 0 && dist % dilation == 0 && dist / dilation < window)
        return 1;
    if (stride > 0 && j <= i && j % stride == 0)
        return 1;
    if (n_global > 0 && j <= i && (j < n_global || i < n_global))
        return 1;
    return 0;
}

/* Dense 0/1 mask, row-major n x n (1 = attends).  [VAR] swa_mask/strided_mask
 * build the same matrix with 0.0 / NEG_INF entries. */
void orc_mask_dense(int64_t n, int64_t window, int64_t stride, int64_t dilation,
                    int64_t n_global, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        for (int64_t j = 0; j < n; ++j)
            out[i * n + j] = (uint8_t)orc_allowed(i, j, n, window, stride, dilation, n_global);
}

/* [VAR] count_nonmasked(M): the number of attended cells, here per row and
 * in total, by visiting every cell. */
int64_t orc_count_nonmasked(int64_t n, int64_t window, int64_t stride, int64_t dilation,
                            int64_t n_global, int64_t *row_counts)
{
    int64_t total = 0;
    for (int64_t i = 0; i < n; ++i) {
        int64_t c = 0;
        for (int64_t j = 0; j < n; ++j)
            c += orc_allowed(i, j, n, window, stride, dilation, n_global);
        if (row_counts)
            row_counts[i] = c;
        total += c;
    }
    return total;
}

/* ------------------------------------------------------------------------ */
/* Block mask (tile list)                                                    */
/* ------------------------------------------------------------------------ */

/* [VAR] create_block_mask turns the pattern into a per-block keep/skip map;
 * blocks with no attended cell are skipped.  For query tile qt (rows
 * qt*bm .. qt*bm+bm-1) and key tile kt (keys kt*bn .. kt*bn+bn-1), both
 * clipped at n, the cells of the tile are visited one by one:
 *   cells == 0                      -> tile not listed
 *   no cell is in the band part     -> kind 2 (prefix-only)
 *   cells == in-range tile area     -> kind 0 (full)
 *   otherwise                       -> kind 1 (partial)
 * The band part of a cell is j <= i with i - j <= (window-1)*dilation (the
 * span of the window).  The other attended cells are "prefix keys":
 * multiples of stride, or global columns j < n_global (which also cover the
 * keys of the global rows, see orc_allowed).
 * prefix_keys[qt] counts the prefix keys inside the prefix-only tiles of
 * query tile qt.  band_begin[qt] is the list index of the first tile of qt
 * that is not prefix-only.
 * Returns nnz, or -1 if the list would exceed cap entries. */
int64_t orc_tile_list(int64_t n, int64_t window, int64_t stride, int64_t dilation,
                      int64_t n_global, int64_t bm, int64_t bn, int32_t *row_ptr,
                      int32_t *kv_tile, uint8_t *kind, int32_t *cells, int32_t *prefix_keys,
                      int32_t *band_begin, int64_t cap)
{
    int64_t nq = (n + bm - 1) / bm, nk = (n + bn - 1) / bn, nnz = 0;
    int64_t span = (window - 1) * dilation;
    for (int64_t qt = 0; qt < nq; ++qt) {
        row_ptr[qt] = (int32_t)nnz;
        prefix_keys[qt] = 0;
        band_begin[qt] = -1;
        int64_t i0 = qt * bm, i1 = i0 + bm < n ? i0 + bm : n;
        for (int64_t kt = 0; kt < nk; ++kt) {
            int64_t j0 = kt * bn, j1 = j0 + bn < n ? j0 + bn : n;
            int64_t c = 0, band = 0;
            for (int64_t i = i0; i < i1; ++i) {
                for (int64_t j = j0; j < j1; ++j) {
                    c += orc_allowed(i, j, n, window, stride, dilation, n_global);
                    band += (j <= i && i - j <= span);
                }
            }
            if (c == 0)
                continue;
            if (nnz >= cap)
                return -1;
            uint8_t k;
            if (band == 0)
                k = 2;
            else if (c == (i1 - i0) * (j1 - j0))
                k = 0;
            else
                k = 1;
            if (k == 2) {
                for (int64_t j = j0; j < j1; ++j)
                    prefix_keys[qt] += (j < n_global || (stride > 0 && j % stride == 0));
            } else if (band_begin[qt] < 0) {
                band_begin[qt] = (int32_t)nnz;
            }
            kv_tile[nnz] = (int32_t)kt;
            kind[nnz] = k;
            cells[nnz] = (int32_t)c;
            ++nnz;
        }
        if (band_begin[qt] < 0)
            band_begin[qt] = (int32_t)nnz;
    }
    row_ptr[nq] = (int32_t)nnz;
    return nnz;
}

/* ------------------------------------------------------------------------ */
/* Attention                                                                 */
/* ------------------------------------------------------------------------ */

/* [EXP] attention_row(q, K, V, mask_row) -> (out, weights), with the score
 * scale of [SSW] §3 (1/sqrt(d_k), passed in as `scale`).  Only keys with
 * mask_row[j] != 0 take part: adding log 0 = -inf to a score gives it zero
 * weight, so the masked keys are simply left out of the softmax.
 *   s_j = scale * sum_c q[c] * K[j][c]
 *   m   = max_j s_j,  e_j = exp(s_j - m),  l = sum_j e_j
 *   w_j = e_j / l,    out[c] = sum_j w_j * V[j][c]
 * k_stride / v_stride are the element distances between consecutive keys.
 * weights (n entries, nullable) receives w_j, 0 for masked keys.
 * Returns the log-sum-exp m + log(l) of the scaled scores (-inf if no key). */
double orc_attention_row(const float *q, const float *K, const float *V, const uint8_t *mask_row,
                         int64_t n, int64_t d, int64_t dv, int64_t k_stride, int64_t v_stride,
                         double scale, double *out, double *weights)
{
    double *s = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    double m = -INFINITY;
    for (int64_t j = 0; j < n; ++j) {
        if (!mask_row[j])
            continue;
        double acc = 0.0;
        for (int64_t c = 0; c < d; ++c)
            acc += (double)q[c] * (double)K[j * k_stride + c];
        s[j] = scale * acc;
        if (s[j] > m)
            m = s[j];
    }
    double l = 0.0;
    for (int64_t j = 0; j < n; ++j)
        if (mask_row[j]) {
            s[j] = exp(s[j] - m);
            l += s[j];
        }
    for (int64_t c = 0; c < dv; ++c)
        out[c] = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        double w = mask_row[j] ? s[j] / l : 0.0;
        if (weights)
            weights[j] = w;
        if (!mask_row[j])
            continue;
        for (int64_t c = 0; c < dv; ++c)
            out[c] += w * (double)V[j * v_stride + c];
    }
    free(s);
    return l > 0.0 ? m + log(l) : -INFINITY;
}

/* [VAR] "Flash style softmax" tiled_softmax_dot(q, Ks, Vs, tile): the same
 * softmax-weighted sum, visiting the keys in tiles of `tile` and keeping a
 * running maximum m, running denominator l and running weighted sum acc.
 * For each tile: m' = max(m, max of the tile's scores);
 * alpha = exp(m - m') (0 while m is still -inf); acc = alpha*acc + sum
 * exp(s_j - m') v_j; l = alpha*l + sum exp(s_j - m').  Result acc / l.
 * Keys run 0..n-1, all attended (the cheatsheet applies it to one row). */
void orc_tiled_softmax_dot(const float *q, const float *K, const float *V, int64_t n,
                           int64_t d, int64_t dv, int64_t tile, double scale, double *out)
{
    double m = -INFINITY, l = 0.0;
    double *acc = (double *)calloc((size_t)dv, sizeof(double));
    double *s = (double *)malloc(sizeof(double) * (size_t)(tile > 0 ? tile : 1));
    for (int64_t t0 = 0; t0 < n; t0 += tile) {
        int64_t t1 = t0 + tile < n ? t0 + tile : n;
        double tmax = -INFINITY;
        for (int64_t j = t0; j < t1; ++j) {
            double a = 0.0;
            for (int64_t c = 0; c < d; ++c)
                a += (double)q[c] * (double)K[j * d + c];
            s[j - t0] = scale * a;
            if (s[j - t0] > tmax)
                tmax = s[j - t0];
        }
        double m_new = m > tmax ? m : tmax;
        double alpha = (m == -INFINITY) ? 0.0 : exp(m - m_new);
        l *= alpha;
        for (int64_t c = 0; c < dv; ++c)
            acc[c] *= alpha;
        for (int64_t j = t0; j < t1; ++j) {
            double e = exp(s[j - t0] - m_new);
            l += e;
            for (int64_t c = 0; c < dv; ++c)
                acc[c] += e * (double)V[j * dv + c];
        }
        m = m_new;
    }
    for (int64_t c = 0; c < dv; ++c)
        out[c] = acc[c] / l;
    free(acc);
    free(s);
}

/* Masked attention over [B, Hq, N, d] queries and [B, Hkv, N, d] / [B, Hkv,
 * N, dv] keys and values, for a list of rows.  Row r is the flat index
 * (b*Hq + h)*N + i.  [SSW] §3 equation per row, with the mask of
 * orc_allowed.  Query heads share key/value heads in contiguous groups of
 * G = Hq/Hkv (grouped-query attention): head h reads key/value head h/G.
 * out is [nrows, dv]; lse (nullable) is [nrows]. */
void orc_attn_rows(const float *q, const float *k, const float *v, int64_t B, int64_t Hq,
                   int64_t Hkv, int64_t N, int64_t d, int64_t dv, int64_t window,
                   int64_t stride, int64_t dilation, int64_t n_global, double scale,
                   const int64_t *rows, int64_t nrows, double *out, double *lse)
{
    int64_t G = Hq / Hkv;
    uint8_t *mrow = (uint8_t *)malloc((size_t)(N > 0 ? N : 1));
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t flat = rows[r];
        if (flat < 0 || flat >= B * Hq * N) { /* not a row of this problem */
            for (int64_t c = 0; c < dv; ++c)
                out[r * dv + c] = NAN;
            if (lse)
                lse[r] = NAN;
            continue;
        }
        int64_t i = flat % N, bh = flat / N, h = bh % Hq, b = bh / Hq, g = h / G;
        for (int64_t j = 0; j < N; ++j)
            mrow[j] = (uint8_t)orc_allowed(i, j, N, window, stride, dilation, n_global);
        const float *qi = q + ((b * Hq + h) * N + i) * d;
        const float *kg = k + (b * Hkv + g) * N * d;
        const float *vg = v + (b * Hkv + g) * N * dv;
        double x = orc_attention_row(qi, kg, vg, mrow, N, d, dv, d, dv, scale, out + r * dv, NULL);
        if (lse)
            lse[r] = x;
    }
    free(mrow);
}

/* All rows of orc_attn_rows; out is [B, Hq, N, dv]. */
void orc_attn_full(const float *q, const float *k, const float *v, int64_t B, int64_t Hq,
                   int64_t Hkv, int64_t N, int64_t d, int64_t dv, int64_t window, int64_t stride,
                   int64_t dilation, int64_t n_global, double scale, double *out, double *lse)
{
    int64_t total = B * Hq * N;
    int64_t *rows = (int64_t *)malloc(sizeof(int64_t) * (size_t)(total > 0 ? total : 1));
    for (int64_t r = 0; r < total; ++r)
        rows[r] = r;
    orc_attn_rows(q, k, v, B, Hq, Hkv, N, d, dv, window, stride, dilation, n_global, scale, rows,
                  total, out, lse);
    free(rows);
}

/* Differential attention.  [LES] and [VAR]: two attention maps from separate
 * query/key pairs over the same values, the second subtracted from the first
 * with weight lambda:
 *   out_i = sum_j (w1_ij - lambda * w2_ij) * v_j
 * where w1 = softmax(scale * q1 k1^T + log M)_i and w2 likewise from (q2, k2),
 * both over the same mask row.  No normalisation follows the subtraction.
 * q1, q2 are [B, Hq, N, d]; k1, k2 are [B, Hkv, N, d]; v is [B, Hkv, N, dv]. */
void orc_diff_rows(const float *q1, const float *k1, const float *q2, const float *k2,
                   const float *v, int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                   int64_t dv, int64_t window, int64_t stride, int64_t dilation,
                   int64_t n_global, double scale, double lambda, const int64_t *rows,
                   int64_t nrows, double *out)
{
    int64_t G = Hq / Hkv;
    uint8_t *mrow = (uint8_t *)malloc((size_t)(N > 0 ? N : 1));
    double *w1 = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
    double *w2 = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
    double *tmp = (double *)malloc(sizeof(double) * (size_t)(dv > 0 ? dv : 1));
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t flat = rows[r];
        if (flat < 0 || flat >= B * Hq * N) { /* not a row of this problem */
            for (int64_t c = 0; c < dv; ++c)
                out[r * dv + c] = NAN;
            continue;
        }
        int64_t i = flat % N, bh = flat / N, h = bh % Hq, b = bh / Hq, g = h / G;
        for (int64_t j = 0; j < N; ++j)
            mrow[j] = (uint8_t)orc_allowed(i, j, N, window, stride, dilation, n_global);
        const float *vg = v + (b * Hkv + g) * N * dv;
        orc_attention_row(q1 + ((b * Hq + h) * N + i) * d, k1 + (b * Hkv + g) * N * d, vg, mrow,
                          N, d, dv, d, dv, scale, tmp, w1);
        orc_attention_row(q2 + ((b * Hq + h) * N + i) * d, k2 + (b * Hkv + g) * N * d, vg, mrow,
                          N, d, dv, d, dv, scale, tmp, w2);
        double *o = out + r * dv;
        for (int64_t c = 0; c < dv; ++c)
            o[c] = 0.0;
        for (int64_t j = 0; j < N; ++j) {
            if (!mrow[j])
                continue;
            double w = w1[j] - lambda * w2[j];
            for (int64_t c = 0; c < dv; ++c)
                o[c] += w * (double)vg[j * dv + c];
        }
    }
    free(mrow);
    free(w1);
    free(w2);
    free(tmp);
}

/* ------------------------------------------------------------------------ */
/* Decode over a rolling KV window                                          */
/* ------------------------------------------------------------------------ */

/* [SSW] §4 and §6: decoding keeps only the most recent `window` tokens' keys
 * and values in a fixed-size rolling buffer, evicting the oldest.  Sequence b
 * has seq_len[b] = L tokens so far, the current one included (its key and
 * value already written).  Position p lives in ring slot p mod window, and
 * the attended positions are max(0, L - window) .. L - 1 -- the window of
 * the current query row L-1 under [VAR] swa_mask.
 * With n_sink > 0 the cache also keeps the first n_sink positions in their
 * own slots (sink slot p for p < n_sink; [SSW] §4 StreamingLLM keeps the
 * first k tokens plus the recent window); a position held by both is
 * attended once, from the ring.
 * q: [B, Hq, d]; k_ring, v_ring: [B, Hkv, window, d|dv];
 * k_sink, v_sink: [B, Hkv, n_sink, d|dv] (unused when n_sink == 0);
 * out: [B, Hq, dv]; lse (nullable): [B, Hq]. */
void orc_decode(const float *q, const float *k_ring, const float *v_ring, const float *k_sink,
                const float *v_sink, const int64_t *seq_len, int64_t B, int64_t Hq, int64_t Hkv,
                int64_t window, int64_t n_sink, int64_t d, int64_t dv, double scale, double *out,
                double *lse)
{
    int64_t G = Hq / Hkv;
    int64_t cap = window + n_sink;
    float *K = (float *)malloc(sizeof(float) * (size_t)(cap * d > 0 ? cap * d : 1));
    float *V = (float *)malloc(sizeof(float) * (size_t)(cap * dv > 0 ? cap * dv : 1));
    uint8_t *ones = (uint8_t *)malloc((size_t)(cap > 0 ? cap : 1));
    memset(ones, 1, (size_t)(cap > 0 ? cap : 1));
    for (int64_t b = 0; b < B; ++b) {
        int64_t L = seq_len[b];
        int64_t first = L - window > 0 ? L - window : 0;
        for (int64_t h = 0; h < Hq; ++h) {
            int64_t g = h / G, n = 0;
            /* gather attended positions in ascending position order */
            for (int64_t p = 0; p < n_sink && p < first; ++p, ++n) {
                memcpy(K + n * d, k_sink + ((b * Hkv + g) * n_sink + p) * d, sizeof(float) * (size_t)d);
                memcpy(V + n * dv, v_sink + ((b * Hkv + g) * n_sink + p) * dv, sizeof(float) * (size_t)dv);
            }
            for (int64_t p = first; p < L; ++p, ++n) {
                int64_t slot = p % window;
                memcpy(K + n * d, k_ring + ((b * Hkv + g) * window + slot) * d, sizeof(float) * (size_t)d);
                memcpy(V + n * dv, v_ring + ((b * Hkv + g) * window + slot) * dv, sizeof(float) * (size_t)dv);
            }
            double x = orc_attention_row(q + (b * Hq + h) * d, K, V, ones, n, d, dv, d, dv, scale,
                                         out + (b * Hq + h) * dv, NULL);
            if (lse)
                lse[b * Hq + h] = x;
        }
    }
    free(K);
    free(V);
    free(ones);
}

/* ------------------------------------------------------------------------ */
/* Counting helpers                                                          */
/* ------------------------------------------------------------------------ */

/* [VAR] count_nsa(N, l, k, W): keys one query of native sparse attention
 * reads -- N/l compressed block keys, k selected blocks of l keys, and a
 * window of W -- with no de-duplication between the three branches. */
int64_t orc_count_nsa(int64_t n, int64_t l, int64_t k, int64_t w)
{
    return n / l + k * l + w;
}

/* [VAR] task table, "KV cache bytes": kv_cache_bytes(N, n_layers, n_heads_kv,
 * d_head, dtype=2) -- the bytes that keep one key and one value vector of
 * d_head elements for each of N positions, key/value heads and layers, at
 * dtype bytes per element.  [EXP] "Quantifying Memory Impact with KV-Cache
 * Calculations" computes the same quantity from layers, KV heads, head
 * dimension and sequence length (in another argument order; the task
 * table's is kept here).  [SSW] §6 "FLOPs & memory" states the position
 * counts it is taken at: all s positions for dense decode, the last w for a
 * rolling window, k sinks plus w for StreamingLLM. */
int64_t orc_kv_cache_bytes(int64_t n, int64_t n_layers, int64_t n_heads_kv, int64_t d_head,
                           int64_t dtype_bytes)
{
    const int64_t per_tensor = n * n_layers * n_heads_kv * d_head * dtype_bytes;
    return 2 * per_tensor;   /* K and V */
}
