/*
 * attn_oracle.c -- plain fp64 CPU reference for exact softmax attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg load this library.  It shares no code with the GPU library.
 *
 * What it computes (page "Attention Kernel", section "问题与成本", the
 * definition P = softmax(QK^T/sqrt(d_h) + M), O = PV):
 *
 *   s_ij  = scale * sum_e q_ie k_je + M_ij   (M_ij finite or -inf)
 *   m_i   = max_j s_ij
 *   l_i   = sum_j exp(s_ij - m_i)                 (safe softmax, page
 *                                                  "Attention 算子加速史", 1.2)
 *   P_ij  = exp(s_ij - m_i) / l_i
 *   O_i   = sum_j P_ij v_j
 *   LSE_i = m_i + ln l_i                          (natural log)
 *
 * Every row's score vector S_i and probability vector P_i are materialised in
 * full, exactly as the standard (non-fused) attention does (page
 * "Attention 算子加速史", 1.1, steps 1-3).  Arithmetic is fp64 throughout; the
 * inputs (fp32 values or bf16 bits) are widened exactly.
 *
 * M_ij is the sum of an optional dense additive term bias[i][j] (dense
 * prefill only: any finite value or -inf, e.g. a relative-position bias, or
 * 0 / -inf for an arbitrary pattern -- page "Attention Kernel", section
 * "可编程 mask", general dense M) and of -inf when any of:
 *   - causal and j > i + (S_k - S_q)   (query i sits at absolute position
 *                                       S_k - S_q + i: bottom-right alignment)
 *   - q_keep[i] == 0  or  k_keep[j] == 0
 *   - m_keep[i][j] == 0  (a dense keep matrix per batch row, dense prefill
 *     and its gradient only: any element rule -- sliding window, document
 *     boundaries -- is handed to the oracle in this form, built from the
 *     rule's definition; page "Attention Kernel", section "可编程 mask")
 *   - block_keep[i / 128][j / 128] == 0  (block sparsity: one flag per
 *     128 x 128 block of (row, key) pairs, per batch row and either shared by
 *     the heads or one per head; same section, the block level of a mask)
 *   - j lies outside i's sequence (packed varlen), or outside a sliding
 *     window i - left <= j <= i + right around the query's position (packed
 *     varlen gradient and paged prefill; -1 leaves a side unbounded)
 * A finite additive term below -FLT_MAX * min(scale, ln 2) is a masking fill
 * value (the float32 minimum is the usual one): it counts as -inf.  Such a
 * term cannot be represented once the score is scaled to base 2 in fp32, and
 * this is the reading taken of a mask given with a finite fill value.
 * A row whose scores are all -inf (including S_k == 0) returns O = 0 and
 * LSE = -inf (page "Attention Kernel", section "Online softmax": a fully
 * masked row must yield an agreed zero output, never NaN).
 *
 * GQA: query head h reads KV head h / (A / A_kv) (contiguous groups; page
 * "Attention Kernel", section "问题与成本", GQA paragraph).
 *
 * Paged decode: logical token t of sequence b lives in physical page
 * block_table[b][t / page_size] at offset t % page_size (page "Attention
 * Kernel", section "Paged 与 ragged KV").
 *
 * Paged prefill (oracle_prefill_paged): the new query chunk of sequence s is
 * the last q_s of its seq_lens[s] cached tokens, so chunk row i sits at
 * position seq_lens[s] - q_s + i and sees cached tokens by that position
 * (causal, windows); keys are gathered through the block table as for decode
 * (page "Attention 算子加速史", section 4.2: prefill chunks and decode rows in
 * one batch over the paged cache).
 *
 * Block mask of a bias (oracle_block_keep_of_bias): flag (qb, kb) is 1 when
 * some entry of the 128 x 128 block (clipped to S_q x S_k) exceeds -inf.
 *
 * Gradient (oracle_attn_bwd): the exact derivative of the batched prefill
 * above with respect to q, k and v, for an incoming output gradient dO.  The
 * probabilities are recomputed from Q and K, as the backward pass of page
 * "Attention 算子加速史" (FAQ Q1) and page "Attention Kernel" (section
 * "Backward 与重计算") describe; the chain rule through O = P V,
 * P = softmax(S), S = scale Q K^T + M, row by row:
 *
 *   dV_j  += P_ij dO_i
 *   dP_ij  = dO_i . v_j
 *   D_i    = sum_j P_ij dP_ij
 *   dS_ij  = P_ij (dP_ij - D_i)
 *   dQ_i   = scale * sum_j dS_ij k_j
 *   dK_j  += scale * dS_ij q_i
 *
 * Masked entries (P_ij = 0) pass no gradient; a fully masked row has dQ_i = 0.
 * Under GQA, dK and dV of a KV head sum over the query heads that read it.
 *
 * Return value: 0 on success, -1 on invalid arguments.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* element types of the inputs; OR_F64 exists for the finite-difference pins
 * of the gradient, which need inputs perturbed below fp32 resolution */
enum { OR_F32 = 0, OR_BF16 = 1, OR_F64 = 2 };

static int dt_ok(int dt) { return dt == OR_F32 || dt == OR_BF16 || dt == OR_F64; }

static double ld(const void *p, int64_t idx, int dt)
{
    if (dt == OR_F64)
        return ((const double *)p)[idx];
    if (dt == OR_F32)
        return (double)((const float *)p)[idx];
    uint32_t u = (uint32_t)((const uint16_t *)p)[idx] << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* finite additive terms below this count as -inf (see the header) */
static double fill_limit(double scale)
{
    const double flt_max = 3.4028234663852886e38, ln2 = 0.69314718055994530942;
    return -flt_max * (scale < ln2 ? scale : ln2);
}

/* block flag of (row i, key j): nonzero = kept; NULL mask = every block kept */
static int block_kept(const uint8_t *block_keep, int block_heads, int b, int h, int S_q, int S_k, int i, int j)
{
    if (!block_keep)
        return 1;
    int64_t nqb = (S_q + 127) / 128, nkb = (S_k + 127) / 128;
    int hm = block_heads == 1 ? 0 : h;
    return block_keep[(((int64_t)b * block_heads + hm) * nqb + i / 128) * nkb + j / 128] != 0;
}

/*
 * One query row against n key/value rows.
 * q_off: element offset of the query row; kv_off[j]: element offset of key j's
 * row in k and of its value row in v; vis[j]: 1 where M_ij = 0, 0 where -inf.
 * s, p: scratch of n doubles (the materialised score and probability rows).
 */
static void attend_row(const void *q, int64_t q_off, const void *k, const void *v, int dt,
                       const int64_t *kv_off, const unsigned char *vis, const float *bias_row,
                       int64_t n, int d, double scale, double *s, double *p, double *o, double *lse)
{
    double m = -INFINITY;
    for (int64_t j = 0; j < n; ++j) {
        if (!vis[j]) {
            s[j] = -INFINITY;
        } else {
            double dot = 0.0;
            for (int e = 0; e < d; ++e)
                dot += ld(q, q_off + e, dt) * ld(k, kv_off[j] + e, dt);
            s[j] = scale * dot;
            if (bias_row) {
                if ((double)bias_row[j] < fill_limit(scale))
                    s[j] = -INFINITY;
                else
                    s[j] += (double)bias_row[j];
            }
        }
        if (s[j] > m)
            m = s[j];
    }
    if (m == -INFINITY) {
        for (int e = 0; e < d; ++e)
            o[e] = 0.0;
        *lse = -INFINITY;
        return;
    }
    double l = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        p[j] = (s[j] == -INFINITY) ? 0.0 : exp(s[j] - m);
        l += p[j];
    }
    for (int64_t j = 0; j < n; ++j)
        p[j] /= l;
    for (int e = 0; e < d; ++e) {
        double acc = 0.0;
        for (int64_t j = 0; j < n; ++j)
            if (p[j] != 0.0)
                acc += p[j] * ld(v, kv_off[j] + e, dt);
        o[e] = acc;
    }
    *lse = m + log(l);
}

struct scratch {
    int64_t *off;
    unsigned char *vis;
    double *s, *p;
};

static int scratch_alloc(struct scratch *w, int64_t n)
{
    size_t m = (size_t)(n > 0 ? n : 1);
    w->off = malloc(m * sizeof *w->off);
    w->vis = malloc(m);
    w->s = malloc(m * sizeof *w->s);
    w->p = malloc(m * sizeof *w->p);
    return (w->off && w->vis && w->s && w->p) ? 0 : -1;
}

static void scratch_free(struct scratch *w)
{
    free(w->off);
    free(w->vis);
    free(w->s);
    free(w->p);
}

/*
 * Batched prefill.  q, o: [B, A, S_q, d]; k, v: [B, A_kv, S_k, d];
 * q_keep: [B, S_q] or NULL; k_keep: [B, S_k] or NULL; m_keep: [B, S_q, S_k]
 * or NULL (shared by every head); bias: [B, bias_heads, S_q, S_k] fp32 or
 * NULL, bias_heads 1 (shared by every head) or A; block_keep:
 * [B, block_heads, ceil(S_q / 128), ceil(S_k / 128)] or NULL, block_heads 1
 * or A.
 * rows: flattened row ids (b*A + h)*S_q + i to compute, or NULL for all rows
 * in order.  o receives [n_rows, d] doubles, lse [n_rows].
 */
int oracle_attn_fwd(const void *q, const void *k, const void *v, int dt,
                    int B, int A, int A_kv, int S_q, int S_k, int d, float scale, int causal,
                    const uint8_t *q_keep, const uint8_t *k_keep, const uint8_t *m_keep,
                    const float *bias, int bias_heads, const uint8_t *block_keep, int block_heads,
                    const int64_t *rows, int64_t n_rows, double *o, double *lse)
{
    if (B <= 0 || A <= 0 || A_kv <= 0 || S_q < 0 || S_k < 0 || d <= 0 || A % A_kv != 0)
        return -1;
    if (bias && bias_heads != 1 && bias_heads != A)
        return -1;
    if (block_keep && block_heads != 1 && block_heads != A)
        return -1;
    if (!dt_ok(dt))
        return -1;
    int64_t total = (int64_t)B * A * S_q;
    if (rows == NULL)
        n_rows = total;
    const int G = A / A_kv;
    int err = 0;
#pragma omp parallel
    {
        struct scratch w;
        int bad = scratch_alloc(&w, S_k);
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < n_rows; ++r) {
            if (bad)
                continue;
            int64_t id = rows ? rows[r] : r;
            if (id < 0 || id >= total) {
                bad = 1;
                continue;
            }
            int i = (int)(id % S_q);
            int64_t bh = id / S_q;
            int h = (int)(bh % A), b = (int)(bh / A);
            int hk = h / G;
            int64_t kv_base = (((int64_t)b * A_kv + hk) * S_k) * d;
            int row_masked = q_keep && !q_keep[(int64_t)b * S_q + i];
            for (int j = 0; j < S_k; ++j) {
                w.off[j] = kv_base + (int64_t)j * d;
                int visible = !row_masked;
                if (causal && (int64_t)j > (int64_t)i + (S_k - S_q))
                    visible = 0;
                if (k_keep && !k_keep[(int64_t)b * S_k + j])
                    visible = 0;
                if (m_keep && !m_keep[((int64_t)b * S_q + i) * S_k + j])
                    visible = 0;
                if (!block_kept(block_keep, block_heads, b, h, S_q, S_k, i, j))
                    visible = 0;
                w.vis[j] = (unsigned char)visible;
            }
            const float *bias_row =
                bias ? bias + (((int64_t)b * bias_heads + (bias_heads == 1 ? 0 : h)) * S_q + i) * S_k : NULL;
            attend_row(q, id * d, k, v, dt, w.off, w.vis, bias_row, S_k, d, (double)scale, w.s, w.p,
                       o + r * d, lse + r);
        }
        if (bad) {
#pragma omp atomic write
            err = 1;
        }
        scratch_free(&w);
    }
    return err ? -1 : 0;
}

/*
 * Gradient of the batched prefill (see the header).  do_ has q's layout and
 * element type.  dq: [B, A, S_q, d]; dk, dv: [B, A_kv, S_k, d]; all doubles,
 * fully written.  One thread owns one (batch, KV head) and every query row
 * that reads it, so the dK / dV sums need no synchronisation.
 */
int oracle_attn_bwd(const void *q, const void *k, const void *v, const void *do_, int dt,
                    int B, int A, int A_kv, int S_q, int S_k, int d, float scale, int causal,
                    const uint8_t *q_keep, const uint8_t *k_keep, const uint8_t *m_keep,
                    const float *bias, int bias_heads, const uint8_t *block_keep, int block_heads,
                    double *dq, double *dk, double *dv)
{
    if (B <= 0 || A <= 0 || A_kv <= 0 || S_q < 0 || S_k < 0 || d <= 0 || A % A_kv != 0)
        return -1;
    if (bias && bias_heads != 1 && bias_heads != A)
        return -1;
    if (block_keep && block_heads != 1 && block_heads != A)
        return -1;
    if (!dt_ok(dt))
        return -1;
    const int G = A / A_kv;
    const double sc = (double)scale;
    int err = 0;
#pragma omp parallel
    {
        struct scratch w;
        int bad = scratch_alloc(&w, S_k);
        double *dp = malloc((size_t)(S_k > 0 ? S_k : 1) * sizeof *dp);
        double *o = malloc((size_t)d * sizeof *o);
        if (!dp || !o)
            bad = 1;
#pragma omp for schedule(dynamic, 1)
        for (int64_t bk = 0; bk < (int64_t)B * A_kv; ++bk) {
            int b = (int)(bk / A_kv), hk = (int)(bk % A_kv);
            int64_t kv_base = bk * S_k * (int64_t)d;
            double *dkg = dk + kv_base, *dvg = dv + kv_base;
            for (int64_t x = 0; x < (int64_t)S_k * d; ++x)
                dkg[x] = dvg[x] = 0.0;
            if (bad)
                continue;
            for (int g = 0; g < G; ++g) {
                int h = hk * G + g;
                for (int i = 0; i < S_q; ++i) {
                    int64_t id = ((int64_t)b * A + h) * S_q + i;
                    double *dqi = dq + id * d;
                    for (int e = 0; e < d; ++e)
                        dqi[e] = 0.0;
                    int row_masked = q_keep && !q_keep[(int64_t)b * S_q + i];
                    for (int j = 0; j < S_k; ++j) {
                        w.off[j] = kv_base + (int64_t)j * d;
                        int visible = !row_masked;
                        if (causal && (int64_t)j > (int64_t)i + (S_k - S_q))
                            visible = 0;
                        if (k_keep && !k_keep[(int64_t)b * S_k + j])
                            visible = 0;
                        if (m_keep && !m_keep[((int64_t)b * S_q + i) * S_k + j])
                            visible = 0;
                        if (!block_kept(block_keep, block_heads, b, h, S_q, S_k, i, j))
                            visible = 0;
                        w.vis[j] = (unsigned char)visible;
                    }
                    const float *bias_row =
                        bias ? bias + (((int64_t)b * bias_heads + (bias_heads == 1 ? 0 : h)) * S_q + i) * S_k
                             : NULL;
                    double lse;
                    attend_row(q, id * d, k, v, dt, w.off, w.vis, bias_row, S_k, d, sc, w.s, w.p, o, &lse);
                    if (lse == -INFINITY)
                        continue;  /* fully masked row: no gradient anywhere */
                    double D = 0.0;
                    for (int j = 0; j < S_k; ++j) {
                        if (!w.vis[j] || w.p[j] == 0.0) {
                            dp[j] = 0.0;
                            continue;
                        }
                        double acc = 0.0;
                        for (int e = 0; e < d; ++e)
                            acc += ld(do_, id * d + e, dt) * ld(v, w.off[j] + e, dt);
                        dp[j] = acc;
                        D += w.p[j] * acc;
                    }
                    for (int j = 0; j < S_k; ++j) {
                        if (!w.vis[j] || w.p[j] == 0.0)
                            continue;
                        double ds = w.p[j] * (dp[j] - D);
                        for (int e = 0; e < d; ++e) {
                            dqi[e] += sc * ds * ld(k, w.off[j] + e, dt);
                            dkg[(int64_t)j * d + e] += sc * ds * ld(q, id * d + e, dt);
                            dvg[(int64_t)j * d + e] += w.p[j] * ld(do_, id * d + e, dt);
                        }
                    }
                }
            }
        }
        if (bad) {
#pragma omp atomic write
            err = 1;
        }
        free(dp);
        free(o);
        scratch_free(&w);
    }
    return err ? -1 : 0;
}

/*
 * Packed varlen prefill.  q, o: [A, T, d]; k, v: [A_kv, T, d];
 * cu_seqlens: [n_seq + 1], non-decreasing, cu[0] = 0, cu[n_seq] = T.
 * Query t of sequence s sees keys of the same sequence only; causal compares
 * positions within the sequence.  q_keep, k_keep: [T] or NULL.
 * rows: flattened ids h*T + t, or NULL for all.
 */
int oracle_attn_fwd_varlen(const void *q, const void *k, const void *v, int dt,
                           const int32_t *cu, int n_seq, int T, int A, int A_kv, int d,
                           float scale, int causal, const uint8_t *q_keep, const uint8_t *k_keep,
                           const int64_t *rows, int64_t n_rows, double *o, double *lse)
{
    if (n_seq < 0 || T < 0 || A <= 0 || A_kv <= 0 || d <= 0 || A % A_kv != 0 || !cu)
        return -1;
    if (!dt_ok(dt))
        return -1;
    if (cu[0] != 0 || cu[n_seq] != T)
        return -1;
    for (int s = 0; s < n_seq; ++s)
        if (cu[s + 1] < cu[s])
            return -1;
    int64_t total = (int64_t)A * T;
    if (rows == NULL)
        n_rows = total;
    const int G = A / A_kv;
    int64_t maxlen = 0;
    for (int s = 0; s < n_seq; ++s)
        if (cu[s + 1] - cu[s] > maxlen)
            maxlen = cu[s + 1] - cu[s];
    int err = 0;
#pragma omp parallel
    {
        struct scratch w;
        int bad = scratch_alloc(&w, maxlen);
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < n_rows; ++r) {
            if (bad)
                continue;
            int64_t id = rows ? rows[r] : r;
            if (id < 0 || id >= total) {
                bad = 1;
                continue;
            }
            int t = (int)(id % T), h = (int)(id / T);
            int s = 0;
            while (!(cu[s] <= t && t < cu[s + 1]))
                ++s;
            int start = cu[s], len = cu[s + 1] - cu[s];
            int i = t - start;
            int64_t kv_base = ((int64_t)(h / G) * T + start) * d;
            int row_masked = q_keep && !q_keep[t];
            /* keys outside the sequence carry M = -inf and contribute exactly
               zero, so only the sequence's own keys are listed */
            for (int j = 0; j < len; ++j) {
                w.off[j] = kv_base + (int64_t)j * d;
                int visible = !row_masked;
                if (causal && j > i)
                    visible = 0;
                if (k_keep && !k_keep[start + j])
                    visible = 0;
                w.vis[j] = (unsigned char)visible;
            }
            attend_row(q, id * d, k, v, dt, w.off, w.vis, NULL, len, d, (double)scale, w.s, w.p,
                       o + r * d, lse + r);
        }
        if (bad) {
#pragma omp atomic write
            err = 1;
        }
        scratch_free(&w);
    }
    return err ? -1 : 0;
}

/*
 * Single-query decode over a paged KV cache.  q, o: [B, A, d];
 * k_cache, v_cache: [num_pages, page_size, A_kv, d];
 * block_table: [B, max_pages]; seq_lens: [B].
 * The query of sequence b sits at position seq_lens[b] - 1 (it is the last
 * token).  win_left >= 0 is a sliding window ("Attention Kernel", section
 * 可编程 mask): key t is visible when t >= seq_lens[b] - 1 - win_left;
 * win_left = -1 leaves every key visible.
 * rows: flattened ids b*A + h, or NULL for all.
 */
int oracle_decode_paged(const void *q, const void *k_cache, const void *v_cache, int dt,
                        const int32_t *block_table, const int32_t *seq_lens,
                        int B, int A, int A_kv, int d, int page_size, int max_pages,
                        int num_pages, float scale, int win_left,
                        const int64_t *rows, int64_t n_rows, double *o, double *lse)
{
    if (B <= 0 || A <= 0 || A_kv <= 0 || d <= 0 || A % A_kv != 0 || page_size <= 0 ||
        max_pages < 0 || num_pages < 0 || win_left < -1)
        return -1;
    if (!dt_ok(dt))
        return -1;
    int64_t maxlen = 0;
    for (int b = 0; b < B; ++b) {
        if (seq_lens[b] < 0 || (int64_t)seq_lens[b] > (int64_t)max_pages * page_size)
            return -1;
        for (int64_t t = 0; t < seq_lens[b]; t += page_size) {
            int32_t pg = block_table[(int64_t)b * max_pages + t / page_size];
            if (pg < 0 || pg >= num_pages)
                return -1;
        }
        if (seq_lens[b] > maxlen)
            maxlen = seq_lens[b];
    }
    int64_t total = (int64_t)B * A;
    if (rows == NULL)
        n_rows = total;
    const int G = A / A_kv;
    int err = 0;
#pragma omp parallel
    {
        struct scratch w;
        int bad = scratch_alloc(&w, maxlen);
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < n_rows; ++r) {
            if (bad)
                continue;
            int64_t id = rows ? rows[r] : r;
            if (id < 0 || id >= total) {
                bad = 1;
                continue;
            }
            int h = (int)(id % A), b = (int)(id / A);
            int hk = h / G;
            int n = seq_lens[b];
            for (int t = 0; t < n; ++t) {
                int64_t page = block_table[(int64_t)b * max_pages + t / page_size];
                int off = t % page_size;
                w.off[t] = ((page * page_size + off) * A_kv + hk) * (int64_t)d;
                w.vis[t] = win_left < 0 || (int64_t)t >= (int64_t)n - 1 - win_left;
            }
            attend_row(q, id * d, k_cache, v_cache, dt, w.off, w.vis, NULL, n, d, (double)scale,
                       w.s, w.p, o + r * d, lse + r);
        }
        if (bad) {
#pragma omp atomic write
            err = 1;
        }
        scratch_free(&w);
    }
    return err ? -1 : 0;
}

/*
 * Gradient of the packed varlen prefill.  q, do_: [A, T, d]; k, v: [A_kv, T,
 * d]; cu: [n_seq + 1]; q_keep, k_keep: [T] or NULL; a sliding window of
 * win_left / win_right keys around each query's position within its
 * sequence (-1 = unbounded).  dq: [A, T, d]; dk, dv: [A_kv, T, d]; fully
 * written.  Each sequence is an independent problem: one thread owns one
 * (KV head, sequence) and every query row of the group that reads it.
 */
int oracle_attn_bwd_varlen(const void *q, const void *k, const void *v, const void *do_, int dt,
                           const int32_t *cu, int n_seq, int T, int A, int A_kv, int d, float scale,
                           int causal, const uint8_t *q_keep, const uint8_t *k_keep, int win_left,
                           int win_right, double *dq, double *dk, double *dv)
{
    if (n_seq < 0 || T < 0 || A <= 0 || A_kv <= 0 || d <= 0 || A % A_kv != 0 || !cu)
        return -1;
    if (!dt_ok(dt) || win_left < -1 || win_right < -1)
        return -1;
    if (cu[0] != 0 || cu[n_seq] != T)
        return -1;
    int64_t maxlen = 0;
    for (int s = 0; s < n_seq; ++s) {
        if (cu[s + 1] < cu[s])
            return -1;
        if (cu[s + 1] - cu[s] > maxlen)
            maxlen = cu[s + 1] - cu[s];
    }
    const int G = A / A_kv;
    const double sc = (double)scale;
    for (int64_t x = 0; x < (int64_t)A * T * d; ++x)
        dq[x] = 0.0;
    for (int64_t x = 0; x < (int64_t)A_kv * T * d; ++x)
        dk[x] = dv[x] = 0.0;
    int err = 0;
#pragma omp parallel
    {
        struct scratch w;
        int bad = scratch_alloc(&w, maxlen);
        double *dp = malloc((size_t)(maxlen > 0 ? maxlen : 1) * sizeof *dp);
        double *o = malloc((size_t)d * sizeof *o);
        if (!dp || !o)
            bad = 1;
#pragma omp for schedule(dynamic, 1)
        for (int64_t ks = 0; ks < (int64_t)A_kv * n_seq; ++ks) {
            if (bad)
                continue;
            int hk = (int)(ks / n_seq), s = (int)(ks % n_seq);
            int start = cu[s], len = cu[s + 1] - cu[s];
            int64_t kv_base = ((int64_t)hk * T + start) * d;
            double *dkg = dk + kv_base, *dvg = dv + kv_base;
            for (int g = 0; g < G; ++g) {
                int h = hk * G + g;
                for (int i = 0; i < len; ++i) {
                    int64_t id = (int64_t)h * T + start + i;
                    double *dqi = dq + id * d;
                    int row_masked = q_keep && !q_keep[start + i];
                    for (int j = 0; j < len; ++j) {
                        w.off[j] = kv_base + (int64_t)j * d;
                        int visible = !row_masked;
                        if (causal && j > i)
                            visible = 0;
                        if (win_left >= 0 && j < i - win_left)
                            visible = 0;
                        if (win_right >= 0 && j > i + win_right)
                            visible = 0;
                        if (k_keep && !k_keep[start + j])
                            visible = 0;
                        w.vis[j] = (unsigned char)visible;
                    }
                    double lse;
                    attend_row(q, id * d, k, v, dt, w.off, w.vis, NULL, len, d, sc, w.s, w.p, o, &lse);
                    if (lse == -INFINITY)
                        continue;  /* fully masked row: no gradient anywhere */
                    double D = 0.0;
                    for (int j = 0; j < len; ++j) {
                        if (!w.vis[j] || w.p[j] == 0.0) {
                            dp[j] = 0.0;
                            continue;
                        }
                        double acc = 0.0;
                        for (int e = 0; e < d; ++e)
                            acc += ld(do_, id * d + e, dt) * ld(v, w.off[j] + e, dt);
                        dp[j] = acc;
                        D += w.p[j] * acc;
                    }
                    for (int j = 0; j < len; ++j) {
                        if (!w.vis[j] || w.p[j] == 0.0)
                            continue;
                        double ds = w.p[j] * (dp[j] - D);
                        for (int e = 0; e < d; ++e) {
                            dqi[e] += sc * ds * ld(k, w.off[j] + e, dt);
                            dkg[(int64_t)j * d + e] += sc * ds * ld(q, id * d + e, dt);
                            dvg[(int64_t)j * d + e] += w.p[j] * ld(do_, id * d + e, dt);
                        }
                    }
                }
            }
        }
        if (bad) {
#pragma omp atomic write
            err = 1;
        }
        free(dp);
        free(o);
        scratch_free(&w);
    }
    return err ? -1 : 0;
}

/*
 * Prefill of query chunks over a paged KV cache.  q, o: [A, T_q, d] packed
 * chunks, chunk s = rows [cu_q[s], cu_q[s+1]); k_cache, v_cache: [num_pages,
 * page_size, A_kv, d]; block_table: [n_seq, max_pages]; seq_lens: [n_seq],
 * each >= its chunk length.  Chunk row i of sequence s sits at position
 * p = seq_lens[s] - q_s + i and sees cached token t when (not causal or
 * t <= p) and the window p - win_left <= t <= p + win_right holds.
 * rows: flattened ids h*T_q + r, or NULL for all.
 */
int oracle_prefill_paged(const void *q, const void *k_cache, const void *v_cache, int dt,
                         const int32_t *block_table, const int32_t *seq_lens, const int32_t *cu_q,
                         int n_seq, int T_q, int A, int A_kv, int d, int page_size, int max_pages,
                         int num_pages, float scale, int causal, int win_left, int win_right,
                         const int64_t *rows, int64_t n_rows, double *o, double *lse)
{
    if (n_seq < 0 || T_q < 0 || A <= 0 || A_kv <= 0 || d <= 0 || A % A_kv != 0 || page_size <= 0 ||
        max_pages < 0 || num_pages < 0 || !cu_q)
        return -1;
    if (!dt_ok(dt) || win_left < -1 || win_right < -1)
        return -1;
    if (cu_q[0] != 0 || cu_q[n_seq] != T_q)
        return -1;
    int64_t maxlen = 0;
    for (int s = 0; s < n_seq; ++s) {
        int q_len = cu_q[s + 1] - cu_q[s];
        if (q_len < 0 || seq_lens[s] < q_len || (int64_t)seq_lens[s] > (int64_t)max_pages * page_size)
            return -1;
        for (int64_t t = 0; t < seq_lens[s]; t += page_size) {
            int32_t pg = block_table[(int64_t)s * max_pages + t / page_size];
            if (pg < 0 || pg >= num_pages)
                return -1;
        }
        if (seq_lens[s] > maxlen)
            maxlen = seq_lens[s];
    }
    int64_t total = (int64_t)A * T_q;
    if (rows == NULL)
        n_rows = total;
    const int G = A / A_kv;
    int err = 0;
#pragma omp parallel
    {
        struct scratch w;
        int bad = scratch_alloc(&w, maxlen);
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < n_rows; ++r) {
            if (bad)
                continue;
            int64_t id = rows ? rows[r] : r;
            if (id < 0 || id >= total) {
                bad = 1;
                continue;
            }
            int x = (int)(id % T_q), h = (int)(id / T_q);
            int s = 0;
            while (!(cu_q[s] <= x && x < cu_q[s + 1]))
                ++s;
            int q_len = cu_q[s + 1] - cu_q[s];
            int L = seq_lens[s];
            int pos = L - q_len + (x - cu_q[s]);
            int hk = h / G;
            for (int t = 0; t < L; ++t) {
                int64_t page = block_table[(int64_t)s * max_pages + t / page_size];
                int off = t % page_size;
                w.off[t] = ((page * page_size + off) * A_kv + hk) * (int64_t)d;
                int visible = 1;
                if (causal && t > pos)
                    visible = 0;
                if (win_left >= 0 && t < pos - win_left)
                    visible = 0;
                if (win_right >= 0 && t > pos + win_right)
                    visible = 0;
                w.vis[t] = (unsigned char)visible;
            }
            attend_row(q, id * d, k_cache, v_cache, dt, w.off, w.vis, NULL, L, d, (double)scale,
                       w.s, w.p, o + r * d, lse + r);
        }
        if (bad) {
#pragma omp atomic write
            err = 1;
        }
        scratch_free(&w);
    }
    return err ? -1 : 0;
}

/*
 * Block mask of a dense additive term.  bias: [B, H, S_q, S_k] fp32;
 * out: [B, H, ceil(S_q / 128), ceil(S_k / 128)], 1 when some entry of the
 * block (rows 128 qb .., keys 128 kb .., clipped to the matrix) is greater
 * than -inf, else 0.
 */
int oracle_block_keep_of_bias(const float *bias, int B, int H, int S_q, int S_k, uint8_t *out)
{
    if (B <= 0 || H <= 0 || S_q < 0 || S_k < 0 || !bias || !out)
        return -1;
    int64_t nqb = (S_q + 127) / 128, nkb = (S_k + 127) / 128;
    for (int64_t x = 0; x < (int64_t)B * H * nqb * nkb; ++x)
        out[x] = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < (int64_t)B * H; ++bh) {
        for (int i = 0; i < S_q; ++i) {
            const float *row = bias + (bh * S_q + i) * (int64_t)S_k;
            for (int j = 0; j < S_k; ++j)
                if (row[j] > -INFINITY)
                    out[(bh * nqb + i / 128) * nkb + j / 128] = 1;
        }
    }
    return 0;
}

/* Number of threads an OpenMP region will use (for reporting). */
int oracle_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            extern int omp_get_num_threads(void);
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}
