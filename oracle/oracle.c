/*
 * Plain fp64 CPU oracle for decode attention over a bf16 KV cache.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path links, loads or calls
 * this file: only tests/, the smoke check and the CPU-baseline leg of the
 * benchmark do. It shares no code, header, table or helper with the HIP
 * library; it is written from the definitions on the source pages, not from
 * the kernels.
 *
 * Every floating-point input arrives as raw bf16 bits (uint16_t) and is turned
 * into a double exactly (a bf16 value is the high half of an IEEE float). All
 * arithmetic after that is double precision, in the order the definition
 * states: scores for every visible cache row, their maximum, the log of the
 * sum of exponentials, then the probability-weighted sum of value rows.
 *
 * Definitions followed:
 *  - MLA in absorbed (latent) form: the score of query row q against cache row j
 *    is the dot product of [q_lat | q_rope] with [Z_j | KPE_j] and the output is
 *    softmax-weighted Z, kept in latent space ("Mla Analysis" skill page,
 *    sections "Absorption Trick (FlashMLA)" and "Tensor Shapes": Z is [B,T,K],
 *    KPE is [B,T,P]). The value is the latent part only; the rope columns take
 *    part in the scores and nothing else.
 *  - GQA/MQA/MHA: query heads are split into contiguous groups of hq/hkv heads
 *    and each group reads one shared K/V head ("Why MLA and MTP Fight Each
 *    Other", the table of attention variants in its introduction; "MQA, GQA &
 *    MLA" lesson, Concept section). kv head = query head / (hq/hkv).
 *  - Softmax attention itself is the textbook definition; the log-sum-exp is in
 *    natural-log units.
 *  - Draft tokens: row i of s query tokens sees the first L - s + i + 1 cache
 *    rows, L being the sequence length including the drafts (causal among the
 *    drafts). Rows that see nothing get output 0 and lse -inf; seqlens are
 *    clamped to [0, t_max].
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

static double bf16_bits_to_double(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static int clamp_len(int32_t len, int t_max)
{
    if (len < 0) return 0;
    if (len > t_max) return t_max;
    return (int)len;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

static void set_threads(int n_threads)
{
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
}

/*
 * Softmax over n scores held in z[0..n), in place: returns the natural-log
 * log-sum-exp and leaves z[j] = exp(z[j] - lse).
 */
static double softmax_in_place(double *z, int n)
{
    double m = -INFINITY;
    for (int j = 0; j < n; ++j)
        if (z[j] > m) m = z[j];
    double sum = 0.0;
    for (int j = 0; j < n; ++j) sum += exp(z[j] - m);
    double lse = m + log(sum);
    for (int j = 0; j < n; ++j) z[j] = exp(z[j] - lse);
    return lse;
}

/*
 * MLA absorbed decode.
 *   q_lat  [b, s, h, k], q_rope [b, s, h, p], cache [b, t_max, k + p]
 *   (latent columns first, then rope columns), seqlens [b].
 * rows: optional list of flattened row ids ((bi * s + i) * h + hh); NULL means
 * every row in order. out [n_rows, k] and lse [n_rows] are written for the
 * listed rows. *macs (if not NULL) receives the number of multiply-adds done.
 */
int oracle_mla(const uint16_t *q_lat, const uint16_t *q_rope, const uint16_t *cache,
               const int32_t *seqlens, int b, int s, int h, int k, int p, int t_max,
               double scale, const int64_t *rows, int64_t n_rows, double *out,
               double *lse, int64_t *macs, int n_threads)
{
    if (b <= 0 || s <= 0 || h <= 0 || k <= 0 || p < 0 || t_max <= 0) return 1;
    int64_t total_rows = (int64_t)b * s * h;
    if (rows == NULL) n_rows = total_rows;
    set_threads(n_threads);
    int64_t mac_total = 0;
    const int64_t cache_row = (int64_t)(k + p);

#pragma omp parallel reduction(+ : mac_total)
    {
        double *z = (double *)malloc(sizeof(double) * (size_t)t_max);
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < n_rows; ++r) {
            int64_t row = rows ? rows[r] : r;
            int hh = (int)(row % h);
            int i = (int)((row / h) % s);
            int bi = (int)(row / ((int64_t)h * s));
            int L = clamp_len(seqlens[bi], t_max);
            int n = L - s + i + 1;
            double *o = out + r * k;
            if (n <= 0) {
                for (int c = 0; c < k; ++c) o[c] = 0.0;
                lse[r] = -INFINITY;
                continue;
            }
            const uint16_t *ql = q_lat + row * k;
            const uint16_t *qr = q_rope + row * p;
            const uint16_t *zc = cache + (int64_t)bi * t_max * cache_row;
            for (int j = 0; j < n; ++j) {
                const uint16_t *cj = zc + (int64_t)j * cache_row;
                double dot = 0.0;
                for (int c = 0; c < k; ++c)
                    dot += bf16_bits_to_double(ql[c]) * bf16_bits_to_double(cj[c]);
                for (int c = 0; c < p; ++c)
                    dot += bf16_bits_to_double(qr[c]) * bf16_bits_to_double(cj[k + c]);
                z[j] = scale * dot;
            }
            lse[r] = softmax_in_place(z, n);
            for (int c = 0; c < k; ++c) o[c] = 0.0;
            for (int j = 0; j < n; ++j) {
                const uint16_t *cj = zc + (int64_t)j * cache_row;
                for (int c = 0; c < k; ++c) o[c] += z[j] * bf16_bits_to_double(cj[c]);
            }
            mac_total += (int64_t)n * (k + p) + (int64_t)n * k;
        }
        free(z);
    }
    if (macs) *macs = mac_total;
    return 0;
}

/*
 * GQA / MQA / MHA decode.
 *   q [b, s, hq, d], kc and vc [b, t_max, hkv, d], seqlens [b].
 * rows: optional flattened row ids ((bi * s + i) * hq + hh); out [n_rows, d].
 */
int oracle_gqa(const uint16_t *q, const uint16_t *kc, const uint16_t *vc,
               const int32_t *seqlens, int b, int s, int hq, int hkv, int d, int t_max,
               double scale, const int64_t *rows, int64_t n_rows, double *out,
               double *lse, int64_t *macs, int n_threads)
{
    if (b <= 0 || s <= 0 || hq <= 0 || hkv <= 0 || d <= 0 || t_max <= 0) return 1;
    if (hq % hkv != 0) return 1;
    int group = hq / hkv;
    int64_t total_rows = (int64_t)b * s * hq;
    if (rows == NULL) n_rows = total_rows;
    set_threads(n_threads);
    int64_t mac_total = 0;
    const int64_t token_stride = (int64_t)hkv * d;

#pragma omp parallel reduction(+ : mac_total)
    {
        double *z = (double *)malloc(sizeof(double) * (size_t)t_max);
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < n_rows; ++r) {
            int64_t row = rows ? rows[r] : r;
            int hh = (int)(row % hq);
            int i = (int)((row / hq) % s);
            int bi = (int)(row / ((int64_t)hq * s));
            int kv = hh / group;
            int L = clamp_len(seqlens[bi], t_max);
            int n = L - s + i + 1;
            double *o = out + r * d;
            if (n <= 0) {
                for (int e = 0; e < d; ++e) o[e] = 0.0;
                lse[r] = -INFINITY;
                continue;
            }
            const uint16_t *qv = q + row * d;
            const uint16_t *kb = kc + (int64_t)bi * t_max * token_stride + (int64_t)kv * d;
            const uint16_t *vb = vc + (int64_t)bi * t_max * token_stride + (int64_t)kv * d;
            for (int j = 0; j < n; ++j) {
                const uint16_t *kj = kb + (int64_t)j * token_stride;
                double dot = 0.0;
                for (int e = 0; e < d; ++e)
                    dot += bf16_bits_to_double(qv[e]) * bf16_bits_to_double(kj[e]);
                z[j] = scale * dot;
            }
            lse[r] = softmax_in_place(z, n);
            for (int e = 0; e < d; ++e) o[e] = 0.0;
            for (int j = 0; j < n; ++j) {
                const uint16_t *vj = vb + (int64_t)j * token_stride;
                for (int e = 0; e < d; ++e) o[e] += z[j] * bf16_bits_to_double(vj[e]);
            }
            mac_total += 2 * (int64_t)n * d;
        }
        free(z);
    }
    if (macs) *macs = mac_total;
    return 0;
}

/*
 * Generic single-head softmax attention in double precision, the textbook
 * definition with separate key and value widths:
 *   Q [nq, dk], K [t, dk], V [t, dv]; query row r sees keys 0 .. n_vis[r]-1.
 *   out [nq, dv], lse [nq] (natural log). Rows with n_vis <= 0 get 0 / -inf.
 */
int oracle_attn_generic(const double *Q, const double *K, const double *V,
                        const int32_t *n_vis, int nq, int t, int dk, int dv,
                        double scale, double *out, double *lse)
{
    if (nq < 0 || t < 0 || dk <= 0 || dv <= 0) return 1;
    double *z = (double *)malloc(sizeof(double) * (size_t)(t > 0 ? t : 1));
    for (int r = 0; r < nq; ++r) {
        int n = n_vis[r] < t ? n_vis[r] : t;
        double *o = out + (int64_t)r * dv;
        for (int e = 0; e < dv; ++e) o[e] = 0.0;
        if (n <= 0) {
            lse[r] = -INFINITY;
            continue;
        }
        for (int j = 0; j < n; ++j) {
            double dot = 0.0;
            for (int e = 0; e < dk; ++e) dot += Q[(int64_t)r * dk + e] * K[(int64_t)j * dk + e];
            z[j] = scale * dot;
        }
        lse[r] = softmax_in_place(z, n);
        for (int j = 0; j < n; ++j)
            for (int e = 0; e < dv; ++e) o[e] += z[j] * V[(int64_t)j * dv + e];
    }
    free(z);
    return 0;
}
