/*
 * CPU oracle of the quantized routed-MoE layer — TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, single-pass C (C11, -O2, -ffp-contract=off, no intrinsics).
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * load it.  It shares no code with the GPU library.
 *
 * What the layer computes (sources are the pages' sections named here):
 *  - Shape: hidden H, E routed experts of which the top k are used, one
 *    shared expert, expert FFN width F ("DeepSeek V4 Flash — DFlash
 *    Integration", Model Architecture table: 4096 / 256 top-6 + 1 / 2048).
 *  - Routing: a learned router with optional bias on most layers, a fixed
 *    token-id -> experts table on the first layers (same table).  Scores are
 *    sigmoids of the router logits (the pages state sigmoid top-k routing for
 *    the Motif-3 family in "ds4: dfm Edition", Motif-3 section; the same
 *    reading is taken here), the bias only shifts the selection key, and the
 *    kept experts' weights are renormalised to sum to one ("DeepSeek V4 Flash —
 *    DFlash Integration", Monolithic HIP, --ds4-expert-top-k; "ds4: dfm
 *    Edition", router top-k returning selected IDs and normalized weights).
 *  - Expert FFN: gate and up projections, SwiGLU, down projection, weighted
 *    sum over the selected experts plus the shared expert ("DwarfStar (ds4) —
 *    ROCm / gfx1151 fork", Performance optimizations: moe_gate_up_mid_* and
 *    moe_down_sum6 kernels; shared experts kept at Q8 per Model Weights).
 *  - Quantization: routed experts in Q8_32 or 2-bit Q2_256 blocks, shared
 *    expert in Q8_32; activations pre-quantized per 32-block to int8 with an
 *    fp32 scale before every quantized dot ("preq" kernels in the same
 *    Performance optimizations list).
 *
 * Readings where the pages are silent (each is listed with its reason in the
 * design notes): router logit = fp32 rounding of an fp64 pairwise sum of the
 * exact products; sigmoid evaluated in fp64 and rounded to fp32; ties in the
 * selection key go to the smaller expert id; hash-routed weights are 1/k (or,
 * in the score-weighted variant, the renormalised router scores);
 * quantizer d = amax/127, q = rint(x * (1/d)) clamped to +-127; h is
 * quantized again before the down projection; the combine weight multiplies
 * the expert output after the down projection; the shared expert has weight 1.
 *
 * Storage formats (little-endian):
 *   Q8_32 block, 34 bytes: fp16 d, 32 int8 codes q; value = d*q.
 *   Q2_256 superblock, 84 bytes: fp16 d, fp16 dmin, sm[16], qs[64]; weight i
 *   has code q_i = (qs[i/4] >> 2*(i%4)) & 3, subblock j = i/16 has scale
 *   s_j = sm[j] & 15 and min m_j = sm[j] >> 4; value = d*s_j*q_i - dmin*m_j.
 *   Matrices are row-major [rows][cols], each row cols/32 (or cols/256)
 *   consecutive blocks; a bank stores its matrices back to back.
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

double orc_f16_to_double(uint16_t h) {
    int sign = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0) v = ldexp((double)m, -24);
    else if (e == 31) v = m ? NAN : INFINITY;
    else v = ldexp((double)(1024 + m), e - 25);
    return sign ? -v : v;
}

static uint16_t rd16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }

static int64_t mat_bytes(int32_t fmt, int64_t rows, int64_t cols) {
    return fmt == ORC_FMT_Q8 ? rows * (cols / 32) * 34 : rows * (cols / 256) * 84;
}

int orc_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
    return omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}

/* Pairwise (tree) summation in fp64 over n = 2^m values: level by level,
 * element i of the next level is v[2i] + v[2i+1].  Works on a copy. */
double orc_pairwise_sum(const double *v, int32_t n) {
    double *t = (double *)malloc(sizeof(double) * (size_t)n);
    memcpy(t, v, sizeof(double) * (size_t)n);
    for (int32_t len = n; len > 1; len /= 2)
        for (int32_t i = 0; i < len / 2; ++i) t[i] = t[2 * i] + t[2 * i + 1];
    double r = t[0];
    free(t);
    return r;
}

/* a1 — router logits: l[t][e] = fp32( pairwise fp64 sum over i of x[t][i]*W[e][i] ).
 * Each fp32*fp32 product is exact in fp64. */
void orc_router_logits(const float *x, const float *w, int32_t T, int32_t E, int32_t H, float *logits) {
#pragma omp parallel
    {
        double *prod = (double *)malloc(sizeof(double) * (size_t)H);
#pragma omp for schedule(static)
        for (int64_t te = 0; te < (int64_t)T * E; ++te) {
            int64_t t = te / E, e = te % E;
            for (int32_t i = 0; i < H; ++i) prod[i] = (double)x[t * H + i] * (double)w[e * H + i];
            for (int32_t len = H; len > 1; len /= 2)
                for (int32_t i = 0; i < len / 2; ++i) prod[i] = prod[2 * i] + prod[2 * i + 1];
            logits[te] = (float)prod[0];
        }
        free(prod);
    }
}

/* sigmoid in fp64, rounded once to fp32 */
float orc_sigmoid(float l) { return (float)(1.0 / (1.0 + exp(-(double)l))); }

/* a2 — learned selection.  key = s + bias (one fp32 add); the k largest keys
 * are taken in rank order (larger key first, equal keys: smaller expert id);
 * S = sum of the selected unbiased scores in rank order (fp32), w_j = s_j / S. */
void orc_route_learned(const float *logits, const float *bias, int32_t T, int32_t E, int32_t k, int32_t *ids,
                       float *w, float *scores) {
    float *s = (float *)malloc(sizeof(float) * (size_t)E);
    float *key = (float *)malloc(sizeof(float) * (size_t)E);
    char *taken = (char *)malloc((size_t)E);
    for (int32_t t = 0; t < T; ++t) {
        for (int32_t e = 0; e < E; ++e) {
            s[e] = orc_sigmoid(logits[(int64_t)t * E + e]);
            key[e] = s[e] + (bias ? bias[e] : 0.0f);
            taken[e] = 0;
            if (scores) scores[(int64_t)t * E + e] = s[e];
        }
        for (int32_t j = 0; j < k; ++j) {
            int32_t best = -1;
            for (int32_t e = 0; e < E; ++e)
                if (!taken[e] && (best < 0 || key[e] > key[best])) best = e;
            taken[best] = 1;
            ids[(int64_t)t * k + j] = best;
        }
        float S = 0.0f;
        for (int32_t j = 0; j < k; ++j) S += s[ids[(int64_t)t * k + j]];
        for (int32_t j = 0; j < k; ++j) w[(int64_t)t * k + j] = s[ids[(int64_t)t * k + j]] / S;
    }
    free(s);
    free(key);
    free(taken);
}

/* a2 — hash selection: the first k entries of the token's table row (rows of
 * table_k >= k entries; keeping fewer than the row holds is the reduced top-k
 * of "DeepSeek V4 Flash — DFlash Integration", Monolithic HIP,
 * --ds4-expert-top-k), in table order, weights 1/k. */
int orc_route_hash(const int32_t *token_ids, const int32_t *table, int32_t vocab, int32_t table_k, int32_t T,
                   int32_t E, int32_t k, int32_t *ids, float *w) {
    if (k < 1 || table_k < k) return -1;
    for (int32_t t = 0; t < T; ++t) {
        int32_t id = token_ids[t];
        if (id < 0 || id >= vocab) return -1;
        for (int32_t j = 0; j < k; ++j) {
            int32_t e = table[(int64_t)id * table_k + j];
            if (e < 0 || e >= E) return -1;
            for (int32_t i = 0; i < j; ++i)
                if (table[(int64_t)id * table_k + i] == e) return -1;
            ids[(int64_t)t * k + j] = e;
            w[(int64_t)t * k + j] = 1.0f / (float)k;
        }
    }
    return 0;
}

/* a2 — score-weighted hash selection: the experts of orc_route_hash, each
 * weighted by its router score s = sigmoid(logit) renormalised over the kept
 * experts: S = sum of their scores in table order (fp32), w_j = s_j / S (the
 * renormalisation of --ds4-expert-top-k applied to table-chosen experts). */
int orc_route_hash_scored(const int32_t *token_ids, const int32_t *table, int32_t vocab, int32_t table_k,
                          const float *logits, int32_t T, int32_t E, int32_t k, int32_t *ids, float *w) {
    if (orc_route_hash(token_ids, table, vocab, table_k, T, E, k, ids, w) != 0) return -1;
    for (int32_t t = 0; t < T; ++t) {
        float S = 0.0f;
        for (int32_t j = 0; j < k; ++j) S += orc_sigmoid(logits[(int64_t)t * E + ids[(int64_t)t * k + j]]);
        for (int32_t j = 0; j < k; ++j)
            w[(int64_t)t * k + j] = orc_sigmoid(logits[(int64_t)t * E + ids[(int64_t)t * k + j]]) / S;
    }
    return 0;
}

/* a3 — per-32-block quantizer: amax = max|x|, d = amax/127 (fp32 divide),
 * q = clamp(rint(x * (1/d)), -127, 127) in fp32 with ties to even; an
 * all-zero block gives d = 0 and q = 0. */
void orc_quantize(const float *x, int64_t n, int8_t *q, float *d) {
    for (int64_t b = 0; b < n / 32; ++b) {
        float amax = 0.0f;
        for (int j = 0; j < 32; ++j) {
            float a = fabsf(x[b * 32 + j]);
            if (a > amax) amax = a;
        }
        float dd = amax / 127.0f;
        float id = dd > 0.0f ? 1.0f / dd : 0.0f;
        for (int j = 0; j < 32; ++j) {
            float v = rintf(x[b * 32 + j] * id);
            if (v > 127.0f) v = 127.0f;
            if (v < -127.0f) v = -127.0f;
            q[b * 32 + j] = (int8_t)v;
        }
        d[b] = dd;
    }
}

/* a4 — pairs p = t*k + j grouped by expert: counts[e], offsets[e] (exclusive
 * prefix, offsets[E] = T*k), perm[] lists each expert's pairs in increasing p. */
void orc_sort_pairs(const int32_t *ids, int32_t T, int32_t k, int32_t E, int32_t *counts, int32_t *offsets,
                    int32_t *perm) {
    int64_t P = (int64_t)T * k;
    for (int32_t e = 0; e < E; ++e) counts[e] = 0;
    for (int64_t p = 0; p < P; ++p) counts[ids[p]]++;
    offsets[0] = 0;
    for (int32_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int32_t *fill = (int32_t *)calloc((size_t)E, sizeof(int32_t));
    for (int64_t p = 0; p < P; ++p) {
        int32_t e = ids[p];
        perm[offsets[e] + fill[e]++] = (int32_t)p;
    }
    free(fill);
}

/* value of weight (r, c) and the codes needed by the block sums */
static double q2_weight(const uint8_t *sb, int i) {
    double d = orc_f16_to_double(rd16(sb)), dmin = orc_f16_to_double(rd16(sb + 2));
    int j = i / 16;
    int s = sb[4 + j] & 15, m = sb[4 + j] >> 4;
    int q = (sb[20 + i / 4] >> (2 * (i % 4))) & 3;
    return d * s * q - dmin * m;
}

static int q2_code(const uint8_t *sb, int i) { return (sb[20 + i / 4] >> (2 * (i % 4))) & 3; }

void orc_matvec(const uint8_t *mat, int32_t fmt, int32_t rows, int32_t cols, const int8_t *aq, const float *ad,
                double *out) {
    for (int32_t r = 0; r < rows; ++r) {
        double acc = 0.0;
        if (fmt == ORC_FMT_Q8) {
            const uint8_t *row = mat + (int64_t)r * (cols / 32) * 34;
            for (int32_t b = 0; b < cols / 32; ++b) {
                double dw = orc_f16_to_double(rd16(row + b * 34));
                double da = (double)ad[b];
                for (int j = 0; j < 32; ++j)
                    acc += (dw * (double)(int8_t)row[b * 34 + 2 + j]) * (da * (double)aq[b * 32 + j]);
            }
        } else {
            const uint8_t *row = mat + (int64_t)r * (cols / 256) * 84;
            for (int32_t s = 0; s < cols / 256; ++s)
                for (int i = 0; i < 256; ++i) {
                    int32_t c = s * 256 + i;
                    acc += q2_weight(row + s * 84, i) * ((double)ad[c / 32] * (double)aq[c]);
                }
        }
        out[r] = acc;
    }
}

void orc_block_sums(const uint8_t *mat, int32_t fmt, int32_t rows, int32_t cols, const int8_t *aq, int32_t *out) {
    for (int32_t r = 0; r < rows; ++r) {
        if (fmt == ORC_FMT_Q8) {
            const uint8_t *row = mat + (int64_t)r * (cols / 32) * 34;
            for (int32_t b = 0; b < cols / 32; ++b) {
                int32_t acc = 0;
                for (int j = 0; j < 32; ++j) acc += (int32_t)(int8_t)row[b * 34 + 2 + j] * (int32_t)aq[b * 32 + j];
                out[(int64_t)r * (cols / 32) + b] = acc;
            }
        } else {
            const uint8_t *row = mat + (int64_t)r * (cols / 256) * 84;
            for (int32_t g = 0; g < cols / 16; ++g) {
                int32_t acc = 0;
                for (int i = 0; i < 16; ++i) {
                    int32_t c = g * 16 + i;
                    acc += q2_code(row + (c / 256) * 84, c % 256) * (int32_t)aq[c];
                }
                out[(int64_t)r * (cols / 16) + g] = acc;
            }
        }
    }
}

/* a5 + a6 (one expert): g = Wg.x, u = Wu.x (fp64), h = SiLU(g)*u = g/(1+e^-g)*u
 * in fp64 rounded to fp32, h quantized per 32-block, y = Wd.h (fp64). */
void orc_expert(const uint8_t *gate, const uint8_t *up, const uint8_t *down, int32_t fmt, int32_t H, int32_t F,
                const int8_t *xq, const float *xd, float *h, int8_t *hq, float *hd, double *y) {
    double *g = (double *)malloc(sizeof(double) * (size_t)F);
    double *u = (double *)malloc(sizeof(double) * (size_t)F);
    float *hf = (float *)malloc(sizeof(float) * (size_t)F);
    int8_t *q = (int8_t *)malloc((size_t)F);
    float *qd = (float *)malloc(sizeof(float) * (size_t)(F / 32));
    orc_matvec(gate, fmt, F, H, xq, xd, g);
    orc_matvec(up, fmt, F, H, xq, xd, u);
    for (int32_t r = 0; r < F; ++r) hf[r] = (float)(g[r] / (1.0 + exp(-g[r])) * u[r]);
    orc_quantize(hf, F, q, qd);
    if (y) orc_matvec(down, fmt, H, F, q, qd, y);
    if (h) memcpy(h, hf, sizeof(float) * (size_t)F);
    if (hq) memcpy(hq, q, (size_t)F);
    if (hd) memcpy(hd, qd, sizeof(float) * (size_t)(F / 32));
    free(g);
    free(u);
    free(hf);
    free(q);
    free(qd);
}

static int is_pow2(int32_t n) { return n > 0 && (n & (n - 1)) == 0; }

int orc_forward(const orc_shape *s, const orc_weights *wt, const float *x, const int32_t *token_ids, int32_t T,
                int32_t dense, float *out, int32_t *ids, float *w, float *logits, int8_t *xq, float *xd, float *h,
                int8_t *hq, float *hd) {
    const int32_t H = s->hidden, E = s->n_experts, k = s->top_k, F = s->ffn;
    if (T < 0 || k < 1 || k > E || H % 32 || F % 32) return -1;
    if (s->routed_fmt == ORC_FMT_Q2 && (H % 256 || F % 256)) return -1;
    const int32_t table_k = s->table_k ? s->table_k : k;
    if (s->route != ORC_ROUTE_HASH && !is_pow2(H)) return -1;
    int32_t *ids_ = ids ? ids : (int32_t *)malloc(sizeof(int32_t) * (size_t)T * k + 1);
    float *w_ = w ? w : (float *)malloc(sizeof(float) * (size_t)T * k + 1);
    int rc = 0;
    if (s->route == ORC_ROUTE_HASH) {
        rc = orc_route_hash(token_ids, wt->table, wt->vocab, table_k, T, E, k, ids_, w_);
    } else {
        float *l = logits ? logits : (float *)malloc(sizeof(float) * (size_t)T * E + 1);
        orc_router_logits(x, wt->router_w, T, E, H, l);
        if (s->route == ORC_ROUTE_LEARNED)
            orc_route_learned(l, wt->router_b, T, E, k, ids_, w_, NULL);
        else
            rc = orc_route_hash_scored(token_ids, wt->table, wt->vocab, table_k, l, T, E, k, ids_, w_);
        if (!logits) free(l);
    }
    if (rc == 0) {
        const int32_t fmt = s->routed_fmt;
        const int64_t gu_bytes = mat_bytes(fmt, F, H), dn_bytes = mat_bytes(fmt, H, F);
        const int32_t S = k + 1; /* slots per token: k routed + shared */
#pragma omp parallel for schedule(dynamic, 1)
        for (int32_t t = 0; t < T; ++t) {
            int8_t *q = (int8_t *)malloc((size_t)H);
            float *qd = (float *)malloc(sizeof(float) * (size_t)(H / 32));
            double *y = (double *)malloc(sizeof(double) * (size_t)H);
            double *acc = (double *)calloc((size_t)H, sizeof(double));
            orc_quantize(x + (int64_t)t * H, H, q, qd);
            if (xq) memcpy(xq + (int64_t)t * H, q, (size_t)H);
            if (xd) memcpy(xd + (int64_t)t * (H / 32), qd, sizeof(float) * (size_t)(H / 32));
            for (int32_t e = 0; e < E; ++e) {
                int32_t slot = -1;
                for (int32_t j = 0; j < k; ++j)
                    if (ids_[(int64_t)t * k + j] == e) slot = j;
                if (slot < 0 && !dense) continue;
                int64_t si = (int64_t)t * S + (slot < 0 ? 0 : slot);
                orc_expert(wt->gate + e * gu_bytes, wt->up + e * gu_bytes, wt->down + e * dn_bytes, fmt, H, F, q,
                           qd, (h && slot >= 0) ? h + si * F : NULL, (hq && slot >= 0) ? hq + si * F : NULL,
                           (hd && slot >= 0) ? hd + si * (F / 32) : NULL, y);
                double we = slot >= 0 ? (double)w_[(int64_t)t * k + slot] : 0.0;
                for (int32_t c = 0; c < H; ++c) acc[c] += we * y[c];
            }
            if (s->has_shared) {
                int64_t si = (int64_t)t * S + k;
                orc_expert(wt->sh_gate, wt->sh_up, wt->sh_down, ORC_FMT_Q8, H, F, q, qd, h ? h + si * F : NULL,
                           hq ? hq + si * F : NULL, hd ? hd + si * (F / 32) : NULL, y);
                for (int32_t c = 0; c < H; ++c) acc[c] += y[c];
            }
            for (int32_t c = 0; c < H; ++c) out[(int64_t)t * H + c] = (float)acc[c];
            free(q);
            free(qd);
            free(y);
            free(acc);
        }
    }
    if (!ids) free(ids_);
    if (!w) free(w_);
    return rc;
}
