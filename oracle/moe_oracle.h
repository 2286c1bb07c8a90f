/*
 * CPU oracle of the quantized routed-MoE layer (DeepSeek V4 Flash shape).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header or table with the GPU library and is never part of the product path.
 *
 * Every floating-point quantity is computed in fp64 except where a float
 * decides an integer or is itself a compared result (router logits, scores,
 * keys, combine weights, quantizer scales and codes): those follow the
 * fp32 definitions stated per function.  Parity of each function is pinned
 * by the CPU test suite (brute force, exact arithmetic, closed forms).
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_FMT_Q8 = 1, ORC_FMT_Q2 = 2 };
enum { ORC_ROUTE_LEARNED = 1, ORC_ROUTE_HASH = 2, ORC_ROUTE_HASH_SCORED = 3 };

typedef struct {
    int32_t hidden;     /* H */
    int32_t n_experts;  /* E */
    int32_t top_k;      /* k */
    int32_t ffn;        /* F (routed and shared) */
    int32_t has_shared; /* 0 or 1 */
    int32_t routed_fmt; /* ORC_FMT_Q8 / ORC_FMT_Q2 (shared is always Q8) */
    int32_t route;      /* ORC_ROUTE_LEARNED / ORC_ROUTE_HASH / ORC_ROUTE_HASH_SCORED */
    int32_t table_k;    /* entries per hash-table row (0: top_k); the first top_k are kept */
} orc_shape;

/* Canonical weights: banks of E matrices (gate/up [F][H], down [H][F]) and the
 * shared expert's three Q8 matrices, in the storage formats of moe_oracle.c. */
typedef struct {
    const float *router_w;   /* [E][H] fp32 (learned, hash_scored) */
    const float *router_b;   /* [E] fp32 or NULL (learned) */
    const int32_t *table;    /* [vocab][table_k] (hash, hash_scored) */
    int32_t vocab;
    const uint8_t *gate, *up, *down;
    const uint8_t *sh_gate, *sh_up, *sh_down;
} orc_weights;

double orc_f16_to_double(uint16_t h);

/* a1: logits [T][E] fp32. */
void orc_router_logits(const float *x, const float *w, int32_t T, int32_t E, int32_t H, float *logits);
/* pairwise fp64 sum of n values (n a power of two); exported for the pins */
double orc_pairwise_sum(const double *v, int32_t n);
float orc_sigmoid(float l);
/* a2: learned selection -> ids [T][k], weights [T][k]; scores [T][E] optional */
void orc_route_learned(const float *logits, const float *bias, int32_t T, int32_t E, int32_t k,
                       int32_t *ids, float *w, float *scores);
/* a2: hash selection from rows of table_k entries (first k kept), weights 1/k;
 * returns 0, or -1 for an out-of-range id or table entry or a repeated expert */
int orc_route_hash(const int32_t *token_ids, const int32_t *table, int32_t vocab, int32_t table_k, int32_t T,
                   int32_t E, int32_t k, int32_t *ids, float *w);
/* a2: hash selection as above, weights = the kept experts' router scores
 * renormalised to sum to one (summed in table order) */
int orc_route_hash_scored(const int32_t *token_ids, const int32_t *table, int32_t vocab, int32_t table_k,
                          const float *logits, int32_t T, int32_t E, int32_t k, int32_t *ids, float *w);
/* a3: quantize n values (n % 32 == 0) into int8 codes and fp32 block scales */
void orc_quantize(const float *x, int64_t n, int8_t *q, float *d);
/* a4: stable counting sort of the T*k (token, slot) pairs by expert */
void orc_sort_pairs(const int32_t *ids, int32_t T, int32_t k, int32_t E, int32_t *counts, int32_t *offsets,
                    int32_t *perm);

/* Dequantized row dot products in fp64 (value of the weight row times the
 * value of the quantized activation): out[r] for r in [0, rows). */
void orc_matvec(const uint8_t *mat, int32_t fmt, int32_t rows, int32_t cols, const int8_t *aq, const float *ad,
                double *out);
/* Exact integer block sums: Q8 -> out[r][cols/32] = sum_j qw*qa over block;
 * Q2 -> out[r][cols/16] = sum_i q_i*qa_i over each 16-weight subblock. */
void orc_block_sums(const uint8_t *mat, int32_t fmt, int32_t rows, int32_t cols, const int8_t *aq, int32_t *out);

/* One expert on one token: gate/up -> SwiGLU -> h (rounded to fp32) ->
 * quantized h -> down.  h, hq, hd, y may be NULL. */
void orc_expert(const uint8_t *gate, const uint8_t *up, const uint8_t *down, int32_t fmt, int32_t H, int32_t F,
                const int8_t *xq, const float *xd, float *h, int8_t *hq, float *hd, double *y);

/* Whole layer on T tokens.  out [T][H] fp32.  Optional outputs (NULL to skip):
 * ids/w [T][k], logits [T][E], xq [T][H], xd [T][H/32],
 * h [T][k+1][F] fp32, hq [T][k+1][F], hd [T][k+1][F/32] — slot j<k is the
 * j-th selected expert in rank order, slot k the shared expert.
 * dense != 0 evaluates every expert and weights unselected ones by 0.
 * Returns 0, or -1 on invalid routing input. */
int orc_forward(const orc_shape *s, const orc_weights *wt, const float *x, const int32_t *token_ids, int32_t T,
                int32_t dense, float *out, int32_t *ids, float *w, float *logits, int8_t *xq, float *xd,
                float *h, int8_t *hq, float *hd);

/* Threads the oracle's token loop may use (OpenMP); returns the count in effect. */
int orc_set_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
