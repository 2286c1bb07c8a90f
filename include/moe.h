/*
 * moe.h — C ABI of the quantized routed mixture-of-experts FFN layer on
 * MI355X (gfx950).
 *
 * The layer is the routed-expert FFN of the DeepSeek V4 Flash model described
 * on "DeepSeek V4 Flash — DFlash Integration" (section Model Architecture:
 * hidden 4096, 256 routed experts top-6 plus 1 shared expert, expert FFN
 * 2048; hash routing by token id on the first layers, top-k over a learned
 * router with optional bias elsewhere).  Per token it computes:
 *
 *   route   learned: logits l = x.W_r (fp64 pairwise sum, rounded to fp32),
 *           scores s = sigmoid(l), key = s + bias, the top-k keys select the
 *           experts and their weights are s / sum(selected s); hash: the
 *           token's row of a fixed table, weights 1/k.  ("DeepSeek V4 Flash —
 *           DFlash Integration", Monolithic HIP: keep the highest-ranked N
 *           experts and renormalise; "ds4: dfm Edition": router top-k
 *           returning selected IDs and normalized weights.)
 *   quant   x split in 32-blocks, each quantized to int8 with an fp32 scale
 *           d = amax/127, q = rint(x/d) ("DwarfStar (ds4) — ROCm / gfx1151
 *           fork", Performance optimizations: the "preq" q8_0 kernels take
 *           pre-quantized activations).
 *   expert  g = Wg.x, u = Wu.x with int32 sums per weight block times the two
 *           block scales, h = SiLU(g)*u, h re-quantized per 32-block,
 *           y = Wd.h; out = sum over selected experts of w_e*y_e plus the
 *           shared expert's y ("DwarfStar (ds4) — ROCm / gfx1151 fork",
 *           Performance optimizations: moe_gate_up_mid_* and moe_down_sum6
 *           kernels; Model Weights: routed experts 2-bit, shared experts Q8).
 *
 * Conventions for every entry point:
 *  - Tensor pointers are DEVICE pointers owned by the caller; the library
 *    never frees them and keeps no reference after a call returns.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls enqueue
 *    work on it and return without synchronising, except where stated.
 *  - Arguments are validated on the host before anything is enqueued; a
 *    rejected call returns a negative moe_status and enqueues nothing.
 *    Launch failures return MOE_ERR_HIP.  Device-side faults, if any, appear
 *    at the caller's next synchronisation.
 *  - Calls sharing one workspace must not overlap (same stream, or ordered).
 */
#ifndef QRMOE_MOE_H
#define QRMOE_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 3
#define MOE_MAX_TOKENS 16384 /* tokens per call; larger batches are refused, not split */

typedef enum moe_status {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = -1,     /* NULL/misaligned/overlapping pointer, bad enum, k > E ... */
    MOE_ERR_UNSUPPORTED = -2,     /* shape outside the compiled set (see moe_shape) */
    MOE_ERR_TOO_MANY_TOKENS = -3, /* tokens > MOE_MAX_TOKENS */
    MOE_ERR_WORKSPACE = -4,       /* workspace smaller than moe_workspace_bytes() or misaligned */
    MOE_ERR_HIP = -5,             /* a HIP runtime call or kernel launch failed */
    MOE_ERR_BAD_TABLE = -6,       /* hash table entry out of range or repeated within a row */
    MOE_ERR_BAD_TOKEN = -7,       /* a token id outside [0, vocab) was seen (moe_workspace_flags) */
    MOE_ERR_NOT_PREPARED = -8     /* a context forward before a successful moe_prepare */
} moe_status;

/* Weight storage formats (canonical, little-endian, row-major [rows][cols]):
 *  MOE_FMT_Q8_32  : per 32 weights one 34-byte block: fp16 d, int8 q[32];
 *                   weight = d*q.  (q8_0-style, "DwarfStar (ds4) — ROCm /
 *                   gfx1151 fork", Performance optimizations.)
 *  MOE_FMT_Q2_256 : per 256 weights one 84-byte superblock: fp16 d, fp16
 *                   dmin, uint8 sm[16], uint8 qs[64]; weight i has 2-bit code
 *                   q = (qs[i/4] >> 2*(i%4)) & 3 and, with j = i/16,
 *                   s = sm[j] & 15, m = sm[j] >> 4, weight = d*s*q - dmin*m.
 *                   (2-bit routed experts: same page, Model Weights.)
 * Forward calls read weights only in the PACKED layout that moe_pack_weights
 * produces from the canonical one (same byte count). */
enum { MOE_FMT_Q8_32 = 1, MOE_FMT_Q2_256 = 2 };
/* Routing (a2).  LEARNED: sigmoid scores of the router logits, the top_k
 * largest score + bias, weights = scores renormalised over the kept experts.
 * HASH: the first top_k entries of the token's row of a fixed table, weights
 * 1/top_k.  HASH_SCORED: the table's experts weighted by their router scores
 * renormalised over the kept experts (summed in table order).  Keeping fewer
 * experts than a table row holds (top_k < table_k), or a smaller top_k for
 * the learned router, is the reduced top-k of "DeepSeek V4 Flash — DFlash
 * Integration", Monolithic HIP (--ds4-expert-top-k). */
enum { MOE_ROUTE_LEARNED = 1, MOE_ROUTE_HASH = 2, MOE_ROUTE_HASH_SCORED = 3 };

/* Layer shape.  Supported: hidden H and ffn F powers of two in [128, 4096]
 * (Q8_32; Q2_256 needs [512, 4096]); 1 <= top_k <= 8; top_k <= n_experts
 * <= 1024; for the two hash routes vocab >= 1 and table_k == 0 (rows of
 * top_k entries) or top_k <= table_k <= 8. */
typedef struct moe_shape {
    int32_t hidden;     /* H */
    int32_t n_experts;  /* E routed experts */
    int32_t top_k;      /* k experts per token */
    int32_t ffn;        /* F, routed and shared experts */
    int32_t has_shared; /* 1: one always-on shared expert (Q8_32), weight 1 */
    int32_t routed_fmt; /* MOE_FMT_* of the routed experts */
    int32_t route;      /* MOE_ROUTE_* */
    int32_t vocab;      /* rows of the hash table (hash routing) */
    int32_t table_k;    /* entries per hash-table row; 0 means top_k */
} moe_shape;

/* Layer weights, all device pointers, 16-byte aligned. */
typedef struct moe_weights {
    const float *router_w;     /* learned, hash_scored: [E][H] fp32 */
    const float *router_b;     /* learned: [E] fp32, or NULL for no bias */
    const int32_t *hash_table; /* hash, hash_scored: [vocab][table_k] int32 expert ids */
    const void *gate;          /* packed bank of E matrices [F][H] in routed_fmt */
    const void *up;            /* packed bank of E matrices [F][H] in routed_fmt */
    const void *down;          /* packed bank of E matrices [H][F] in routed_fmt */
    const void *sh_gate;       /* packed Q8_32 [F][H]; NULL iff has_shared == 0 */
    const void *sh_up;         /* packed Q8_32 [F][H] */
    const void *sh_down;       /* packed Q8_32 [H][F] */
} moe_weights;

/* Optional copies of intermediate results for verification (device
 * pointers; any may be NULL).  Pair index p = t*k + j for the j-th selected
 * expert of token t (rank order), p = T*k + t for the shared expert. */
typedef struct moe_debug {
    int32_t *ids;      /* [T][k] selected experts, rank order */
    float *w;          /* [T][k] combine weights */
    float *logits;     /* [T][E] router logits (learned, hash_scored) */
    int8_t *xq;        /* [T][H] quantized x */
    float *xd;         /* [T][H/32] x block scales */
    int32_t *counts;   /* [E] pairs per expert */
    int32_t *offsets;  /* [E+1] exclusive prefix of counts */
    int32_t *perm;     /* [T*k] pairs grouped by expert, increasing p within an expert */
    int8_t *hq;        /* [P][F] quantized h, P = T*k + T*has_shared */
    float *hd;         /* [P][F/32] h block scales */
    /* Exact integer block sums of sampled weight rows (rows r with
     * r % sum_row_stride == 0, stride a power of two <= min(H, F)): Q8 per 32-block,
     * Q2 per 16-weight subblock.  gate_sums/up_sums [P][F/stride][W_h],
     * down_sums [P][H/stride][W_f] with W_h = H/16, W_f = F/16 when the routed
     * experts are Q2_256 and H/32, F/32 otherwise; a Q8_32 pair (the shared
     * expert) fills the first H/32 (F/32) entries of its row. */
    int32_t *gate_sums;
    int32_t *up_sums;
    int32_t *down_sums;
    int32_t sum_row_stride; /* >= 1 when any *_sums pointer is set */
} moe_debug;

int moe_abi_version(void);
const char *moe_status_string(int status);
/* Name of the last HIP error behind an MOE_ERR_HIP returned on the calling
 * thread ("hipSuccess" if there was none).  The string is static. */
const char *moe_last_hip_error(void);

/* Bytes of one matrix [rows][cols] in fmt (canonical and packed layouts have
 * the same size), or -1 when cols does not fit the format. */
int64_t moe_matrix_bytes(int32_t fmt, int64_t rows, int64_t cols);

/* Repack n_mats canonical matrices [rows][cols] (back to back) into the
 * library's packed layout.  canonical and packed are device buffers of
 * n_mats*moe_matrix_bytes() bytes, 16-byte aligned, not overlapping.  This is
 * the load-time step that builds the aligned weight artifacts ("ds4: dfm
 * Edition", About this fork: aligned SoA artifacts built in-process at load). */
int moe_pack_weights(int32_t fmt, const void *canonical, void *packed, int64_t n_mats, int64_t rows, int64_t cols,
                     void *stream);

/* Check a hash table [vocab][row_k] on the device (row_k = the shape's
 * table_k, or top_k when that is 0; at most 8): every entry in
 * [0, n_experts) and no expert twice in a row.  Synchronises `stream`.  Needs
 * a workspace of at least 256 bytes.  Returns MOE_OK or MOE_ERR_BAD_TABLE
 * with the first bad row in *bad_row (host pointer, may be NULL). */
int moe_check_hash_table(const int32_t *table, int32_t vocab, int32_t row_k, int32_t n_experts, void *workspace,
                         size_t workspace_bytes, int32_t *bad_row, void *stream);

/* Device workspace bytes a forward call with `tokens` tokens needs (0 when
 * the shape is unsupported).  Monotone in tokens, so a workspace sized for
 * the largest batch serves every smaller one.  256-byte alignment required. */
size_t moe_workspace_bytes(const moe_shape *shape, int32_t tokens);

/* The layer: out[T][H] (fp32, overwritten) from x[T][H] (fp32).  token_ids
 * [T] int32 is required for hash routing and ignored otherwise.  out must not
 * overlap x.  tokens == 0 is a no-op (pointers may then be NULL).  The
 * workspace must have been initialised (moe_workspace_init).
 * Token ids outside [0, vocab) are clamped to row 0 of the table and
 * recorded in the workspace flags (see moe_workspace_flags). */
int moe_layer_forward(const moe_shape *shape, const moe_weights *weights, const float *x, const int32_t *token_ids,
                      int32_t tokens, float *out, void *workspace, size_t workspace_bytes, void *stream);

/* For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): moe_layer_forward without
 * a workspace argument.  Its workspace is a fixed device array of
 * MOE_STATIC_SCRATCH_BYTES inside the library, one copy per GPU, held until
 * the process ends; the call allocates nothing.  A batch whose workspace
 * (moe_workspace_bytes) exceeds it is refused with MOE_ERR_WORKSPACE before
 * anything is enqueued (at hidden 4096, 256 experts top-6 and ffn 2048 the
 * limit admits batches of up to 120 tokens).  The first call on a device
 * looks up that device's copy and enqueues the clearing of its control words
 * on `stream`.  Every call on one GPU shares its array: calls that overlap on
 * one GPU (different streams, or threads without ordering) race and must not
 * be issued.  Sticky flags are kept in the array but cannot be read through
 * this entry point (out-of-range ids are still clamped). */
#define MOE_STATIC_SCRATCH_BYTES (16u << 20)
int moe_layer_forward_static(const moe_shape *shape, const moe_weights *weights, const float *x,
                             const int32_t *token_ids, int32_t tokens, float *out, void *stream);

/* Same computation, plus copies of intermediates into `dbg`. */
int moe_layer_forward_debug(const moe_shape *shape, const moe_weights *weights, const float *x,
                            const int32_t *token_ids, int32_t tokens, float *out, void *workspace,
                            size_t workspace_bytes, const moe_debug *dbg, void *stream);

/* Zero a workspace's control words (work-list length, sticky flags).
 * Required once after allocating a workspace, before its first forward call. */
int moe_workspace_init(void *workspace, size_t workspace_bytes, void *stream);

/* Read the sticky device-side flags of a workspace (MOE_FLAG_* bits): a
 * token id outside [0, vocab) (clamped to row 0), a hash-table entry outside
 * [0, E) (clamped to expert 0), or a kept hash-table row that names one
 * expert twice.  The last two describe a table that moe_check_hash_table
 * rejects; the layer still runs without faulting, but a repeated expert is
 * weighted once where the row names it twice, so that call's output is not
 * the layer's.  The flags stay set until moe_workspace_init.  Synchronises
 * `stream`. */
enum { MOE_FLAG_BAD_TOKEN = 1, MOE_FLAG_BAD_TABLE_ENTRY = 2, MOE_FLAG_REPEATED_EXPERT = 4 };
int moe_workspace_flags(void *workspace, int32_t *flags, void *stream);

/* ------------------------------------------------- library-owned layers
 * A context owns everything one layer needs between forward calls: a
 * workspace sized for max_tokens, packed copies of the expert banks, and
 * copies of the router weights, bias and hash table.  The lifecycle is
 * create -> prepare (once per set of weights) -> forward (any number of
 * times) -> destroy, the load-time preparation and fenced forward of "ds4:
 * dfm Edition" (About this fork: aligned artifacts built in-process at load;
 * Benchmarking: typed refusals instead of silent fallbacks), behind a plain C
 * handle as in "Working on the ds4 Backend" (Wire shape: engine open, session
 * create).  The caller-workspace calls above stay available for callers that
 * manage memory themselves.
 *
 * A context lives on the device current at moe_ctx_create (moe_prepare and
 * moe_ctx_forward return MOE_ERR_INVALID_ARG when another device is current)
 * and is used from one stream at a time.  It allocates device memory (hipMalloc) only in
 * moe_ctx_create and the first moe_prepare, and frees it in moe_ctx_destroy. */
typedef struct moe_ctx moe_ctx;

/* Validate the shape (MOE_ERR_INVALID_ARG / MOE_ERR_UNSUPPORTED), allocate a
 * workspace for batches of up to max_tokens (1..MOE_MAX_TOKENS) and enqueue
 * its initialisation on `stream`.  *ctx is set only on success. */
int moe_ctx_create(const moe_shape *shape, int32_t max_tokens, moe_ctx **ctx, void *stream);

/* Load one set of weights into the context.  `canonical` holds device
 * pointers in the CANONICAL formats above (gate/up/down banks of E matrices,
 * the shared expert's three Q8_32 matrices, router weights [E][H] fp32, bias
 * [E] fp32 or NULL, hash table [vocab][table_k or top_k] int32), 16-byte
 * aligned; they are only read during this call.  The banks are repacked into
 * library-owned memory, router, bias and table are copied, and the table is
 * validated (every kept entry in [0, E), no expert twice in a row): a bad
 * table returns MOE_ERR_BAD_TABLE and leaves the context unprepared, so no
 * forward call runs on it.  Synchronises `stream`.  A later moe_prepare
 * replaces the weights in place. */
int moe_prepare(moe_ctx *ctx, const moe_weights *canonical, void *stream);

/* moe_layer_forward on the context's weights and workspace: out[T][H] from
 * x[T][H], token_ids [T] for the hash routes.  MOE_ERR_NOT_PREPARED before a
 * successful moe_prepare; MOE_ERR_TOO_MANY_TOKENS when tokens > max_tokens. */
int moe_ctx_forward(moe_ctx *ctx, const float *x, const int32_t *token_ids, int32_t tokens, float *out,
                    void *stream);

/* The context workspace's sticky flags (moe_workspace_flags); reset = 1
 * clears them after reading.  Synchronises `stream`. */
int moe_ctx_flags(moe_ctx *ctx, int32_t *flags, int32_t reset, void *stream);

/* Free the context and everything it owns (waits for its pending work).
 * NULL is a no-op. */
void moe_ctx_destroy(moe_ctx *ctx);

/* Per-stage timing with HIP events.  While a profiler is attached to the
 * calling thread, every kernel a forward call launches records its own start
 * and end into two events (hipExtLaunchKernelGGL; dispatch latency between
 * kernels is not counted).  moe_prof_collect waits for the recorded
 * events, adds the elapsed milliseconds and launch counts per stage into the
 * caller's arrays (n_stages entries, index = stage id) and forgets them. */
typedef struct moe_prof moe_prof;
enum {
    MOE_STAGE_ROUTE = 0,   /* decode batches: quantize x, router logits */
    MOE_STAGE_QUANT = 1,   /* batched: activation quantizer */
    MOE_STAGE_LOGITS = 2,  /* batched: router logits */
    MOE_STAGE_SELECT = 3,  /* top-k / hash selection (decode batches of 2..32: + sort, work list) */
    MOE_STAGE_SORT = 4,    /* batched: token sort into per-expert work lists */
    MOE_STAGE_GATEUP = 5,  /* routed and shared gate/up + SwiGLU + quantize h (one token: + selection, work list) */
    MOE_STAGE_DOWN = 6,    /* expert down projection (one token: + the weighted combine) */
    MOE_STAGE_COMBINE = 7, /* sum over each token's experts (ascending id) + shared */
    MOE_N_STAGES = 8
};
const char *moe_stage_name(int32_t stage);
int moe_prof_create(moe_prof **prof, int32_t max_events);
void moe_prof_destroy(moe_prof *prof);
int moe_prof_attach(moe_prof *prof); /* NULL detaches */
int moe_prof_collect(moe_prof *prof, float *stage_ms, int32_t *stage_launches, int32_t n_stages);

#ifdef __cplusplus
}
#endif
#endif
