// Host side of the C ABI declared in include/moe.h: argument validation,
// workspace layout, kernel dispatch and per-stage event timing.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/moe.h"
#include "common.hpp"

using namespace qrmoe;

namespace {

// Last HIP failure seen by a library call on this thread (hipSuccess if none).
thread_local hipError_t t_last_hip = hipSuccess;

int hip_status(hipError_t e) {
    if (e == hipSuccess) return MOE_OK;
    t_last_hip = e;
    return MOE_ERR_HIP;
}

constexpr size_t kAlign = 256;
constexpr int kMfmaTile = 64;  // pairs per MFMA work tile
// Smallest batch whose 2-bit experts take the MFMA GEMMs (Q8: every batch
// past the decode sizes).  A tile's compute time is fixed however few pairs
// it holds, and the 2-bit body's is the larger; measured at H 4096, 256
// experts top-6, F 2048: 33 tokens 412 us on the VALU kernels vs 543 us on
// the GEMMs, 48 tokens 491 vs 590, 64 tokens 584 vs 593, 128 tokens 949 vs 657.
constexpr int kMfmaMinTokensQ2 = 64;
// Largest batch past the decode sizes whose quantization and router logits
// run in the decode front kernel (one logit per workgroup).  The 32x32-tile
// logits kernel's grid fills the chip only for long batches; measured at H
// 4096, 256 experts (quantization + logits): 33 tokens 20 us vs 123 us tiled,
// 128 tokens 68 vs 124, 192 tokens 98 vs 124, 256 tokens 128 vs 124.  Both
// compute the same tree, so the results are the same bits.
constexpr int kFrontMaxTokens = 224;
// Largest decode batch whose selection, sort and work list run in the
// one-workgroup decode select kernel; past it, one wave per token selects
// (select_kernel) and the sort kernel builds the work list.  Measured
// (select + sort, 4096 hidden, 256 experts top-6): learned 8 tokens 8.4 us vs
// 8.3, 12 tokens 11.0 vs 8.3, 32 tokens 25.8 vs 8.6; hash 16 tokens 7.4 vs
// 8.5, 24 tokens 9.6 vs 8.4, 32 tokens 11.4 vs 8.4.  Same results either way.
constexpr int kDecodeSelectMaxLearned = 8, kDecodeSelectMaxHash = 20;

inline size_t up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
inline bool pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }
inline bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

int validate_shape(const moe_shape *s) {
    if (!s) return MOE_ERR_INVALID_ARG;
    if (s->routed_fmt != MOE_FMT_Q8_32 && s->routed_fmt != MOE_FMT_Q2_256) return MOE_ERR_INVALID_ARG;
    if (s->route != MOE_ROUTE_LEARNED && s->route != MOE_ROUTE_HASH && s->route != MOE_ROUTE_HASH_SCORED)
        return MOE_ERR_INVALID_ARG;
    if (s->has_shared != 0 && s->has_shared != 1) return MOE_ERR_INVALID_ARG;
    if (s->top_k < 1 || s->n_experts < s->top_k) return MOE_ERR_INVALID_ARG;
    if (s->route != MOE_ROUTE_LEARNED) {
        if (s->vocab < 1) return MOE_ERR_INVALID_ARG;
        if (s->table_k != 0 && (s->table_k < s->top_k || s->table_k > 8)) return MOE_ERR_INVALID_ARG;
    }
    if (s->top_k > 8 || s->n_experts > 1024) return MOE_ERR_UNSUPPORTED;
    const int lo = s->routed_fmt == MOE_FMT_Q2_256 ? 512 : 128;
    if (!pow2(s->hidden) || !pow2(s->ffn) || s->hidden < lo || s->ffn < lo || s->hidden > 4096 || s->ffn > 4096)
        return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

// Upper bound of the work-list length: sum over experts of ceil(n_e / G)
// with sum n_e = P and at most min(E, P) non-empty experts, plus the shared
// expert's ceil(T / G) groups.
int64_t max_groups(const moe_shape *s, int64_t T, int64_t G) {
    const int64_t P = T * s->top_k;
    const int64_t active = P < s->n_experts ? P : s->n_experts;
    return (P + active * (G - 1)) / G + (s->has_shared ? (T + G - 1) / G : 0);
}

struct Layout {
    size_t ctl, logits, scores, keys, ids, w, xq, xd, xs16, counts, offsets, perm, groups, hq, hd, hs16, y, total;
};


Layout make_layout(const moe_shape *s, int64_t T) {
    const int64_t H = s->hidden, E = s->n_experts, k = s->top_k, F = s->ffn;
    const int64_t P = T * k + (s->has_shared ? T : 0);
    int64_t G = max_groups(s, T, kVecTok);
    const int64_t G2 = max_groups(s, T, kMfmaTile);
    if (G2 > G) G = G2;
    if (G < 16) G = 16;  // the one-token down kernel reads the first 8 entries unconditionally
    Layout L{};
    size_t o = 0;
    auto take = [&](size_t bytes) {
        size_t at = o;
        o += up(bytes == 0 ? 1 : bytes);
        return at;
    };
    L.ctl = take(kCtlWords * 4);
    L.logits = take(T * E * 4);
    L.scores = take(T * E * 4);
    L.keys = take(T * E * 4);
    L.ids = take(T * k * 4);
    L.w = take(T * k * 4);
    L.xq = take(T * H);
    L.xd = take(T * (H / 32) * 4);
    L.xs16 = take(T * (H / 16) * 4);
    L.counts = take(E * 4);
    L.offsets = take((E + 1) * 4);
    L.perm = take(T * k * 4);
    L.groups = take(G * 16);
    L.hq = take(P * F);
    L.hd = take(P * (F / 32) * 4);
    // the 2-bit down GEMM of batches past the decode sizes reads h's subblock sums
    L.hs16 = take(s->routed_fmt == MOE_FMT_Q2_256 && T >= kMfmaMinTokensQ2 ? P * (F / 16) * 4 : 0);
    L.y = take(P * H * 4);
    L.total = o;
    return L;
}

struct EventPair {
    hipEvent_t a, b;
    int stage;
};

}  // namespace

struct moe_prof {
    std::vector<hipEvent_t> pool;
    std::vector<EventPair> used;
    size_t next = 0;
};

static thread_local moe_prof *t_prof = nullptr;
static thread_local int t_stage = -1;  // stage of the forward call running on this thread, or -1

namespace qrmoe {
bool next_launch_events(hipEvent_t *start, hipEvent_t *stop) {
    moe_prof *p = t_prof;
    if (!p || t_stage < 0 || p->next + 2 > p->pool.size()) return false;
    *start = p->pool[p->next++];
    *stop = p->pool[p->next++];
    p->used.push_back(EventPair{*start, *stop, t_stage});
    return true;
}
}  // namespace qrmoe

namespace {

// Runs one stage's launches with the stage recorded for the profiler: each
// kernel the stage launches is timed on its own (the chunked sort, for one,
// launches three).
template <class F>
hipError_t timed(int stage, F &&launch) {
    t_stage = stage;
    const hipError_t err = launch();
    t_stage = -1;
    return err;
}

// Host-side checks of a forward call's shape, weights, activations and debug
// request (everything but the workspace).  MOE_OK for tokens == 0 without
// looking at the pointers: the empty batch is a no-op.
int check_forward_args(const moe_shape *shape, const moe_weights *wts, const float *x, const int32_t *token_ids,
                       int32_t tokens, const float *out, const moe_debug *dbg) {
    int st = validate_shape(shape);
    if (st != MOE_OK) return st;
    if (tokens < 0) return MOE_ERR_INVALID_ARG;
    if (tokens > MOE_MAX_TOKENS) return MOE_ERR_TOO_MANY_TOKENS;
    if (tokens == 0) return MOE_OK;  // empty batch: nothing is read or written, buffers may be NULL
    if (!wts || !x || !out) return MOE_ERR_INVALID_ARG;
    const bool router = shape->route != MOE_ROUTE_HASH;     // logits are computed
    const bool hashed = shape->route != MOE_ROUTE_LEARNED;  // experts come from the table
    if (router && !wts->router_w) return MOE_ERR_INVALID_ARG;
    if (hashed && (!wts->hash_table || !token_ids)) return MOE_ERR_INVALID_ARG;
    if (!wts->gate || !wts->up || !wts->down) return MOE_ERR_INVALID_ARG;
    if (shape->has_shared && (!wts->sh_gate || !wts->sh_up || !wts->sh_down)) return MOE_ERR_INVALID_ARG;
    if (!shape->has_shared && (wts->sh_gate || wts->sh_up || wts->sh_down)) return MOE_ERR_INVALID_ARG;
    const void *al16[] = {x, out, wts->router_w, wts->gate, wts->up, wts->down, wts->sh_gate, wts->sh_up, wts->sh_down};
    for (const void *p : al16)
        if (p && !aligned(p, 16)) return MOE_ERR_INVALID_ARG;
    const int64_t T = tokens, H = shape->hidden;
    {
        const uintptr_t xa = (uintptr_t)x, oa = (uintptr_t)out, n = (uintptr_t)(T * H * 4);
        if (T > 0 && xa < oa + n && oa < xa + n) return MOE_ERR_INVALID_ARG;
    }
    if (dbg && (dbg->gate_sums || dbg->up_sums || dbg->down_sums) &&
        (!pow2(dbg->sum_row_stride) || dbg->sum_row_stride > shape->ffn || dbg->sum_row_stride > shape->hidden))
        return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

int forward_impl(const moe_shape *shape, const moe_weights *wts, const float *x, const int32_t *token_ids,
                 int32_t tokens, float *out, void *workspace, size_t ws_bytes, const moe_debug *dbg, void *stream) {
    const int st = check_forward_args(shape, wts, x, token_ids, tokens, out, dbg);
    if (st != MOE_OK || tokens == 0) return st;
    if (!workspace) return MOE_ERR_INVALID_ARG;
    if (!aligned(workspace, kAlign)) return MOE_ERR_WORKSPACE;
    const int64_t T = tokens, H = shape->hidden;
    const bool router = shape->route != MOE_ROUTE_HASH;     // logits are computed
    const bool hashed = shape->route != MOE_ROUTE_LEARNED;  // experts come from the table
    const Layout L = make_layout(shape, T);
    if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;

    hipStream_t s = (hipStream_t)stream;
    uint8_t *base = (uint8_t *)workspace;
    LayerArgs a{};
    a.d = Dims{(int32_t)T, shape->hidden, shape->n_experts, shape->top_k, shape->ffn, shape->has_shared,
               shape->routed_fmt, shape->route, shape->vocab,
               (int32_t)(T * shape->top_k + (shape->has_shared ? T : 0)),
               hashed && shape->table_k ? shape->table_k : shape->top_k,
               // the score-weighted hash reads only the scores of its table's
               // experts; the debug call copies every logit, so it computes all
               (int32_t)(shape->route == MOE_ROUTE_HASH_SCORED && !dbg)};
    a.wt = Weights{wts->router_w, wts->router_b, wts->hash_table, (const uint8_t *)wts->gate,
                   (const uint8_t *)wts->up, (const uint8_t *)wts->down, (const uint8_t *)wts->sh_gate,
                   (const uint8_t *)wts->sh_up, (const uint8_t *)wts->sh_down};
    a.ws = Ws{(int32_t *)(base + L.ctl), (float *)(base + L.logits), (int32_t *)(base + L.ids),
              (float *)(base + L.w), (int8_t *)(base + L.xq), (float *)(base + L.xd),
              (int32_t *)(base + L.xs16), (int32_t *)(base + L.counts), (int32_t *)(base + L.offsets),
              (int32_t *)(base + L.perm), (int4 *)(base + L.groups), (int8_t *)(base + L.hq),
              (float *)(base + L.hd), (float *)(base + L.y), (float *)(base + L.scores),
              (float *)(base + L.keys), (int32_t *)(base + L.hs16)};
    const bool dump = dbg && (dbg->gate_sums || dbg->up_sums || dbg->down_sums);
    const bool q2 = shape->routed_fmt == MOE_FMT_Q2_256;
    a.dump = Dump{dump ? dbg->gate_sums : nullptr, dump ? dbg->up_sums : nullptr, dump ? dbg->down_sums : nullptr,
                  dump ? dbg->sum_row_stride : 1, (int32_t)(q2 ? H / 16 : H / 32),
                  (int32_t)(q2 ? shape->ffn / 16 : shape->ffn / 32)};
    a.x = x;
    a.token_ids = token_ids;
    a.out = out;

    hipError_t err = hipSuccess;
    auto run = [&](int stage, auto &&fn) {
        if (err == hipSuccess) err = timed(stage, fn);
    };
    const int64_t mg = max_groups(shape, T, kVecTok);
    a.group_tok = kVecTok;
    if (T <= kDecodeMaxT) {
        run(MOE_STAGE_ROUTE, [&] { return launch_decode_front(a, s); });
        if (T == 1) {
            // one token: the selection runs inside the gate/up workgroups
            run(MOE_STAGE_GATEUP, [&] { return launch_decode_gateup1(a, dump, s); });
            run(MOE_STAGE_DOWN, [&] { return launch_decode_down1(a, dump, s); });
        } else {
            if (T <= (shape->route == MOE_ROUTE_LEARNED ? kDecodeSelectMaxLearned : kDecodeSelectMaxHash)) {
                run(MOE_STAGE_SELECT, [&] { return launch_decode_select(a, s); });
            } else {
                run(MOE_STAGE_SELECT, [&] { return launch_select(a, s); });
                run(MOE_STAGE_SORT, [&] { return launch_sort(a, s); });
            }
            run(MOE_STAGE_GATEUP, [&] { return launch_gateup_vec(a, (int)mg, dump, s); });
            run(MOE_STAGE_DOWN, [&] { return launch_down_vec(a, (int)mg, dump, s); });
            run(MOE_STAGE_COMBINE, [&] { return launch_combine(a, s); });
        }
    } else {
        // Q8 and 2-bit experts go through the grouped int8 MFMA GEMMs (64-pair
        // tiles); the smallest shapes, and 2-bit batches below
        // kMfmaMinTokensQ2, stay on the VALU kernels.
        const bool mfma = H >= 256 && shape->ffn >= 256 && (!q2 || T >= kMfmaMinTokensQ2);
        const int64_t tiles = mfma ? max_groups(shape, T, kMfmaTile) : mg;
        a.group_tok = mfma ? kMfmaTile : kVecTok;
        if (T <= kFrontMaxTokens) {
            run(MOE_STAGE_ROUTE, [&] { return launch_decode_front(a, s); });
        } else {
            run(MOE_STAGE_QUANT, [&] { return launch_quant(a, s); });
            if (router) run(MOE_STAGE_LOGITS, [&] { return launch_logits(a, s); });
        }
        run(MOE_STAGE_SELECT, [&] { return launch_select(a, s); });
        run(MOE_STAGE_SORT, [&] { return launch_sort(a, s); });
        if (mfma) {
            run(MOE_STAGE_GATEUP, [&] { return launch_gateup_mfma(a, (int)tiles, dump, s); });
            run(MOE_STAGE_DOWN, [&] { return launch_down_mfma(a, (int)tiles, dump, s); });
        } else {
            run(MOE_STAGE_GATEUP, [&] { return launch_gateup_vec(a, (int)mg, dump, s); });
            run(MOE_STAGE_DOWN, [&] { return launch_down_vec(a, (int)mg, dump, s); });
        }
        run(MOE_STAGE_COMBINE, [&] { return launch_combine(a, s); });
    }
    if (err == hipSuccess && dbg) {
        const int64_t E = shape->n_experts, k = shape->top_k, F = shape->ffn, P = a.d.P;
        auto cp = [&](void *dst, const void *src, size_t n) {
            if (dst && err == hipSuccess) err = hipMemcpyAsync(dst, src, n, hipMemcpyDeviceToDevice, s);
        };
        cp(dbg->ids, a.ws.ids, T * k * 4);
        cp(dbg->w, a.ws.w, T * k * 4);
        if (router) cp(dbg->logits, a.ws.logits, T * E * 4);
        cp(dbg->xq, a.ws.xq, T * H);
        cp(dbg->xd, a.ws.xd, T * (H / 32) * 4);
        cp(dbg->counts, a.ws.counts, E * 4);
        cp(dbg->offsets, a.ws.offsets, (E + 1) * 4);
        cp(dbg->perm, a.ws.perm, T * k * 4);
        cp(dbg->hq, a.ws.hq, P * F);
        cp(dbg->hd, a.ws.hd, P * (F / 32) * 4);
    }
    return hip_status(err);
}

}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char *moe_status_string(int status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARG: return "invalid argument";
        case MOE_ERR_UNSUPPORTED: return "unsupported shape";
        case MOE_ERR_TOO_MANY_TOKENS: return "too many tokens";
        case MOE_ERR_WORKSPACE: return "workspace too small or misaligned";
        case MOE_ERR_HIP: return "HIP runtime error";
        case MOE_ERR_BAD_TABLE: return "invalid hash table";
        case MOE_ERR_BAD_TOKEN: return "token id out of range";
        case MOE_ERR_NOT_PREPARED: return "context has no prepared weights";
        default: return "unknown status";
    }
}

const char *moe_last_hip_error(void) { return hipGetErrorName(t_last_hip); }

int64_t moe_matrix_bytes(int32_t fmt, int64_t rows, int64_t cols) {
    if (rows < 0 || cols <= 0) return -1;
    if (fmt == MOE_FMT_Q8_32 && cols % 32 == 0) return q8_bytes(rows, cols);
    if (fmt == MOE_FMT_Q2_256 && cols % 256 == 0) return q2_bytes(rows, cols);
    return -1;
}

int moe_pack_weights(int32_t fmt, const void *canonical, void *packed, int64_t n_mats, int64_t rows, int64_t cols,
                     void *stream) {
    const int64_t mb = moe_matrix_bytes(fmt, rows, cols);
    if (mb < 0 || n_mats < 0 || !canonical || !packed) return MOE_ERR_INVALID_ARG;
    if (!aligned(canonical, 16) || !aligned(packed, 16)) return MOE_ERR_INVALID_ARG;
    const uintptr_t c = (uintptr_t)canonical, p = (uintptr_t)packed, n = (uintptr_t)(n_mats * mb);
    if (n > 0 && c < p + n && p < c + n) return MOE_ERR_INVALID_ARG;
    if (n_mats == 0 || rows == 0) return MOE_OK;
    hipError_t err = launch_pack(fmt, (const uint8_t *)canonical, (uint8_t *)packed, n_mats, rows, cols,
                                 (hipStream_t)stream);
    return hip_status(err);
}

int moe_check_hash_table(const int32_t *table, int32_t vocab, int32_t row_k, int32_t n_experts, void *workspace,
                         size_t workspace_bytes, int32_t *bad_row, void *stream) {
    if (!table || !workspace || vocab < 1 || row_k < 1 || row_k > 8 || n_experts < row_k) return MOE_ERR_INVALID_ARG;
    if (workspace_bytes < 256 || !aligned(workspace, kAlign)) return MOE_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    int32_t *res = (int32_t *)workspace + (kCtlWords - 1);  // scratch word of the ctl area, never a counter
    if (workspace_bytes < (size_t)kCtlWords * 4) res = (int32_t *)workspace;
    hipError_t err = launch_check_table(table, vocab, row_k, n_experts, res, s);
    int32_t host = 0;
    if (err == hipSuccess) err = hipMemcpyAsync(&host, res, 4, hipMemcpyDeviceToHost, s);
    if (err == hipSuccess) err = hipStreamSynchronize(s);
    if (err != hipSuccess) return hip_status(err);
    if (bad_row) *bad_row = host == INT32_MAX ? -1 : host;
    return host == INT32_MAX ? MOE_OK : MOE_ERR_BAD_TABLE;
}

size_t moe_workspace_bytes(const moe_shape *shape, int32_t tokens) {
    if (validate_shape(shape) != MOE_OK || tokens < 0 || tokens > MOE_MAX_TOKENS) return 0;
    return make_layout(shape, tokens).total;
}

int moe_workspace_init(void *workspace, size_t workspace_bytes, void *stream) {
    if (!workspace || !aligned(workspace, kAlign)) return MOE_ERR_INVALID_ARG;
    if (workspace_bytes < (size_t)kCtlWords * 4) return MOE_ERR_WORKSPACE;
    hipError_t err = launch_ws_init((int32_t *)workspace, kCtlWords, (hipStream_t)stream);
    return hip_status(err);
}

int moe_workspace_flags(void *workspace, int32_t *flags, void *stream) {
    if (!workspace || !flags || !aligned(workspace, kAlign)) return MOE_ERR_INVALID_ARG;
    hipStream_t s = (hipStream_t)stream;
    int32_t *dev = (int32_t *)workspace + kCtlFlags;
    int32_t host = 0;
    hipError_t err = hipMemcpyAsync(&host, dev, 4, hipMemcpyDeviceToHost, s);
    if (err == hipSuccess) err = hipStreamSynchronize(s);
    if (err != hipSuccess) return hip_status(err);
    *flags = host;
    return MOE_OK;
}

int moe_layer_forward(const moe_shape *shape, const moe_weights *weights, const float *x, const int32_t *token_ids,
                      int32_t tokens, float *out, void *workspace, size_t workspace_bytes, void *stream) {
    return forward_impl(shape, weights, x, token_ids, tokens, out, workspace, workspace_bytes, nullptr, stream);
}

int moe_layer_forward_debug(const moe_shape *shape, const moe_weights *weights, const float *x,
                            const int32_t *token_ids, int32_t tokens, float *out, void *workspace,
                            size_t workspace_bytes, const moe_debug *dbg, void *stream) {
    if (!dbg) return MOE_ERR_INVALID_ARG;
    return forward_impl(shape, weights, x, token_ids, tokens, out, workspace, workspace_bytes, dbg, stream);
}

}  // extern "C"

// ------------------------------------------------ allocation-free forward
// The workspace of moe_layer_forward_static: a device array in the library's
// code object, one copy per GPU.  In host code `scratch` names a host-side
// stand-in, not device memory: kernels receive the device address that
// hipGetSymbolAddress returns for the current device, looked up once per
// device and kept in g_scratch.
static __device__ __align__(256) uint8_t scratch[MOE_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices] = {};

// The current device's copy of `scratch`; on first use on a device, also
// enqueue the clearing of its control words (a kernel, so the call may be
// captured into a graph).
hipError_t static_scratch(hipStream_t s, void **out) {
    int dev = -1;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *ptr = nullptr;
        err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (err != hipSuccess) return err;
        if (!ptr) return hipErrorInvalidSymbol;
        err = launch_ws_init((int32_t *)ptr, kCtlWords, s);
        if (err != hipSuccess) return err;
        g_scratch[dev] = ptr;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}
}  // namespace

extern "C" int moe_layer_forward_static(const moe_shape *shape, const moe_weights *weights, const float *x,
                                        const int32_t *token_ids, int32_t tokens, float *out, void *stream) {
    // every host-side check comes before the device lookup
    const int st = check_forward_args(shape, weights, x, token_ids, tokens, out, nullptr);
    if (st != MOE_OK || tokens == 0) return st;
    if (make_layout(shape, tokens).total > (size_t)MOE_STATIC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
    void *ws = nullptr;
    const hipError_t err = static_scratch((hipStream_t)stream, &ws);
    if (err != hipSuccess) return hip_status(err);
    return forward_impl(shape, weights, x, token_ids, tokens, out, ws, MOE_STATIC_SCRATCH_BYTES, nullptr, stream);
}

// ------------------------------------------------- library-owned layers
struct moe_ctx {
    moe_shape shape{};
    int32_t max_tokens = 0;
    int device = 0;
    void *ws = nullptr;
    size_t ws_bytes = 0;
    // library-owned weights: packed banks, router, bias and table copies
    void *gate = nullptr, *up = nullptr, *down = nullptr;
    void *sh_gate = nullptr, *sh_up = nullptr, *sh_down = nullptr;
    void *router_w = nullptr, *router_b = nullptr, *table = nullptr;
    bool prepared = false;
};

namespace {

void ctx_free_weights(moe_ctx *c) {
    for (void **p : {&c->gate, &c->up, &c->down, &c->sh_gate, &c->sh_up, &c->sh_down, &c->router_w, &c->router_b,
                     &c->table}) {
        if (*p) (void)hipFree(*p);
        *p = nullptr;
    }
}

// Device buffer of `bytes` owned by the context, allocated on first use and
// reused by later prepares (a context's shape fixes every size).
hipError_t ctx_buffer(void **p, size_t bytes) {
    if (*p) return hipSuccess;
    return hipMalloc(p, bytes == 0 ? 1 : bytes);
}

}  // namespace

extern "C" {

int moe_ctx_create(const moe_shape *shape, int32_t max_tokens, moe_ctx **ctx, void *stream) {
    if (!ctx) return MOE_ERR_INVALID_ARG;
    const int st = validate_shape(shape);
    if (st != MOE_OK) return st;
    if (max_tokens < 1) return MOE_ERR_INVALID_ARG;
    if (max_tokens > MOE_MAX_TOKENS) return MOE_ERR_TOO_MANY_TOKENS;
    moe_ctx *c = new moe_ctx();
    c->shape = *shape;
    c->max_tokens = max_tokens;
    c->ws_bytes = make_layout(shape, max_tokens).total;
    hipError_t err = hipGetDevice(&c->device);
    if (err == hipSuccess) err = hipMalloc(&c->ws, c->ws_bytes);
    if (err == hipSuccess) err = launch_ws_init((int32_t *)c->ws, kCtlWords, (hipStream_t)stream);
    if (err != hipSuccess) {
        if (c->ws) (void)hipFree(c->ws);
        delete c;
        return hip_status(err);
    }
    *ctx = c;
    return MOE_OK;
}

int moe_prepare(moe_ctx *c, const moe_weights *w, void *stream) {
    if (!c || !w) return MOE_ERR_INVALID_ARG;
    const moe_shape &sh = c->shape;
    const bool router = sh.route != MOE_ROUTE_HASH, hashed = sh.route != MOE_ROUTE_LEARNED;
    if (router && !w->router_w) return MOE_ERR_INVALID_ARG;
    if (sh.route != MOE_ROUTE_LEARNED && w->router_b) return MOE_ERR_INVALID_ARG;
    if (hashed && !w->hash_table) return MOE_ERR_INVALID_ARG;
    if (!w->gate || !w->up || !w->down) return MOE_ERR_INVALID_ARG;
    if (sh.has_shared && (!w->sh_gate || !w->sh_up || !w->sh_down)) return MOE_ERR_INVALID_ARG;
    if (!sh.has_shared && (w->sh_gate || w->sh_up || w->sh_down)) return MOE_ERR_INVALID_ARG;
    const void *al16[] = {w->router_w, w->router_b, w->hash_table, w->gate,   w->up,
                          w->down,     w->sh_gate,  w->sh_up,      w->sh_down};
    for (const void *p : al16)
        if (p && !aligned(p, 16)) return MOE_ERR_INVALID_ARG;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != c->device) return MOE_ERR_INVALID_ARG;
    c->prepared = false;
    const int64_t H = sh.hidden, E = sh.n_experts, F = sh.ffn;
    const int32_t row_k = hashed && sh.table_k ? sh.table_k : sh.top_k;
    const int64_t gu = moe_matrix_bytes(sh.routed_fmt, F, H), dn = moe_matrix_bytes(sh.routed_fmt, H, F);
    const int64_t qgu = moe_matrix_bytes(MOE_FMT_Q8_32, F, H), qdn = moe_matrix_bytes(MOE_FMT_Q8_32, H, F);
    hipStream_t s = (hipStream_t)stream;
    hipError_t err = hipSuccess;
    auto step = [&](auto &&fn) {
        if (err == hipSuccess) err = fn();
    };
    // the packed banks, from the canonical ones
    auto pack = [&](void **dst, const void *src, int fmt, int64_t n, int64_t rows, int64_t cols, int64_t mb) {
        step([&] { return ctx_buffer(dst, (size_t)(n * mb)); });
        step([&] { return launch_pack(fmt, (const uint8_t *)src, (uint8_t *)*dst, n, rows, cols, s); });
    };
    pack(&c->gate, w->gate, sh.routed_fmt, E, F, H, gu);
    pack(&c->up, w->up, sh.routed_fmt, E, F, H, gu);
    pack(&c->down, w->down, sh.routed_fmt, E, H, F, dn);
    if (sh.has_shared) {
        pack(&c->sh_gate, w->sh_gate, MOE_FMT_Q8_32, 1, F, H, qgu);
        pack(&c->sh_up, w->sh_up, MOE_FMT_Q8_32, 1, F, H, qgu);
        pack(&c->sh_down, w->sh_down, MOE_FMT_Q8_32, 1, H, F, qdn);
    }
    auto copy = [&](void **dst, const void *src, size_t bytes) {
        step([&] { return ctx_buffer(dst, bytes); });
        step([&] { return hipMemcpyAsync(*dst, src, bytes, hipMemcpyDeviceToDevice, s); });
    };
    if (router) copy(&c->router_w, w->router_w, (size_t)(E * H * 4));
    if (w->router_b) {
        copy(&c->router_b, w->router_b, (size_t)E * 4);
    } else if (c->router_b) {
        (void)hipFree(c->router_b);  // no bias this time
        c->router_b = nullptr;
    }
    if (hashed) copy(&c->table, w->hash_table, (size_t)sh.vocab * row_k * 4);
    if (err != hipSuccess) return hip_status(err);
    if (hashed) {
        int32_t bad = -1;
        const int st = moe_check_hash_table((const int32_t *)c->table, sh.vocab, row_k, (int32_t)E, c->ws,
                                            c->ws_bytes, &bad, stream);
        if (st != MOE_OK) return st;
    }
    step([&] { return hipStreamSynchronize(s); });
    if (err != hipSuccess) return hip_status(err);
    c->prepared = true;
    return MOE_OK;
}

int moe_ctx_forward(moe_ctx *c, const float *x, const int32_t *token_ids, int32_t tokens, float *out,
                    void *stream) {
    if (!c) return MOE_ERR_INVALID_ARG;
    if (!c->prepared) return MOE_ERR_NOT_PREPARED;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != c->device) return MOE_ERR_INVALID_ARG;
    if (tokens > c->max_tokens) return MOE_ERR_TOO_MANY_TOKENS;
    const moe_weights w{(const float *)c->router_w, (const float *)c->router_b, (const int32_t *)c->table,
                        c->gate, c->up, c->down, c->sh_gate, c->sh_up, c->sh_down};
    return forward_impl(&c->shape, &w, x, token_ids, tokens, out, c->ws, c->ws_bytes, nullptr, stream);
}

int moe_ctx_flags(moe_ctx *c, int32_t *flags, int32_t reset, void *stream) {
    if (!c || !flags) return MOE_ERR_INVALID_ARG;
    const int st = moe_workspace_flags(c->ws, flags, stream);
    if (st != MOE_OK || !reset) return st;
    return hip_status(launch_ws_init((int32_t *)c->ws, kCtlWords, (hipStream_t)stream));
}

void moe_ctx_destroy(moe_ctx *c) {
    if (!c) return;
    ctx_free_weights(c);
    if (c->ws) (void)hipFree(c->ws);
    delete c;
}

}  // extern "C"

extern "C" {

const char *moe_stage_name(int32_t stage) {
    static const char *names[MOE_N_STAGES] = {"route", "quant", "logits", "select", "sort", "gateup", "down", "combine"};
    return (stage >= 0 && stage < MOE_N_STAGES) ? names[stage] : "?";
}

int moe_prof_create(moe_prof **prof, int32_t max_events) {
    if (!prof || max_events < 2) return MOE_ERR_INVALID_ARG;
    moe_prof *p = new moe_prof();
    p->pool.resize((size_t)max_events);
    for (auto &e : p->pool) {
        const hipError_t ce = hipEventCreate(&e);
        if (ce != hipSuccess) {
            for (auto &f : p->pool)
                if (f) hipEventDestroy(f);
            delete p;
            return hip_status(ce);
        }
    }
    *prof = p;
    return MOE_OK;
}

void moe_prof_destroy(moe_prof *prof) {
    if (!prof) return;
    if (t_prof == prof) t_prof = nullptr;
    for (auto &e : prof->pool) hipEventDestroy(e);
    delete prof;
}

int moe_prof_attach(moe_prof *prof) {
    t_prof = prof;
    return MOE_OK;
}

int moe_prof_collect(moe_prof *prof, float *stage_ms, int32_t *stage_launches, int32_t n_stages) {
    if (!prof || !stage_ms || !stage_launches || n_stages < 1) return MOE_ERR_INVALID_ARG;
    for (auto &ev : prof->used) {
        hipError_t e = hipEventSynchronize(ev.b);
        float ms = 0.0f;
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, ev.a, ev.b);
        if (e != hipSuccess) return hip_status(e);
        if (ev.stage < n_stages) {
            stage_ms[ev.stage] += ms;
            stage_launches[ev.stage] += 1;
        }
    }
    prof->used.clear();
    prof->next = 0;
    return MOE_OK;
}

}  // extern "C"
