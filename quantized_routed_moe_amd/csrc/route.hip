// Routing, activation quantization and token grouping for the routed-MoE
// layer.
//
//  - Router logit (learned layers): fp32 rounding of the fp64 pairwise
//    (adjacent-pair tree) sum of the exact fp64 products x_i * W_e,i.  The
//    fixed tree makes batched and single-token calls agree bit for bit, the
//    row-stable reduction order the "ds4: dfm Edition" page asks of its F32
//    router projection.
//  - Score s = sigmoid(l) in fp64 rounded to fp32; key = s + bias (fp32); the
//    k largest keys (ties: smaller expert id) are kept and weighted by
//    s / sum(kept s) ("DeepSeek V4 Flash — DFlash Integration", Model
//    Architecture and Monolithic HIP --ds4-expert-top-k).
//  - Hash layers: the token id's row of the table, weights 1/k (same page,
//    Model Architecture: first 3 layers hash-routed).
//  - Per-32-block int8 quantizer of x ("DwarfStar (ds4) — ROCm / gfx1151
//    fork", Performance optimizations: pre-quantized activation kernels).
//  - Stable sort of the (token, slot) pairs by expert and the per-expert
//    work lists the expert kernels consume ("ds4: dfm Edition": per-expert
//    worklists, expert-major schedule).
#include "dev_route.hpp"

namespace qrmoe {

// ------------------------------------------------- sort + work-list build
// Runs in ONE workgroup of 256 threads.  Stable counting sort of the P = T*k
// pairs by expert; then the work list: each expert's pairs cut into groups of
// at most G, followed by the shared expert's tokens cut the same way.
struct SortSmem {
    int cnt[1024];
    int off[1025];
    int fill[1024];
    int wcnt[4][1024];
    int nch[1024];
    int gbase[1024];
    int tmp[4];
    int total;
};

__device__ void sort_and_group(const Dims &d, const Ws &ws, int G, SortSmem &sm) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int E = d.E, P = d.T * d.k;
    for (int e = tid; e < E; e += 256) {
        sm.cnt[e] = 0;
        sm.fill[e] = 0;
        for (int w = 0; w < 4; ++w) sm.wcnt[w][e] = 0;
    }
    __syncthreads();
    for (int p = tid; p < P; p += 256) atomicAdd(&sm.cnt[ws.ids[p]], 1);
    __syncthreads();
    block_excl_scan(sm.cnt, sm.off, E, sm.tmp, &sm.total);
    if (tid == 0) sm.off[E] = sm.total;
    __syncthreads();
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int base = 0; base < P; base += 256) {
        const int p = base + tid;
        const bool valid = p < P;
        const int e = valid ? ws.ids[p] : 1023 + 1;  // sentinel never matches a real expert
        uint64_t same = ~0ull;
#pragma unroll
        for (int bit = 0; bit < 11; ++bit) {
            const uint64_t b = __ballot((e >> bit) & 1);
            same &= ((e >> bit) & 1) ? b : ~b;
        }
        const int rank_w = __popcll(same & lt_mask);
        const bool leader = rank_w == 0;
        if (valid && leader) sm.wcnt[wave][e] = __popcll(same);
        __syncthreads();
        if (valid) {
            int r = sm.fill[e] + rank_w;
            for (int w = 0; w < wave; ++w) r += sm.wcnt[w][e];
            ws.perm[sm.off[e] + r] = p;
        }
        __syncthreads();
        if (valid && leader) {
            atomicAdd(&sm.fill[e], __popcll(same));
            sm.wcnt[wave][e] = 0;
        }
        __syncthreads();
    }
    for (int e = tid; e < E; e += 256) {
        ws.counts[e] = sm.cnt[e];
        ws.offsets[e] = sm.off[e];
        sm.nch[e] = (sm.cnt[e] + G - 1) / G;
    }
    if (tid == 0) ws.offsets[E] = sm.off[E];
    __syncthreads();
    block_excl_scan(sm.nch, sm.gbase, E, sm.tmp, &sm.total);
    const int routed_groups = sm.total;
    for (int e = tid; e < E; e += 256) {
        const int c = sm.cnt[e];
        for (int j = 0; j < sm.nch[e]; ++j) {
            const int n = min(G, c - j * G);
            ws.groups[sm.gbase[e] + j] = make_int4(e, sm.off[e] + j * G, n, 0);
        }
    }
    const int shared_groups = d.has_shared ? (d.T + G - 1) / G : 0;
    for (int j = tid; j < shared_groups; j += 256)
        ws.groups[routed_groups + j] = make_int4(E, j * G, min(G, d.T - j * G), 0);
    if (tid == 0) ws.ctl[kCtlGroups] = routed_groups + shared_groups;
}

// --------------------------------------------------- batched (large T)
__global__ __launch_bounds__(256) void quant_kernel(LayerArgs a) {
    const int nblk = a.d.T * (a.d.H / 32);
    for (int b = blockIdx.x * 256 + threadIdx.x; b < nblk; b += gridDim.x * 256)
        quant_one_block(a.x, a.ws.xq, a.ws.xd, a.d.fmt == kFmtQ2 ? a.ws.xs16 : nullptr, b);
}

hipError_t launch_quant(const LayerArgs &a, hipStream_t s) {
    int blocks = (a.d.T * (a.d.H / 32) + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    klaunch(quant_kernel, dim3(blocks), dim3(256), s, a);
    return hipGetLastError();
}

// Tiled logits: a workgroup computes a 32-token x 32-expert tile, each thread
// 2 tokens x 2 experts.  The H-long sum is the adjacent-pair tree: chunks of
// 64 elements staged in LDS give the level-6 nodes, and the chunk loop is a
// compile-time recursion that combines chunk sums in the same tree order.
constexpr int kLogTile = 32;
constexpr int kLogChunk = 64;

struct LogitsSmem {
    float xs[kLogTile][kLogChunk + 4];
    float wsm[kLogTile][kLogChunk + 4];
};

template <int N>
__device__ __forceinline__ void tile_prod_tree(const LogitsSmem &sm, int t0, int e0, int i0, double r[4]) {
    if constexpr (N == 4) {
        const float4 x0 = *reinterpret_cast<const float4 *>(&sm.xs[t0][i0]);
        const float4 x1 = *reinterpret_cast<const float4 *>(&sm.xs[t0 + 16][i0]);
        const float4 w0 = *reinterpret_cast<const float4 *>(&sm.wsm[e0][i0]);
        const float4 w1 = *reinterpret_cast<const float4 *>(&sm.wsm[e0 + 16][i0]);
        const float xa[2][4] = {{x0.x, x0.y, x0.z, x0.w}, {x1.x, x1.y, x1.z, x1.w}};
        const float wa[2][4] = {{w0.x, w0.y, w0.z, w0.w}, {w1.x, w1.y, w1.z, w1.w}};
#pragma unroll
        for (int ti = 0; ti < 2; ++ti)
#pragma unroll
            for (int ei = 0; ei < 2; ++ei) r[ti * 2 + ei] = prod_tree<4>(xa[ti], wa[ei]);
    } else {
        double a[4], b[4];
        tile_prod_tree<N / 2>(sm, t0, e0, i0, a);
        tile_prod_tree<N / 2>(sm, t0, e0, i0 + N / 2, b);
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = a[i] + b[i];
    }
}

// Stage chunk c0 (64 elements) of the tile's 32 x-rows and 32 W-rows into LDS.
__device__ __forceinline__ void stage_logit_chunk(LogitsSmem &sm, const float *__restrict__ x,
                                                  const float *__restrict__ w, int H, int T, int E, int tb, int eb,
                                                  int c0) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int idx = tid + 256 * i, row = idx >> 4, col = (idx & 15) * 4;
        const int t = tb + row, e = eb + row;
        float4 xv = make_float4(0.f, 0.f, 0.f, 0.f), wv = xv;
        if (t < T) xv = *reinterpret_cast<const float4 *>(x + (int64_t)t * H + c0 * kLogChunk + col);
        if (e < E) wv = *reinterpret_cast<const float4 *>(w + (int64_t)e * H + c0 * kLogChunk + col);
        *reinterpret_cast<float4 *>(&sm.xs[row][col]) = xv;
        *reinterpret_cast<float4 *>(&sm.wsm[row][col]) = wv;
    }
}

// The chunk sums (level-6 nodes of the tree) are merged with a binary
// counter: after chunk c, merge with the stacked left siblings once per
// trailing one bit of c.  With 2^m chunks this yields exactly the
// adjacent-pair tree; the merges are uniform branches, no dynamic indexing.
__global__ __launch_bounds__(256) void logits_tiled_kernel(LayerArgs a) {
    __shared__ LogitsSmem sm;
    const int H = a.d.H;
    const int tb = blockIdx.x * kLogTile, eb = blockIdx.y * kLogTile;
    const int nch = H / kLogChunk;
    double st[7][4];
#pragma unroll
    for (int l = 0; l < 7; ++l)
#pragma unroll
        for (int i = 0; i < 4; ++i) st[l][i] = 0.0;
    for (int c = 0; c < nch; ++c) {
        __syncthreads();
        stage_logit_chunk(sm, a.x, a.wt.router_w, H, a.d.T, a.d.E, tb, eb, c);
        __syncthreads();
        double v[4];
        tile_prod_tree<kLogChunk>(sm, threadIdx.x >> 4, threadIdx.x & 15, 0, v);
        const int ones = __builtin_ctz(~c);
#pragma unroll
        for (int l = 0; l < 6; ++l)
            if (l < ones)
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] = st[l][i] + v[i];
#pragma unroll
        for (int l = 0; l < 7; ++l)
            if (l == ones)
#pragma unroll
                for (int i = 0; i < 4; ++i) st[l][i] = v[i];
    }
    int top = 0;
    while ((1 << top) < nch) ++top;  // nch = 2^top, the total sits at level top
    double r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = 0.0;
#pragma unroll
    for (int l = 0; l < 7; ++l)
        if (l == top)
#pragma unroll
            for (int i = 0; i < 4; ++i) r[i] = st[l][i];
    const int tl = threadIdx.x >> 4, el = threadIdx.x & 15;
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
        for (int ei = 0; ei < 2; ++ei) {
            const int t = tb + tl + 16 * ti, e = eb + el + 16 * ei;
            if (t < a.d.T && e < a.d.E) {
                const int64_t i = (int64_t)t * a.d.E + e;
                const float l = (float)r[ti * 2 + ei];
                a.ws.logits[i] = l;
                score_key(l, a.wt.router_b, e, a.ws.scores + i, a.ws.keys + i);
            }
        }
}

hipError_t launch_logits(const LayerArgs &a, hipStream_t s) {
    if (a.d.H < kLogChunk || a.d.H > kLogChunk * 64) return hipErrorInvalidValue;
    dim3 grid((a.d.T + kLogTile - 1) / kLogTile, (a.d.E + kLogTile - 1) / kLogTile);
    klaunch(logits_tiled_kernel, grid, dim3(256), s, a);
    return hipGetLastError();
}

__device__ __forceinline__ void select_token(const LayerArgs &a, int t, int32_t *ids, float *w, int lane) {
    const Dims &d = a.d;
    if (d.route == kRouteLearned)
        select_keys_wave(a.ws.keys + (int64_t)t * d.E, a.ws.scores + (int64_t)t * d.E, d.E, d.k, ids, w, lane);
    else
        select_hash_wave(a.token_ids, a.wt.table, t, d.vocab, d.E, d.k, ids, w, a.ws.ctl + kCtlFlags, lane);
}

__global__ __launch_bounds__(256) void select_kernel(LayerArgs a) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= a.d.T) return;
    select_token(a, t, a.ws.ids + t * a.d.k, a.ws.w + t * a.d.k, lane);
}


hipError_t launch_select(const LayerArgs &a, hipStream_t s) {
    klaunch(select_kernel, dim3((a.d.T + 3) / 4), dim3(256), s, a);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void sort_kernel(LayerArgs a) {
    __shared__ SortSmem sm;
    sort_and_group(a.d, a.ws, a.group_tok, sm);
}

hipError_t launch_sort(const LayerArgs &a, hipStream_t s) {
    klaunch(sort_kernel, dim3(1), dim3(256), s, a);
    return hipGetLastError();
}

}  // namespace qrmoe
