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
// Stable counting sort of the P = T*k pairs by expert, then the work list:
// the shared expert's tokens cut into groups of at most G (full groups, so
// their workgroups start first rather than trail), followed by each
// expert's pairs cut the same way.  Up to kSortOneWg pairs it runs in ONE
// workgroup of 256 threads; larger batches take three kernels: per-chunk
// histograms, one workgroup for the prefix sums and the work list, and a
// per-chunk stable scatter.
constexpr int kSortOneWg = 4096;
constexpr int kSortChunk = 1024;  // pairs per workgroup of the histogram and scatter kernels

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

// Stable placement of the pairs [base, base + 256) (this thread: base + tid)
// given fill[e] = the next free slot of expert e in perm; advances fill.
// Within the batch a pair's rank among the same expert's pairs comes from
// the wave's ballots over the id bits, then the lower waves' counts.
__device__ __forceinline__ void place_batch(const Ws &ws, int P, int base, int *fill, int (*wcnt)[1024]) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
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
    if (valid && leader) wcnt[wave][e] = __popcll(same);
    __syncthreads();
    if (valid) {
        int r = fill[e] + rank_w;
        for (int w = 0; w < wave; ++w) r += wcnt[w][e];
        ws.perm[r] = p;
    }
    __syncthreads();
    if (valid && leader) {
        atomicAdd(&fill[e], __popcll(same));
        wcnt[wave][e] = 0;
    }
    __syncthreads();
}

// counts, offsets and the work list from the per-expert counts in sm.cnt
// (every thread of one workgroup)
__device__ void write_work_list(const Dims &d, const Ws &ws, int G, SortSmem &sm) {
    const int tid = threadIdx.x, E = d.E;
    block_excl_scan(sm.cnt, sm.off, E, sm.tmp, &sm.total);
    if (tid == 0) sm.off[E] = sm.total;
    __syncthreads();
    for (int e = tid; e < E; e += 256) {
        ws.counts[e] = sm.cnt[e];
        ws.offsets[e] = sm.off[e];
        sm.nch[e] = (sm.cnt[e] + G - 1) / G;
    }
    if (tid == 0) ws.offsets[E] = sm.off[E];
    __syncthreads();
    block_excl_scan(sm.nch, sm.gbase, E, sm.tmp, &sm.total);
    const int routed_groups = sm.total;
    const int shared_groups = d.has_shared ? (d.T + G - 1) / G : 0;
    for (int j = tid; j < shared_groups; j += 256)
        ws.groups[j] = make_int4(E, j * G, min(G, d.T - j * G), 0);
    for (int e = tid; e < E; e += 256) {
        const int c = sm.cnt[e];
        for (int j = 0; j < sm.nch[e]; ++j) {
            const int n = min(G, c - j * G);
            ws.groups[shared_groups + sm.gbase[e] + j] = make_int4(e, sm.off[e] + j * G, n, 0);
        }
    }
    if (tid == 0) ws.ctl[kCtlGroups] = routed_groups + shared_groups;
}

__device__ void sort_and_group(const Dims &d, const Ws &ws, int G, SortSmem &sm) {
    const int tid = threadIdx.x;
    const int E = d.E, P = d.T * d.k;
    for (int e = tid; e < E; e += 256) {
        sm.cnt[e] = 0;
        for (int w = 0; w < 4; ++w) sm.wcnt[w][e] = 0;
    }
    __syncthreads();
    for (int p = tid; p < P; p += 256) atomicAdd(&sm.cnt[ws.ids[p]], 1);
    __syncthreads();
    write_work_list(d, ws, G, sm);
    for (int e = tid; e < E; e += 256) sm.fill[e] = sm.off[e];
    __syncthreads();
    for (int base = 0; base < P; base += 256) place_batch(ws, P, base, sm.fill, sm.wcnt);
}

// Per-chunk expert histograms hist[chunk][e], kept in the y region of the
// workspace (unused until the down projection writes it).
__device__ __forceinline__ int *sort_hist(const Ws &ws) { return reinterpret_cast<int *>(ws.y); }

__global__ __launch_bounds__(256) void sort_hist_kernel(LayerArgs a) {
    __shared__ int cnt[1024];
    const int tid = threadIdx.x, c = blockIdx.x, E = a.d.E, P = a.d.T * a.d.k;
    for (int e = tid; e < E; e += 256) cnt[e] = 0;
    __syncthreads();
    const int end = min(P, (c + 1) * kSortChunk);
    for (int p = c * kSortChunk + tid; p < end; p += 256) atomicAdd(&cnt[a.ws.ids[p]], 1);
    __syncthreads();
    for (int e = tid; e < E; e += 256) sort_hist(a.ws)[(int64_t)c * E + e] = cnt[e];
}

// One workgroup: hist[c][e] becomes the number of expert-e pairs in chunks
// before c; the totals give counts, offsets and the work list.
__global__ __launch_bounds__(256) void sort_scan_kernel(LayerArgs a, int nchunks) {
    __shared__ SortSmem sm;
    const int tid = threadIdx.x, E = a.d.E;
    int *hist = sort_hist(a.ws);
    for (int e = tid; e < E; e += 256) {
        int run = 0;
        for (int c = 0; c < nchunks; ++c) {
            const int v = hist[(int64_t)c * E + e];
            hist[(int64_t)c * E + e] = run;
            run += v;
        }
        sm.cnt[e] = run;
    }
    __syncthreads();
    write_work_list(a.d, a.ws, a.group_tok, sm);
}

// Per chunk: each pair's slot = offset of its expert + that expert's pairs in
// earlier chunks + its rank within the chunk (stable).
__global__ __launch_bounds__(256) void sort_scatter_kernel(LayerArgs a) {
    __shared__ int fill[1024];
    __shared__ int wcnt[4][1024];
    const int tid = threadIdx.x, c = blockIdx.x, E = a.d.E, P = a.d.T * a.d.k;
    const int *hist = sort_hist(a.ws);
    for (int e = tid; e < E; e += 256) {
        fill[e] = a.ws.offsets[e] + hist[(int64_t)c * E + e];
        for (int w = 0; w < 4; ++w) wcnt[w][e] = 0;
    }
    __syncthreads();
    const int end = min(P, (c + 1) * kSortChunk);
    for (int base = c * kSortChunk; base < end; base += 256) place_batch(a.ws, end, base, fill, wcnt);
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
// 2 tokens x 2 experts.  The H-long sum is the adjacent-pair tree of the
// exact fp64 products:
//  - chunks of 128 elements of the tile's x and W rows are staged in LDS
//    (x as fp64, W as fp32, see below); the next chunk's global loads are in
//    flight while the current one is reduced;
//  - each 8-element run gives a level-3 node in registers, its level-1 nodes
//    as fma(x1, w1, x0 * w0) (both products are exact in fp64, so this
//    rounds exactly like the sum of the two products); the chunk's 16 runs
//    combine into its level-7 node by a compile-time tree;
//  - the chunk nodes are merged by a binary counter: after chunk c, merge
//    with the stacked left siblings once per trailing one bit of c.  With
//    2^m chunks this is exactly the adjacent-pair tree.  The merges are
//    selects on every level, so fewer, longer chunks cost fewer of them
//    (and fewer barriers): 128-element chunks took the 2048-token router
//    from 216 to 200 us against 64-element ones.
constexpr int kLogTile = 32;
constexpr int kLogChunk = 128;
constexpr int kLogRun = 8;      // elements per register subtree (a level-3 node)
constexpr int kLogLevels = 6;   // stack levels: up to 2^5 chunks, H <= 4096
constexpr int kLogPad = 4;      // row padding (keeps 16-byte rows aligned)

// x rows are staged already converted to fp64 (each x element meets 32 W
// rows, so converting it once saves half the conversions; every lane group of
// 16 reads the same x row, so the wider rows cost little LDS bandwidth).  W
// rows stay fp32: a wave reads 16 different W rows, and as fp64 they would
// double the LDS bytes of the operand that is not broadcast.
struct LogitsSmem {
    alignas(16) double xs[kLogTile][kLogChunk + kLogPad / 2];
    alignas(16) float wsm[kLogTile][kLogChunk + kLogPad];
};

// One thread's share of a chunk in registers: NV float4 of x rows and NV of
// W rows (32 rows of kLogChunk elements each, 16-byte pieces).
struct LogitChunkRegs {
    static constexpr int NV = kLogTile * kLogChunk / 4 / 256;
    static constexpr int PR = kLogChunk / 4;  // pieces per row
    float4 x[NV], w[NV];
    __device__ __forceinline__ void load(const float *__restrict__ x0, const float *__restrict__ w0, int H, int T,
                                         int E, int tb, int eb, int c) {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int idx = threadIdx.x + 256 * i, row = idx / PR, col = (idx % PR) * 4;
            const int t = tb + row, e = eb + row;
            // rows past T / E read row 0 of the tile and are zeroed at the store
            x[i] = *reinterpret_cast<const float4 *>(x0 + (int64_t)(t < T ? t : tb) * H + c * kLogChunk + col);
            w[i] = *reinterpret_cast<const float4 *>(w0 + (int64_t)(e < E ? e : eb) * H + c * kLogChunk + col);
        }
    }
    // (component selects: a select of whole float4 values goes through memory)
    static __device__ __forceinline__ float4 keep(bool ok, float4 v) {
        return make_float4(ok ? v.x : 0.f, ok ? v.y : 0.f, ok ? v.z : 0.f, ok ? v.w : 0.f);
    }
    __device__ __forceinline__ void store(LogitsSmem &sm, int T, int E, int tb, int eb) const {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int idx = threadIdx.x + 256 * i, row = idx / PR, col = (idx % PR) * 4;
            const float4 xv = keep(tb + row < T, x[i]);
            *reinterpret_cast<double2 *>(&sm.xs[row][col]) = make_double2((double)xv.x, (double)xv.y);
            *reinterpret_cast<double2 *>(&sm.xs[row][col + 2]) = make_double2((double)xv.z, (double)xv.w);
            *reinterpret_cast<float4 *>(&sm.wsm[row][col]) = keep(eb + row < E, w[i]);
        }
    }
};

// Level-3 nodes of the 4 (token, expert) pairs of this thread over the run
// of 8 elements at i0 of the staged chunk (W elements converted to fp64
// where they are used).
__device__ __forceinline__ void logit_run(const LogitsSmem &sm, int t0, int e0, int i0, double r[4]) {
    double xa[2][kLogRun];
    float wa[2][kLogRun];
#pragma unroll
    for (int q = 0; q < kLogRun; q += 4) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const double2 x01 = *reinterpret_cast<const double2 *>(&sm.xs[t0 + 16 * k][i0 + q]);
            const double2 x23 = *reinterpret_cast<const double2 *>(&sm.xs[t0 + 16 * k][i0 + q + 2]);
            const float4 wv = *reinterpret_cast<const float4 *>(&sm.wsm[e0 + 16 * k][i0 + q]);
            xa[k][q] = x01.x;
            xa[k][q + 1] = x01.y;
            xa[k][q + 2] = x23.x;
            xa[k][q + 3] = x23.y;
            wa[k][q] = wv.x;
            wa[k][q + 1] = wv.y;
            wa[k][q + 2] = wv.z;
            wa[k][q + 3] = wv.w;
        }
    }
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
        for (int ei = 0; ei < 2; ++ei) {
            double n1[kLogRun / 2];
#pragma unroll
            for (int j = 0; j < kLogRun / 2; ++j)
                n1[j] = __fma_rn(xa[ti][2 * j + 1], (double)wa[ei][2 * j + 1],
                                 __dmul_rn(xa[ti][2 * j], (double)wa[ei][2 * j]));
            r[ti * 2 + ei] = __dadd_rn(__dadd_rn(n1[0], n1[1]), __dadd_rn(n1[2], n1[3]));
        }
}

// Node over the N elements at i0 (N a multiple of the run) of the staged chunk.
template <int N>
__device__ __forceinline__ void logit_tree(const LogitsSmem &sm, int t0, int e0, int i0, double r[4]) {
    if constexpr (N == kLogRun) {
        logit_run(sm, t0, e0, i0, r);
    } else {
        double a[4], b[4];
        logit_tree<N / 2>(sm, t0, e0, i0, a);
        logit_tree<N / 2>(sm, t0, e0, i0 + N / 2, b);
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = __dadd_rn(a[i], b[i]);
    }
}

__global__ __launch_bounds__(256) void logits_tiled_kernel(LayerArgs a) {
    __shared__ LogitsSmem sm;
    const int H = a.d.H, T = a.d.T, E = a.d.E;
    const int tb = blockIdx.x * kLogTile, eb = blockIdx.y * kLogTile;
    const int t0 = threadIdx.x >> 4, e0 = threadIdx.x & 15;
    const int nch = H / kLogChunk;
    double st[kLogLevels][4];
#pragma unroll
    for (int l = 0; l < kLogLevels; ++l)
#pragma unroll
        for (int i = 0; i < 4; ++i) st[l][i] = 0.0;
    LogitChunkRegs cr;
    cr.load(a.x, a.wt.router_w, H, T, E, tb, eb, 0);
    for (int c = 0; c < nch; ++c) {
        __syncthreads();  // the previous chunk's reads are done
        cr.store(sm, T, E, tb, eb);
        __syncthreads();
        if (c + 1 < nch) cr.load(a.x, a.wt.router_w, H, T, E, tb, eb, c + 1);
        double v[4];
        logit_tree<kLogChunk>(sm, t0, e0, 0, v);
        const int ones = __builtin_ctz(~c);
#pragma unroll
        for (int l = 0; l < kLogLevels - 1; ++l)
            if (l < ones)
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] = __dadd_rn(st[l][i], v[i]);
#pragma unroll
        for (int l = 0; l < kLogLevels; ++l)
            if (l == ones)
#pragma unroll
                for (int i = 0; i < 4; ++i) st[l][i] = v[i];
    }
    int top = 0;
    while ((kLogChunk << top) < H) ++top;  // H / 128 = 2^top chunks: the total sits at level top
    double r[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int l = 0; l < kLogLevels; ++l)
        if (l == top)
#pragma unroll
            for (int i = 0; i < 4; ++i) r[i] = st[l][i];
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
        for (int ei = 0; ei < 2; ++ei) {
            const int t = tb + t0 + 16 * ti, e = eb + e0 + 16 * ei;
            if (t < T && e < E) {
                const int64_t i = (int64_t)t * E + e;
                const float l = (float)r[ti * 2 + ei];
                a.ws.logits[i] = l;
                score_key(l, a.wt.router_b, e, a.ws.scores + i, a.ws.keys + i);
            }
        }
}

hipError_t launch_logits(const LayerArgs &a, hipStream_t s) {
    // H a power of two (validated with the shape): 2^k whole chunks
    if (a.d.H < kLogChunk || a.d.H > (kLogChunk << (kLogLevels - 1))) return hipErrorInvalidValue;
    dim3 grid((a.d.T + kLogTile - 1) / kLogTile, (a.d.E + kLogTile - 1) / kLogTile);
    klaunch(logits_tiled_kernel, grid, dim3(256), s, a);
    return hipGetLastError();
}

__device__ __forceinline__ void select_token(const LayerArgs &a, int t, int32_t *ids, float *w, int lane) {
    const Dims &d = a.d;
    if (d.route == kRouteLearned)
        select_keys_wave(a.ws.keys + (int64_t)t * d.E, a.ws.scores + (int64_t)t * d.E, d.E, d.k, ids, w, lane);
    else
        select_hash_wave(a.token_ids, a.wt.table, t, d.vocab, d.table_k, d.E, d.k, ids, w, a.ws.ctl + kCtlFlags,
                         d.route == kRouteHashScored ? a.ws.scores + (int64_t)t * d.E : nullptr, lane);
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
    const int P = a.d.T * a.d.k;
    if (P <= kSortOneWg) {
        klaunch(sort_kernel, dim3(1), dim3(256), s, a);
        return hipGetLastError();
    }
    // the histograms (nchunks * E ints) fit the y region (P * H floats) by far
    const int nchunks = (P + kSortChunk - 1) / kSortChunk;
    klaunch(sort_hist_kernel, dim3(nchunks), dim3(256), s, a);
    klaunch(sort_scan_kernel, dim3(1), dim3(256), s, a, nchunks);
    klaunch(sort_scatter_kernel, dim3(nchunks), dim3(256), s, a);
    return hipGetLastError();
}

}  // namespace qrmoe
