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
#include <climits>
#include <cmath>

#include "common.hpp"

namespace qrmoe {

// ------------------------------------------------------------ quantizer
// One thread quantizes one 32-block of a row of H floats.
__device__ __forceinline__ void quant_one_block(const float *__restrict__ x, int8_t *__restrict__ xq,
                                                float *__restrict__ xd, int32_t *__restrict__ xs16, int64_t blk) {
    const float4 *src = reinterpret_cast<const float4 *>(x + blk * 32);
    float v[32];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float4 f = src[i];
        v[4 * i] = f.x;
        v[4 * i + 1] = f.y;
        v[4 * i + 2] = f.z;
        v[4 * i + 3] = f.w;
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    const float d = quant_scale(amax);
    const float inv = d > 0.0f ? 1.0f / d : 0.0f;
    uint32_t words[8];
    int s0 = 0, s1 = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t wv = 0;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            int q = quant_code(v[4 * i + c], inv);
            if (i < 4) s0 += q; else s1 += q;
            wv |= ((uint32_t)q & 0xffu) << (8 * c);
        }
        words[i] = wv;
    }
    uint4 *dst = reinterpret_cast<uint4 *>(xq + blk * 32);
    dst[0] = make_uint4(words[0], words[1], words[2], words[3]);
    dst[1] = make_uint4(words[4], words[5], words[6], words[7]);
    xd[blk] = d;
    if (xs16) {
        xs16[2 * blk] = s0;
        xs16[2 * blk + 1] = s1;
    }
}

// --------------------------------------------------------- router logits
// Pairwise fp64 tree of n = N products held in registers.  Level 1 may be
// contracted to fma(a1, b1, a0*b0): both products are exact in fp64, so the
// fused and unfused forms round identically.
template <int N>
__device__ __forceinline__ double prod_tree(const float *a, const float *b) {
    if constexpr (N == 1) {
        return (double)a[0] * (double)b[0];
    } else {
        return prod_tree<N / 2>(a, b) + prod_tree<N / 2>(a + N / 2, b + N / 2);
    }
}

template <int N>
__device__ __forceinline__ double dtree(const double *v) {
    if constexpr (N == 1) {
        return v[0];
    } else {
        return dtree<N / 2>(v) + dtree<N / 2>(v + N / 2);
    }
}

// Pairwise sum over one lane's aligned segment of SEG elements.
template <int SEG>
__device__ __forceinline__ double segment_tree(const float *__restrict__ xa, const float *__restrict__ wa) {
    constexpr int CH = SEG < 16 ? SEG : 16;
    constexpr int NC = SEG / CH;
    double part[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        float xv[CH], wv[CH];
        if constexpr (CH % 4 == 0) {
#pragma unroll
            for (int i = 0; i < CH / 4; ++i) {
                float4 a = reinterpret_cast<const float4 *>(xa + c * CH)[i];
                float4 b = reinterpret_cast<const float4 *>(wa + c * CH)[i];
                xv[4 * i] = a.x; xv[4 * i + 1] = a.y; xv[4 * i + 2] = a.z; xv[4 * i + 3] = a.w;
                wv[4 * i] = b.x; wv[4 * i + 1] = b.y; wv[4 * i + 2] = b.z; wv[4 * i + 3] = b.w;
            }
        } else {
#pragma unroll
            for (int i = 0; i < CH; ++i) {
                xv[i] = xa[c * CH + i];
                wv[i] = wa[c * CH + i];
            }
        }
        part[c] = prod_tree<CH>(xv, wv);
    }
    return dtree<NC>(part);
}

// One wave computes one logit: lane l owns elements [l*SEG, (l+1)*SEG); the
// segment sums are combined by an xor butterfly whose pairing (1, 2, 4, ...)
// is the upper part of the same adjacent-pair tree.
template <int H>
__device__ __forceinline__ float wave_logit(const float *__restrict__ xrow, const float *__restrict__ wrow, int lane) {
    constexpr int SEG = H / 64;
    double v = segment_tree<SEG>(xrow + lane * SEG, wrow + lane * SEG);
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o);
    return (float)v;
}

// ------------------------------------------------------------- selection
__device__ __forceinline__ float score_of(float l) { return (float)(1.0 / (1.0 + exp(-(double)l))); }

// One wave selects the top-k experts of one token.
__device__ void select_learned_wave(const float *__restrict__ lrow, const float *__restrict__ bias, int E, int k,
                                    int32_t *ids_out, float *w_out, int lane) {
    constexpr int MAXPER = 16;  // E <= 1024
    const int per = (E + 63) / 64;
    float key[MAXPER], sc[MAXPER];
#pragma unroll
    for (int i = 0; i < MAXPER; ++i) {
        key[i] = -INFINITY;
        sc[i] = 0.0f;
        const int e = lane + 64 * i;
        if (i < per && e < E) {
            sc[i] = score_of(lrow[e]);
            key[i] = sc[i] + (bias ? bias[e] : 0.0f);
        }
    }
    int sel_e[8];
    float sel_s[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        sel_e[j] = 0;
        sel_s[j] = 0.0f;
        if (j < k) {
            float bk = -INFINITY;
            int be = INT_MAX;
#pragma unroll
            for (int i = 0; i < MAXPER; ++i) {
                const int e = lane + 64 * i;
                if (i < per && e < E && (key[i] > bk || (key[i] == bk && e < be))) {
                    bk = key[i];
                    be = e;
                }
            }
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) {
                float ok = __shfl_xor(bk, o);
                int oe = __shfl_xor(be, o);
                if (ok > bk || (ok == bk && oe < be)) {
                    bk = ok;
                    be = oe;
                }
            }
            const int owner = be & 63, slot = be >> 6;
            float mine = 0.0f;
#pragma unroll
            for (int i = 0; i < MAXPER; ++i)
                if (i == slot) {
                    mine = sc[i];
                    if (lane == owner) key[i] = -INFINITY;
                }
            sel_s[j] = __shfl(mine, owner);
            sel_e[j] = be;
        }
    }
    float S = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
        if (j < k) S += sel_s[j];
    if (lane == 0) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (j < k) {
                ids_out[j] = sel_e[j];
                w_out[j] = sel_s[j] / S;
            }
    }
}

__device__ void select_hash_wave(const int32_t *__restrict__ token_ids, const int32_t *__restrict__ table, int t,
                                 int vocab, int E, int k, int32_t *ids_out, float *w_out, int32_t *flags, int lane) {
    int id = token_ids[t];
    if (id < 0 || id >= vocab) {
        if (lane == 0) atomicOr(flags, 1);
        id = 0;
    }
    if (lane < k) {
        int e = table[(int64_t)id * k + lane];
        if (e < 0 || e >= E) {
            atomicOr(flags, 2);
            e = 0;
        }
        ids_out[lane] = e;
        w_out[lane] = 1.0f / (float)k;
    }
}

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

// ------------------------------------------------------ decode routing
// Kernel 1 (many workgroups): quantize x; learned layers also compute the
// T*E logits, one wave per logit.  Kernel 2 (one workgroup): select, sort,
// build the work list.  The kernel boundary orders the two; no device-scope
// fences are used (on this multi-XCD part they write back and invalidate L2).
template <int H>
__global__ __launch_bounds__(256) void route_logits_kernel(LayerArgs a) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const Dims &d = a.d;
    const int nblk = d.T * (H / 32);
    for (int b = blockIdx.x * 256 + tid; b < nblk; b += gridDim.x * 256)
        quant_one_block(a.x, a.ws.xq, a.ws.xd, d.fmt == kFmtQ2 ? a.ws.xs16 : nullptr, b);
    if (d.route == kRouteLearned) {
        const int nlog = d.T * d.E;
        for (int le = blockIdx.x * 4 + wave; le < nlog; le += gridDim.x * 4) {
            const int t = le / d.E, e = le % d.E;
            float l = wave_logit<H>(a.x + (int64_t)t * H, a.wt.router_w + (int64_t)e * H, lane);
            if (lane == 0) a.ws.logits[le] = l;
        }
    }
}

__global__ __launch_bounds__(256) void select_sort_kernel(LayerArgs a) {
    __shared__ SortSmem sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const Dims &d = a.d;
    for (int t = wave; t < d.T; t += 4) {
        if (d.route == kRouteLearned)
            select_learned_wave(a.ws.logits + (int64_t)t * d.E, a.wt.router_b, d.E, d.k, a.ws.ids + t * d.k,
                                a.ws.w + t * d.k, lane);
        else
            select_hash_wave(a.token_ids, a.wt.table, t, d.vocab, d.E, d.k, a.ws.ids + t * d.k, a.ws.w + t * d.k,
                             a.ws.ctl + kCtlFlags, lane);
    }
    __syncthreads();
    sort_and_group(d, a.ws, a.group_tok, sm);
}

template <int H>
static hipError_t launch_route_logits_h(const LayerArgs &a, hipStream_t s) {
    const int work_waves = a.d.route == kRouteLearned ? a.d.T * a.d.E : 0;
    int blocks = (work_waves + 3) / 4;
    const int qblocks = (a.d.T * (H / 32) + 255) / 256;
    if (blocks < qblocks) blocks = qblocks;
    if (blocks > 2048) blocks = 2048;
    if (blocks < 1) blocks = 1;
    route_logits_kernel<H><<<dim3(blocks), dim3(256), 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_route_decode(const LayerArgs &a, hipStream_t s) {
    hipError_t err;
    switch (a.d.H) {
        case 128: err = launch_route_logits_h<128>(a, s); break;
        case 256: err = launch_route_logits_h<256>(a, s); break;
        case 512: err = launch_route_logits_h<512>(a, s); break;
        case 1024: err = launch_route_logits_h<1024>(a, s); break;
        case 2048: err = launch_route_logits_h<2048>(a, s); break;
        case 4096: err = launch_route_logits_h<4096>(a, s); break;
        default: return hipErrorInvalidValue;
    }
    return err;
}

hipError_t launch_select_sort(const LayerArgs &a, hipStream_t s) {
    select_sort_kernel<<<dim3(1), dim3(256), 0, s>>>(a);
    return hipGetLastError();
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
    quant_kernel<<<dim3(blocks), dim3(256), 0, s>>>(a);
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
            if (t < a.d.T && e < a.d.E) a.ws.logits[(int64_t)t * a.d.E + e] = (float)r[ti * 2 + ei];
        }
}

hipError_t launch_logits(const LayerArgs &a, hipStream_t s) {
    if (a.d.H < kLogChunk || a.d.H > kLogChunk * 64) return hipErrorInvalidValue;
    dim3 grid((a.d.T + kLogTile - 1) / kLogTile, (a.d.E + kLogTile - 1) / kLogTile);
    logits_tiled_kernel<<<grid, dim3(256), 0, s>>>(a);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void select_kernel(LayerArgs a) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= a.d.T) return;
    if (a.d.route == kRouteLearned)
        select_learned_wave(a.ws.logits + (int64_t)t * a.d.E, a.wt.router_b, a.d.E, a.d.k, a.ws.ids + t * a.d.k,
                            a.ws.w + t * a.d.k, lane);
    else
        select_hash_wave(a.token_ids, a.wt.table, t, a.d.vocab, a.d.E, a.d.k, a.ws.ids + t * a.d.k, a.ws.w + t * a.d.k,
                         a.ws.ctl + kCtlFlags, lane);
}

hipError_t launch_select(const LayerArgs &a, hipStream_t s) {
    select_kernel<<<dim3((a.d.T + 3) / 4), dim3(256), 0, s>>>(a);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void sort_kernel(LayerArgs a) {
    __shared__ SortSmem sm;
    sort_and_group(a.d, a.ws, a.group_tok, sm);
}

hipError_t launch_sort(const LayerArgs &a, hipStream_t s) {
    sort_kernel<<<dim3(1), dim3(256), 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace qrmoe
