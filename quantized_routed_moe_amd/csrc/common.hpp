// Internal definitions shared by the HIP kernels and the host dispatcher of
// the routed-MoE layer (gfx950, wave64).  Not part of the public ABI.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qrmoe {

typedef __attribute__((address_space(3))) void *lds_ptr;  // LDS address for global->LDS loads

constexpr int kWave = 64;
constexpr int kThreads = 256;       // every kernel runs 4 waves per workgroup
constexpr int kVecTok = 8;          // tokens per work group of the VALU expert kernels
constexpr int kVecRows = 32;        // weight rows per workgroup of the VALU expert kernels (= one h block)
constexpr int kDecodeMaxT = 32;     // batches up to this size take the decode path
constexpr int kFmtQ8 = 1, kFmtQ2 = 2;
constexpr int kRouteLearned = 1, kRouteHash = 2, kRouteHashScored = 3;

// ctl[] words of the workspace
enum : int { kCtlGroups = 1, kCtlFlags = 2, kCtlMagic = 3 };
constexpr int kCtlWords = 64;
constexpr int32_t kWsMagic = 0x4F4D5251;  // set by moe_workspace_init

// ------------------------------------------------------------------------
// Packed weight layouts (what moe_pack_weights writes; same byte count as the
// canonical AoS blocks):
//   Q8 matrix [R][K]: int8 codes plane R*K (row-major), then fp16 scale plane
//                     R*(K/32) (row-major).
//   Q2 matrix [R][K]: codes plane R*K/4 bytes, then scale/min plane R*K/16
//                     bytes (same nibble order as canonical sm), then the
//                     (fp16 d, fp16 dmin) plane R*(K/256)*4 bytes.  In the
//                     codes plane each 32-bit word holds one 16-weight
//                     subblock: byte c, bits [2s, 2s+2) hold the code of
//                     weight 4s + c, so (word >> 2s) & 0x03030303 yields the
//                     codes of weights 4s..4s+3 in bytes 0..3.
// ------------------------------------------------------------------------
__host__ __device__ inline int64_t q8_bytes(int64_t R, int64_t K) { return R * K + R * (K / 32) * 2; }
__host__ __device__ inline int64_t q2_bytes(int64_t R, int64_t K) { return R * K / 4 + R * K / 16 + R * (K / 256) * 4; }
__host__ __device__ inline int64_t mat_bytes(int fmt, int64_t R, int64_t K) {
    return fmt == kFmtQ8 ? q8_bytes(R, K) : q2_bytes(R, K);
}

struct Dims {
    int32_t T, H, E, k, F, has_shared, fmt, route, vocab;
    int32_t P;  // pairs including the shared expert's: T*k + T*has_shared
    int32_t table_k;  // entries per hash-table row (>= k)
    int32_t table_logits;  // score-weighted hash, decode sizes, no debug copies: only the table's logits
};

// Workspace pointers (device).
struct Ws {
    int32_t *ctl;
    float *logits;
    int32_t *ids;
    float *w;
    int8_t *xq;
    float *xd;
    int32_t *xs16;   // [T][H/16] sums of xq over 16-subblocks (Q2 experts)
    int32_t *counts;
    int32_t *offsets;
    int32_t *perm;
    int4 *groups;    // {expert (E = shared), first index into perm (or first token), count, first pair}
    int8_t *hq;
    float *hd;
    float *y;        // [P][H] weighted expert outputs (w already applied)
    float *scores;   // [T][E] sigmoid scores
    float *keys;     // [T][E] selection keys (score + bias)
    int32_t *hs16;   // [P][F/16] sums of hq over 16-subblocks (2-bit down GEMM; batched path only)
};

struct Weights {
    const float *router_w, *router_b;
    const int32_t *table;
    const uint8_t *gate, *up, *down;
    const uint8_t *sh_gate, *sh_up, *sh_down;
};

struct Dump {
    int32_t *gate_sums, *up_sums, *down_sums;
    int32_t stride;           // sampled rows: r % stride == 0
    int32_t pitch_gu, pitch_dn;  // int32 entries per sampled row (H/32 or H/16, F/32 or F/16)
};

struct LayerArgs {
    Dims d;
    Weights wt;
    Ws ws;
    Dump dump;
    const float *x;
    const int32_t *token_ids;
    float *out;
    int32_t group_tok;  // tokens per group in the work list (kVecTok or the MFMA tile)
};

// ------------------------------------------------------------------ device
__device__ __forceinline__ float f16_to_f32(uint16_t h) { return __half2float(__ushort_as_half(h)); }

// ------------------------------------------------ cross-lane butterflies
// Reductions over aligned groups of W lanes (W a power of two up to 64) as an
// xor butterfly, smallest distance first, every lane of a group ending with
// the same value.  Partner values come from registers, not from LDS:
//  - xor 1, xor 2: DPP quad permutations [1,0,3,2] and [2,3,0,1];
//  - xor 4, xor 8: DPP half-row mirror (l <-> 7-l) and row mirror
//    (l <-> 15-l).  After the previous steps every lane of a 4-lane (8-lane)
//    group holds the same value, so the mirror partner's value equals the
//    xor-4 (xor-8) partner's;
//  - xor 16, xor 32: v_permlane16_swap / v_permlane32_swap, which exchange
//    the odd 16-lane rows (upper 32 lanes) of one copy with the even rows
//    (lower 32 lanes) of another, so lane l sees lane l^16 (l^32).
// Each step combines the two values commutatively, so partners compute the
// same bits.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
}

// The two 32-bit values of the butterfly pair at distance D, as (this lane's,
// partner's) for D <= 8 and as (lower lane's, upper lane's) for D = 16, 32.
template <int D>
__device__ __forceinline__ void bfly_pair_u32(uint32_t v, uint32_t &a, uint32_t &b) {
    if constexpr (D <= 8) {
        constexpr int ctrl = D == 1 ? 0xB1 : D == 2 ? 0x4E : D == 4 ? 0x141 : 0x140;
        a = v;
        b = dpp_u32<ctrl>(v);
    } else if constexpr (D == 16) {
        const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        a = p[0];
        b = p[1];
    } else {
        static_assert(D == 32, "butterfly distance");
        const auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        a = p[0];
        b = p[1];
    }
}

template <int D, class Op>
__device__ __forceinline__ float bfly_step(float v, Op op) {
    uint32_t a, b;
    bfly_pair_u32<D>(__float_as_uint(v), a, b);
    return op(__uint_as_float(a), __uint_as_float(b));
}

template <int D, class Op>
__device__ __forceinline__ uint32_t bfly_step(uint32_t v, Op op) {
    uint32_t a, b;
    bfly_pair_u32<D>(v, a, b);
    return op(a, b);
}

template <int D, class Op>
__device__ __forceinline__ double bfly_step(double v, Op op) {
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    uint32_t la, lb, ha, hb;
    bfly_pair_u32<D>((uint32_t)u, la, lb);
    bfly_pair_u32<D>((uint32_t)(u >> 32), ha, hb);
    return op(__longlong_as_double((long long)(((uint64_t)ha << 32) | la)),
              __longlong_as_double((long long)(((uint64_t)hb << 32) | lb)));
}

template <int W, class T, class Op>
__device__ __forceinline__ T group_reduce(T v, Op op) {
    static_assert(W >= 1 && W <= 64 && (W & (W - 1)) == 0, "group width");
    if constexpr (W >= 2) v = bfly_step<1>(v, op);
    if constexpr (W >= 4) v = bfly_step<2>(v, op);
    if constexpr (W >= 8) v = bfly_step<4>(v, op);
    if constexpr (W >= 16) v = bfly_step<8>(v, op);
    if constexpr (W >= 32) v = bfly_step<16>(v, op);
    if constexpr (W >= 64) v = bfly_step<32>(v, op);
    return v;
}

template <int W>
__device__ __forceinline__ float group_sum(float v) {
    return group_reduce<W>(v, [](float a, float b) { return a + b; });
}

// fp64 sum over the whole wave: the adjacent-pair tree of the 64 lane values
// (lane l's value is leaf l).
__device__ __forceinline__ double wave_sum_f64(double v) {
    return group_reduce<64>(v, [](double a, double b) { return a + b; });
}

template <int W>
__device__ __forceinline__ float group_max(float v) {
    return group_reduce<W>(v, [](float a, float b) { return fmaxf(a, b); });
}

__device__ __forceinline__ int sdot4(int a, int b, int c) { return __builtin_amdgcn_sdot4(a, b, c, false); }

typedef int i32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming load (each weight byte is used once per call).
__device__ __forceinline__ int4 load_stream16(const void *p) {
    const i32x4 v = __builtin_nontemporal_load(reinterpret_cast<const i32x4 *>(p));
    return make_int4(v.x, v.y, v.z, v.w);
}

// ------------------------------------------- direct global -> LDS staging
// buffer_load_dword{,x4} ... lds writes lane l's 4 (16) bytes to LDS at
// base + 4l (16l): one wave fills 256 B (1 KB) of LDS with no VGPRs and no
// ds_write.  The loads go through a buffer descriptor whose record count is
// the source tensor's size, so an offset past it reads zeros instead of
// touching other memory.  A wave waits for its own loads of a chunk with an
// explicit vmcnt count, then a barrier makes every wave's loads visible.
typedef __attribute__((address_space(3))) void *lds_ptr;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *base, uint32_t bytes) {
    // raw byte buffer: stride 0, range check against `bytes`, 32-bit data format
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void *lds, uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)lds, 16, (int)voff, 0, 0, 0);
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, void *lds, uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)lds, 4, (int)voff, 0, 0, 0);
}
template <int N>
__device__ __forceinline__ void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Per-32-block quantizer: d = amax/127, q = clamp(rint(v * (1/d)), +-127);
// amax == 0 gives d = 0, q = 0.  Same definition as the layer's activation
// quantizer for x and h.
__device__ __forceinline__ float quant_scale(float amax) { return amax / 127.0f; }
__device__ __forceinline__ int quant_code(float v, float inv) {
    float r = rintf(v * inv);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (int)r;
}

// One 32-block of fp32 values held in registers, then quantized: codes,
// scale and (for Q2 experts) the two 16-subblock code sums.
struct QBlock {
    float v[32];
    __device__ __forceinline__ void load(const float *__restrict__ x, int64_t blk) {
        const float4 *src = reinterpret_cast<const float4 *>(x + blk * 32);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float4 f = src[i];
            v[4 * i] = f.x;
            v[4 * i + 1] = f.y;
            v[4 * i + 2] = f.z;
            v[4 * i + 3] = f.w;
        }
    }
    // codes -> xq[blk*32 ..], scale -> xd[blk], (xs16) code sums of the two 16-halves
    __device__ __forceinline__ void store(int8_t *__restrict__ xq, float *__restrict__ xd, int32_t *__restrict__ xs16,
                                         int64_t blk) const {
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
                const int q = quant_code(v[4 * i + c], inv);
                if (i < 4) s0 += q;
                else s1 += q;
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
};

// One thread quantizes the 32-block `blk` of x into codes, scale and (when
// xs16 is given) the two 16-subblock code sums.
__device__ __forceinline__ void quant_one_block(const float *__restrict__ x, int8_t *__restrict__ xq,
                                                float *__restrict__ xd, int32_t *__restrict__ xs16, int64_t blk) {
    QBlock q;
    q.load(x, blk);
    q.store(xq, xd, xs16, blk);
}

// Exclusive scan of n <= 1024 ints in LDS (in place into `out`), 256 threads.
__device__ inline void block_excl_scan(const int *in, int *out, int n, int *tmp_wave /*[4]*/, int *total) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int v[4], s = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int idx = tid * 4 + i;
        v[i] = idx < n ? in[idx] : 0;
        s += v[i];
    }
    int inc = s;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int t = __shfl_up(inc, o);
        if (lane >= o) inc += t;
    }
    if (lane == 63) tmp_wave[wave] = inc;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave; ++w) base += tmp_wave[w];
    int run = base + inc - s;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int idx = tid * 4 + i;
        if (idx < n) out[idx] = run;
        run += v[i];
    }
    if (tid == 255) *total = run;
    __syncthreads();
}

// ------------------------------------------------------------- launchers
// While a stage profiler is attached to the calling thread and a forward call
// runs one of its stages, every kernel launch takes its own pair of events
// from the profiler (api.cpp) and goes through hipExtLaunchKernelGGL, whose
// events take the kernel's own start and end times (no dispatch latency).
bool next_launch_events(hipEvent_t *start, hipEvent_t *stop);

template <class... KArgs, class... Args>
void klaunch(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t s, Args... args) {
    hipEvent_t start, stop;
    if (next_launch_events(&start, &stop))
        hipExtLaunchKernelGGL(kernel, grid, block, 0, s, start, stop, 0, args...);
    else
        kernel<<<grid, block, 0, s>>>(args...);
}

hipError_t launch_pack(int fmt, const uint8_t *canon, uint8_t *packed, int64_t n_mats, int64_t rows, int64_t cols,
                       hipStream_t s);
hipError_t launch_check_table(const int32_t *table, int32_t vocab, int32_t k, int32_t E, int32_t *result,
                              hipStream_t s);
hipError_t launch_ws_init(int32_t *ctl, int64_t n_words, hipStream_t s);
hipError_t launch_decode_front(const LayerArgs &a, hipStream_t s);
hipError_t launch_decode_select(const LayerArgs &a, hipStream_t s);
hipError_t launch_select_sort(const LayerArgs &a, hipStream_t s);
hipError_t launch_decode_gateup1(const LayerArgs &a, bool dump, hipStream_t s);
hipError_t launch_decode_down1(const LayerArgs &a, bool dump, hipStream_t s);
hipError_t launch_quant(const LayerArgs &a, hipStream_t s);
hipError_t launch_logits(const LayerArgs &a, hipStream_t s);
hipError_t launch_select(const LayerArgs &a, hipStream_t s);
hipError_t launch_sort(const LayerArgs &a, hipStream_t s);
hipError_t launch_gateup_vec(const LayerArgs &a, int max_groups, bool dump, hipStream_t s);
hipError_t launch_down_vec(const LayerArgs &a, int max_groups, bool dump, hipStream_t s);
hipError_t launch_combine(const LayerArgs &a, hipStream_t s);
hipError_t launch_gateup_mfma(const LayerArgs &a, int max_tiles, bool dump, hipStream_t s);
hipError_t launch_down_mfma(const LayerArgs &a, int max_tiles, bool dump, hipStream_t s);

}  // namespace qrmoe
