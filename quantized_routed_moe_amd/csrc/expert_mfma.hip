// Grouped int8 MFMA GEMMs of the expert FFN for batched tokens (Q8_32
// weights): the token sort gives each expert a list of pairs, cut into tiles
// of 64 (the expert-tile prefill kernels of "DwarfStar (ds4) — ROCm / gfx1151
// fork", Performance optimizations, moe_gate_up_mid_expert_tile* /
// moe_down_expert_tile*; the expert-major schedule of "ds4: dfm Edition",
// About this fork).  Every 32-element quantization block is one
// v_mfma_i32_32x32x32_i8 (K = 32 = one block), so the MFMA returns the exact
// int32 block sum of every (pair, row); those are scaled by the two block
// scales and accumulated in fp32 in block order.  The scale products
// dx[t] * dw[r] of a 32x32 tile come from one v_mfma_f32_32x32x1_2b_f32 (two
// outer products per instruction, exactly rounded), which leaves one
// conversion and one fma per output per block on the VALU.
//
// Lane layouts (wave64): v_mfma_i32_32x32x32_i8 takes from lane l the bytes
// [16*(l/32), +16) of the block for A row l%32 and B column l%32; register i
// of lane l holds C[8*(i/4) + 4*(l/32) + i%4][l%32].  The 2b outer product
// takes A[j][l%32] and B[j][l%32] with j = l/32 and puts product j in
// registers [16j, 16j+16) with the same row/column mapping.
//
// Workgroup: 4 waves as 2 (pairs) x 2 (columns), each wave 32 x 32; tile =
// 64 pairs x 64 columns.  K runs in chunks of 4 blocks staged in LDS (padded
// rows), the next chunk's global loads held in registers meanwhile.
//
//  gate/up  B = 64 gate rows + 64 up rows; epilogue SwiGLU and the per-32
//           column quantization of h (a wave's 32 columns = one block).
//  down     B = 64 down rows (output rows); y = w_pair * acc, combined
//           afterwards in ascending expert id by the combine kernel.
#include "dev_vec.hpp"

namespace qrmoe {

constexpr int kTM = 64;                  // pairs per tile
constexpr int kTN = 64;                  // columns per tile
constexpr int kKC = 4;                   // blocks per staged K chunk
constexpr int kRowB = kKC * 32 + 16;     // padded LDS row (bytes)

typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v32f __attribute__((ext_vector_type(32)));

template <int NBR>
struct GemmSmem {
    alignas(16) int8_t A[kTM][kRowB];    // activation codes of the chunk
    alignas(16) int8_t B[NBR][kRowB];    // weight codes of the chunk
    float sa[kKC][kTM];                  // activation block scales of the chunk
    int32_t arow[kTM];                   // activation row of each tile row
    int32_t pair[kTM];
    float w[kTM];
};

__device__ __forceinline__ i32x4 g16(const void *p) { return *reinterpret_cast<const i32x4 *>(p); }
__device__ __forceinline__ i32x4 g16nt(const void *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const i32x4 *>(p));
}
__device__ __forceinline__ int acc_row(int i, int lane) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); }

// Staging registers of one K chunk: 2 activation and NBR/32 weight 16-byte
// pieces plus one activation scale per thread.
template <int NBR>
struct Stage {
    static constexpr int NW = NBR * 8 / 256;
    i32x4 a[2];
    i32x4 b[NW];
    float s;
};

// Tile setup: pairs, activation rows (token for x, pair for h) and weights.
template <int NBR>
__device__ __forceinline__ void setup_tile(const LayerArgs &a, GemmSmem<NBR> &sm, int4 grp, bool shared,
                                           bool act_is_h) {
    const int tid = threadIdx.x;
    const Dims &d = a.d;
    if (tid < kTM) {
        const int m = tid < grp.z ? tid : 0;  // rows past the tile's count repeat row 0; discarded
        const int p = shared ? d.T * d.k + grp.y + m : a.ws.perm[grp.y + m];
        sm.pair[tid] = p;
        sm.arow[tid] = act_is_h ? p : (shared ? grp.y + m : p / d.k);
        sm.w[tid] = shared ? 1.0f : a.ws.w[p];
    }
    __syncthreads();
}

// Global -> registers for chunk c.  brow(j) gives the weight row pointer of B
// staging row j (0..NBR-1).
template <int K, int NBR, class BRow>
__device__ __forceinline__ void load_chunk(Stage<NBR> &st, const GemmSmem<NBR> &sm, const int8_t *__restrict__ act,
                                           const float *__restrict__ ascale, BRow brow, int c) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int idx = tid + 256 * i, row = idx >> 3, piece = idx & 7;
        st.a[i] = g16(act + (int64_t)sm.arow[row] * K + c * (kKC * 32) + piece * 16);
    }
#pragma unroll
    for (int i = 0; i < Stage<NBR>::NW; ++i) {
        const int idx = tid + 256 * i, row = idx >> 3, piece = idx & 7;
        st.b[i] = g16nt(brow(row) + c * (kKC * 32) + piece * 16);
    }
    {
        const int kb = tid >> 6, m = tid & 63;
        st.s = ascale[(int64_t)sm.arow[m] * (K / 32) + c * kKC + kb];
    }
}

template <int NBR>
__device__ __forceinline__ void store_chunk(GemmSmem<NBR> &sm, const Stage<NBR> &st) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int idx = tid + 256 * i, row = idx >> 3, piece = idx & 7;
        *reinterpret_cast<i32x4 *>(&sm.A[row][piece * 16]) = st.a[i];
    }
#pragma unroll
    for (int i = 0; i < Stage<NBR>::NW; ++i) {
        const int idx = tid + 256 * i, row = idx >> 3, piece = idx & 7;
        *reinterpret_cast<i32x4 *>(&sm.B[row][piece * 16]) = st.b[i];
    }
    sm.sa[tid >> 6][tid & 63] = st.s;
}

// Weight block scales of one chunk for this lane's weight row: 4 fp16.
__device__ __forceinline__ uint2 chunk_scales(const uint16_t *srow, int c) {
    return *reinterpret_cast<const uint2 *>(srow + c * kKC);
}
__device__ __forceinline__ float scale_of(uint2 v, int kb) {
    const uint32_t word = kb < 2 ? v.x : v.y;
    return f16_to_f32((uint16_t)((kb & 1) ? (word >> 16) : (word & 0xffff)));
}

// ------------------------------------------------------------- gate / up
template <int H, bool DUMP>
__global__ __launch_bounds__(256) void gateup_mfma_kernel(LayerArgs a) {
    constexpr int NB = H / 32, NC = NB / kKC, NBR = 2 * kTN;
    __shared__ GemmSmem<NBR> sm;
    const int g = blockIdx.y;
    if (g >= a.ws.ctl[kCtlGroups]) return;
    const int4 grp = a.ws.groups[g];
    const bool shared = grp.x == a.d.E;
    const Dims &d = a.d;
    setup_tile(a, sm, grp, shared, false);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, half = lane >> 5, n = lane & 31;
    const int wm = wave >> 1, wn = wave & 1;
    const uint8_t *gmat = shared ? a.wt.sh_gate : a.wt.gate + grp.x * q8_bytes(d.F, H);
    const uint8_t *umat = shared ? a.wt.sh_up : a.wt.up + grp.x * q8_bytes(d.F, H);
    const int c0 = blockIdx.x * kTN;
    auto brow = [&](int j) -> const uint8_t * {
        return j < kTN ? gmat + (int64_t)(c0 + j) * H : umat + (int64_t)(c0 + j - kTN) * H;
    };
    const int col = c0 + wn * 32 + n;  // this lane's h column (gate/up row)
    // outer-product operand B: lanes 0..31 the gate scales, 32..63 the up scales of column col
    const uint16_t *srow = reinterpret_cast<const uint16_t *>((half ? umat : gmat) + (int64_t)d.F * H) +
                           (int64_t)col * NB;
    float accg[16], accu[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) accg[i] = accu[i] = 0.0f;
    Stage<NBR> st;
    load_chunk<H>(st, sm, a.ws.xq, a.ws.xd, brow, 0);
    uint2 wnext = chunk_scales(srow, 0);
#pragma unroll 1
    for (int c = 0; c < NC; ++c) {
        __syncthreads();
        store_chunk(sm, st);
        const uint2 wsc = wnext;
        __syncthreads();
        if (c + 1 < NC) {
            load_chunk<H>(st, sm, a.ws.xq, a.ws.xd, brow, c + 1);
            wnext = chunk_scales(srow, c + 1);
        }
#pragma unroll
        for (int kb = 0; kb < kKC; ++kb) {
            const int b = c * kKC + kb;
            const i32x4 av = *reinterpret_cast<const i32x4 *>(&sm.A[wm * 32 + n][kb * 32 + 16 * half]);
            const i32x4 gv = *reinterpret_cast<const i32x4 *>(&sm.B[wn * 32 + n][kb * 32 + 16 * half]);
            const i32x4 uv = *reinterpret_cast<const i32x4 *>(&sm.B[kTN + wn * 32 + n][kb * 32 + 16 * half]);
            const float dx = sm.sa[kb][wm * 32 + n];
            const float dw = scale_of(wsc, kb);
            const v16i zero = {};
            const v16i cg = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, gv, zero, 0, 0, 0);
            const v16i cu = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, uv, zero, 0, 0, 0);
            const v32f pz = {};
            const v32f ps = __builtin_amdgcn_mfma_f32_32x32x1f32(dx, dw, pz, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                accg[i] = __fmaf_rn((float)cg[i], ps[i], accg[i]);
                accu[i] = __fmaf_rn((float)cu[i], ps[16 + i], accu[i]);
            }
            if (DUMP && (col % a.dump.stride == 0)) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int m = wm * 32 + acc_row(i, lane);
                    if (m < grp.z) {
                        const int64_t base = ((int64_t)sm.pair[m] * (d.F / a.dump.stride) + col / a.dump.stride) *
                                                 a.dump.pitch_gu + b;
                        a.dump.gate_sums[base] = cg[i];
                        a.dump.up_sums[base] = cu[i];
                    }
                }
            }
        }
    }
    // SwiGLU, then quantize each pair's 32 columns (the 32 lanes of this half)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float hv = swiglu(accg[i], accu[i]);
        const float amax = group_max<32>(fabsf(hv));
        const float dsc = quant_scale(amax);
        const float inv = dsc > 0.0f ? 1.0f / dsc : 0.0f;
        const int m = wm * 32 + acc_row(i, lane);
        if (m < grp.z) {
            const int64_t p = sm.pair[m];
            a.ws.hq[p * d.F + col] = (int8_t)quant_code(hv, inv);
            if (n == 0) a.ws.hd[p * (d.F / 32) + col / 32] = dsc;
        }
    }
}

// ------------------------------------------------------------------ down
template <int F, bool DUMP>
__global__ __launch_bounds__(256) void down_mfma_kernel(LayerArgs a) {
    constexpr int NB = F / 32, NC = NB / kKC, NBR = kTN;
    __shared__ GemmSmem<NBR> sm;
    const int g = blockIdx.y;
    if (g >= a.ws.ctl[kCtlGroups]) return;
    const int4 grp = a.ws.groups[g];
    const bool shared = grp.x == a.d.E;
    const Dims &d = a.d;
    setup_tile(a, sm, grp, shared, true);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, half = lane >> 5, n = lane & 31;
    const int wm = wave >> 1, wn = wave & 1;
    const uint8_t *dmat = shared ? a.wt.sh_down : a.wt.down + grp.x * q8_bytes(d.H, F);
    const int r0 = blockIdx.x * kTN;
    auto brow = [&](int j) -> const uint8_t * { return dmat + (int64_t)(r0 + j) * F; };
    const int row = r0 + wn * 32 + n;  // this lane's output row
    float acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
    // outer product: both halves use this lane's row scale; products j = 0, 1 coincide
    const uint16_t *srow = reinterpret_cast<const uint16_t *>(dmat + (int64_t)d.H * F) + (int64_t)row * NB;
    Stage<NBR> st;
    load_chunk<F>(st, sm, a.ws.hq, a.ws.hd, brow, 0);
    uint2 wnext = chunk_scales(srow, 0);
#pragma unroll 1
    for (int c = 0; c < NC; ++c) {
        __syncthreads();
        store_chunk(sm, st);
        const uint2 wsc = wnext;
        __syncthreads();
        if (c + 1 < NC) {
            load_chunk<F>(st, sm, a.ws.hq, a.ws.hd, brow, c + 1);
            wnext = chunk_scales(srow, c + 1);
        }
#pragma unroll
        for (int kb = 0; kb < kKC; ++kb) {
            const int b = c * kKC + kb;
            const i32x4 av = *reinterpret_cast<const i32x4 *>(&sm.A[wm * 32 + n][kb * 32 + 16 * half]);
            const i32x4 wv = *reinterpret_cast<const i32x4 *>(&sm.B[wn * 32 + n][kb * 32 + 16 * half]);
            const float dh = sm.sa[kb][wm * 32 + n];
            const float dw = scale_of(wsc, kb);
            const v16i zero = {};
            const v16i cv = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, wv, zero, 0, 0, 0);
            const v32f pz = {};
            const v32f ps = __builtin_amdgcn_mfma_f32_32x32x1f32(dh, dw, pz, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[i] = __fmaf_rn((float)cv[i], ps[i], acc[i]);
            if (DUMP && (row % a.dump.stride == 0)) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int m = wm * 32 + acc_row(i, lane);
                    if (m < grp.z)
                        a.dump.down_sums[((int64_t)sm.pair[m] * (d.H / a.dump.stride) + row / a.dump.stride) *
                                             a.dump.pitch_dn + b] = cv[i];
                }
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int m = wm * 32 + acc_row(i, lane);
        if (m < grp.z) a.ws.y[(int64_t)sm.pair[m] * d.H + row] = __fmul_rn(sm.w[m], acc[i]);
    }
}

// ------------------------------------------------------------- launchers
template <bool DUMP>
static hipError_t gateup_m(const LayerArgs &a, dim3 grid, hipStream_t s) {
    switch (a.d.H) {
        case 256: klaunch(gateup_mfma_kernel<256, DUMP>, grid, 256, s, a); break;
        case 512: klaunch(gateup_mfma_kernel<512, DUMP>, grid, 256, s, a); break;
        case 1024: klaunch(gateup_mfma_kernel<1024, DUMP>, grid, 256, s, a); break;
        case 2048: klaunch(gateup_mfma_kernel<2048, DUMP>, grid, 256, s, a); break;
        case 4096: klaunch(gateup_mfma_kernel<4096, DUMP>, grid, 256, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_gateup_mfma(const LayerArgs &a, int max_tiles, bool dump, hipStream_t s) {
    if (a.d.F % kTN || a.d.H < 256) return hipErrorInvalidValue;
    dim3 grid(a.d.F / kTN, max_tiles);
    return dump ? gateup_m<true>(a, grid, s) : gateup_m<false>(a, grid, s);
}

template <bool DUMP>
static hipError_t down_m(const LayerArgs &a, dim3 grid, hipStream_t s) {
    switch (a.d.F) {
        case 256: klaunch(down_mfma_kernel<256, DUMP>, grid, 256, s, a); break;
        case 512: klaunch(down_mfma_kernel<512, DUMP>, grid, 256, s, a); break;
        case 1024: klaunch(down_mfma_kernel<1024, DUMP>, grid, 256, s, a); break;
        case 2048: klaunch(down_mfma_kernel<2048, DUMP>, grid, 256, s, a); break;
        case 4096: klaunch(down_mfma_kernel<4096, DUMP>, grid, 256, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_down_mfma(const LayerArgs &a, int max_tiles, bool dump, hipStream_t s) {
    if (a.d.H % kTN || a.d.F < 256) return hipErrorInvalidValue;
    dim3 grid(a.d.H / kTN, max_tiles);
    return dump ? down_m<true>(a, grid, s) : down_m<false>(a, grid, s);
}

}  // namespace qrmoe
