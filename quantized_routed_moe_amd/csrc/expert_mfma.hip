// Grouped int8 MFMA GEMMs of the expert FFN for batched tokens, Q8_32 and
// 2-bit Q2_256 weights (the 2-bit body is described at expert_gemm_q2).  The
// token sort gives each expert a list of pairs, cut into tiles of 64 (the
// expert-tile prefill kernels of "DwarfStar (ds4) — ROCm / gfx1151 fork",
// Performance optimizations, moe_gate_up_mid_expert_tile* /
// moe_down_expert_tile*; the expert-major schedule of "ds4: dfm Edition",
// About this fork).  For Q8 weights every 32-element quantization block is one
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
// One workgroup = 8 waves over a tile of 64 pairs x 128 weight rows, each
// wave one 32 x 32 block of it: (B rows 0..63 | 64..127) x 2 (pairs) x
// 2 (rows).
//  gate/up  B rows 0..63 are 64 gate rows, 64..127 the same 64 up rows; after
//           K, all sums pass through LDS and every wave applies SwiGLU and
//           the per-32-column quantization of h to 8 pairs.
//  down     B rows are 128 consecutive rows of the down matrix; y = w_pair *
//           acc, combined afterwards in ascending expert id by the combine
//           kernel.
// K runs in chunks of 4 blocks through a 3-stage LDS ring: chunk c+2 streams
// in while chunk c is computed, with one barrier per chunk.  A staged row
// holds a chunk's 128 code bytes as 8 16-byte slots, slot q of row r holding
// piece q ^ (r & 7), so the MFMA operand reads (8 consecutive rows at one
// piece) fall on 8 different bank groups.
#include <type_traits>

#include "dev_vec.hpp"

namespace qrmoe {

constexpr int kTM = 64;           // pairs per tile
constexpr int kTB = 128;          // weight rows per tile (gate/up: 64 of each)
constexpr int kKC = 4;            // blocks per K chunk
constexpr int kStages = 3;        // LDS ring depth
constexpr int kRow = kKC * 32;    // staged bytes per row and chunk

typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v32f __attribute__((ext_vector_type(32)));
typedef float v16f __attribute__((ext_vector_type(16)));

__device__ __forceinline__ int acc_row(int i, int lane) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); }

struct RingStage {
    int8_t A[kTM * kRow];      // activation codes of the chunk (swizzled rows)
    int8_t B[kTB * kRow];      // weight codes of the chunk (swizzled rows)
    float sa[kTM * kKC];       // activation block scales [pair][block]
    uint16_t sw[kTB * kKC];    // weight block scales [row][block], fp16
};
// A stage of the 2-bit ring: chunk c covers weights [128c, 128c + 128) of
// every row = 4 activation blocks = 8 weight subblocks of superblock c/2.
struct RingStageQ2 {
    int8_t A[kTM * kRow];      // activation codes of the chunk (swizzled rows, as for Q8)
    uint32_t Bq[kTB * 8];      // packed codes [row][subblock], one word per 16 weights
    uint32_t Bsm[kTB * 2];     // scale/min bytes [row][subblock] (4 per word)
    float sa[kTM * kKC];       // activation block scales [pair][block]
    int32_t as16[kTM * 8];     // activation code sums [pair][subblock]
    uint32_t dd[kTB];          // (fp16 d, fp16 dmin) of each row's superblock
};
struct RingSmem {
    union {
        RingStage st[kStages];
        RingStageQ2 q2[kStages];
    };
    int32_t arow[kTM];         // activation row of each tile row (token for x, pair for h)
    int32_t pair[kTM];
    float w[kTM];
};
static_assert(sizeof(RingStage) % 16 == 0 && sizeof(RingStageQ2) % 16 == 0, "stage alignment");
static_assert(2 * kTM * (kTB / 2) * 4 <= kStages * (int)sizeof(RingStageQ2), "SwiGLU exchange fits in the ring");

// Tile setup: pairs, activation rows and combine weights of the tile's rows.
__device__ __forceinline__ void setup_tile(const LayerArgs &a, RingSmem &sm, int4 grp, bool shared, bool act_is_h) {
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

// End of a tile.  gate/up: SwiGLU and the per-32-column quantization of h,
// spread over all waves: every wave parks its sums in LDS (the ring is
// drained: the last chunk waited for every load), then lane l of wave w takes
// pair 8w + l/8 and its 8 columns 8(l%8) .. +7; the 4 lanes of one 32-column
// block share its scale.  With HS16 the sums of h's codes over 16-column
// subblocks are stored too (the 2-bit down GEMM's activation sums).
// down: y[pair][row] = w_pair * acc, combined afterwards in ascending expert
// id by the combine kernel.
template <bool GU, bool HS16>
__device__ __forceinline__ void tile_epilogue(const LayerArgs &a, RingSmem &sm, int4 grp, const float (&acc)[16],
                                              int r0, int col, bool live) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, n = lane & 31;
    const int which = wave >> 2, wm = (wave >> 1) & 1, wn = wave & 1;
    const Dims &d = a.d;
    if constexpr (GU) {
        __syncthreads();
        float *gx = reinterpret_cast<float *>(&sm.st[0]);  // [64 pairs][64 columns] gate, then up
#pragma unroll
        for (int i = 0; i < 16; ++i)
            gx[which * kTM * (kTB / 2) + (wm * 32 + acc_row(i, lane)) * (kTB / 2) + wn * 32 + n] = acc[i];
        __syncthreads();
        const int m = 8 * wave + (lane >> 3), cg = lane & 7;
        const float *grow = gx + m * (kTB / 2) + 8 * cg, *urow = grow + kTM * (kTB / 2);
        const float4 g0 = *reinterpret_cast<const float4 *>(grow), g1 = *reinterpret_cast<const float4 *>(grow + 4);
        const float4 u0 = *reinterpret_cast<const float4 *>(urow), u1 = *reinterpret_cast<const float4 *>(urow + 4);
        const float hv[8] = {swiglu(g0.x, u0.x), swiglu(g0.y, u0.y), swiglu(g0.z, u0.z), swiglu(g0.w, u0.w),
                             swiglu(g1.x, u1.x), swiglu(g1.y, u1.y), swiglu(g1.z, u1.z), swiglu(g1.w, u1.w)};
        float amax = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(hv[j]));
        amax = group_max<4>(amax);
        const float dsc = quant_scale(amax);
        const float inv = dsc > 0.0f ? 1.0f / dsc : 0.0f;
        uint32_t q0 = 0, q1 = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            q0 |= ((uint32_t)quant_code(hv[j], inv) & 0xffu) << (8 * j);
            q1 |= ((uint32_t)quant_code(hv[4 + j], inv) & 0xffu) << (8 * j);
        }
        const int64_t p = sm.pair[m];
        const int hc = r0 + 8 * cg;  // first h column of this lane
        if (m < grp.z) {
            *reinterpret_cast<uint2 *>(&a.ws.hq[p * d.F + hc]) = make_uint2(q0, q1);
            if ((cg & 3) == 0) a.ws.hd[p * (d.F / 32) + hc / 32] = dsc;
        }
        if constexpr (HS16) {
            // lanes cg, cg ^ 1 hold the two halves of one 16-column subblock
            int cs = sdot4((int)q0, 0x01010101, 0);
            cs = sdot4((int)q1, 0x01010101, cs);
            cs += __shfl_xor(cs, 1);
            if (m < grp.z && (cg & 1) == 0) a.ws.hs16[p * (d.F / 16) + hc / 16] = cs;
        }
    } else if (live) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int m = wm * 32 + acc_row(i, lane);
            if (m < grp.z) a.ws.y[(int64_t)sm.pair[m] * d.H + col] = __fmul_rn(sm.w[m], acc[i]);
        }
    }
}

// One expert tile of the gate/up (GU) or down GEMM, K = H or F.
template <int K, bool GU, bool DUMP>
__device__ __forceinline__ void expert_gemm(const LayerArgs &a, RingSmem &sm, int4 grp, bool shared) {
    constexpr int NB = K / 32, NC = NB / kKC;
    static_assert(NC >= 2 && NB % kKC == 0, "K chunks");
    const Dims &d = a.d;
    setup_tile(a, sm, grp, shared, !GU);
    const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, n = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int which = wave >> 2, wm = (wave >> 1) & 1, wn = wave & 1;  // which: B rows 0..63 or 64..127
    const int R = GU ? d.F : d.H;  // rows of each weight matrix
    const uint32_t mat_bytes = (uint32_t)q8_bytes(R, K);
    const uint8_t *m0, *m1;  // matrices of B rows 0..63 and 64..127
    if constexpr (GU) {
        m0 = shared ? a.wt.sh_gate : a.wt.gate + grp.x * q8_bytes(R, K);
        m1 = shared ? a.wt.sh_up : a.wt.up + grp.x * q8_bytes(R, K);
    } else {
        m0 = m1 = shared ? a.wt.sh_down : a.wt.down + grp.x * q8_bytes(R, K);
    }
    // first weight row of B rows 0..63 and of 64..127
    const int r0 = GU ? blockIdx.x * (kTB / 2) : blockIdx.x * kTB;
    const int r1 = GU ? r0 : r0 + kTB / 2;
    const int8_t *act = GU ? a.ws.xq : a.ws.hq;
    const float *ascale = GU ? a.ws.xd : a.ws.hd;
    const int64_t act_rows = GU ? d.T : d.P;

    // ---- this wave's four loads per chunk (byte offsets at chunk 0)
    const __amdgpu_buffer_rsrc_t r_act = buf_rsrc(act, (uint32_t)(act_rows * K));
    const __amdgpu_buffer_rsrc_t r_b0 = buf_rsrc(m0, mat_bytes), r_b1 = buf_rsrc(m1, mat_bytes);
    const int lrow = 8 * wave + (lane >> 3), piece = (lane & 7) ^ (lane >> 3);
    const uint32_t off_a = (uint32_t)sm.arow[lrow] * K + 16 * piece;   // activation row lrow
    const uint32_t off_b0 = (uint32_t)(r0 + lrow) * K + 16 * piece;     // B row lrow
    const uint32_t off_b1 = (uint32_t)(r1 + lrow) * K + 16 * piece;     // B row 64 + lrow
    __amdgpu_buffer_rsrc_t r_s;
    uint32_t off_s;
    if (wave < 4) {  // activation scales: pairs 16 wave .. +15, 4 blocks each
        r_s = buf_rsrc(ascale, (uint32_t)(act_rows * (K / 32) * 4));
        off_s = ((uint32_t)sm.arow[16 * wave + (lane >> 2)] * (K / 32) + (lane & 3)) * 4;
    } else {         // weight scales: B rows 32 (wave-4) .. +31, two dwords (4 fp16) each
        const int rr = 32 * (wave - 4) + (lane >> 1);
        r_s = wave < 6 ? r_b0 : r_b1;
        off_s = (uint32_t)R * K + (uint32_t)((wave < 6 ? r0 : r1) + (rr & 63)) * (K / 32) * 2 + 4 * (lane & 1);
    }
    auto issue = [&](int c, int stg) {
        RingStage &S = sm.st[stg];
        dma16(r_act, &S.A[wave * 1024], off_a + c * kRow);
        dma16(r_b0, &S.B[wave * 1024], off_b0 + c * kRow);
        dma16(r_b1, &S.B[(kTB / 2) * kRow + wave * 1024], off_b1 + c * kRow);
        if (wave < 4) dma4(r_s, &S.sa[wave * 64], off_s + c * (kKC * 4));
        else dma4(r_s, &S.sw[(wave - 4) * 128], off_s + c * (kKC * 2));
    };

    // ---- this lane's LDS reads: operand rows and the swizzled slot of each block half
    const int am = wm * 32 + n, bj = which * (kTB / 2) + wn * 32 + n;
    uint32_t slot[kKC];
#pragma unroll
    for (int kb = 0; kb < kKC; ++kb) slot[kb] = 16 * ((2 * kb + half) ^ (n & 7));
    // this lane's weight row: its h column (gate/up) or output row (down)
    const int col = GU ? r0 + wn * 32 + n : r0 + bj;
    const bool live = wm * 32 < grp.z;  // this wave's 32 pairs hold at least one real pair
    float acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.0f;

    issue(0, 0);
    issue(1, 1);
    auto compute = [&](int c, const RingStage &S) {
        auto block_mfma = [&](int kb) {
            const i32x4 av = *reinterpret_cast<const i32x4 *>(&S.A[am * kRow + slot[kb]]);
            const i32x4 bv = *reinterpret_cast<const i32x4 *>(&S.B[bj * kRow + slot[kb]]);
            const v16i zero = {};
            return __builtin_amdgcn_mfma_i32_32x32x32_i8(av, bv, zero, 0, 0, 0);
        };
        v16i cnext = block_mfma(0);
#pragma unroll
        for (int kb = 0; kb < kKC; kb += 2) {
            // scale products of blocks kb (registers 0..15) and kb+1 (16..31)
            const float dx = S.sa[am * kKC + kb + half];
            const float dw = f16_to_f32(S.sw[bj * kKC + kb + half]);
            const v32f pz = {};
            const v32f ps = __builtin_amdgcn_mfma_f32_32x32x1f32(dx, dw, pz, 0, 0, 0);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int b = c * kKC + kb + j;
                const v16i cv = cnext;
                if (kb + j + 1 < kKC) cnext = block_mfma(kb + j + 1);
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[i] = __fmaf_rn((float)cv[i], ps[16 * j + i], acc[i]);
                if (DUMP && (col % a.dump.stride == 0)) {
                    int32_t *dst = GU ? (which ? a.dump.up_sums : a.dump.gate_sums) : a.dump.down_sums;
                    const int pitch = GU ? a.dump.pitch_gu : a.dump.pitch_dn;
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int m = wm * 32 + acc_row(i, lane);
                        if (m < grp.z)
                            dst[((int64_t)sm.pair[m] * (R / a.dump.stride) + col / a.dump.stride) * pitch + b] = cv[i];
                    }
                }
            }
        }
    };
    // chunk c: wait for this wave's loads of c (those of c+1 may still fly),
    // barrier (every wave's loads of c landed, every wave done with c-1),
    // refill the stage of c-1 with c+2, compute c.
    auto step = [&](int c, auto stg_c) {
        constexpr int stg = decltype(stg_c)::value;
        if (c + 1 < NC) wait_vm<4>();
        else wait_vm<0>();
        lds_barrier();
        if (c + 2 < NC) issue(c + 2, (stg + 2) % kStages);
        if (live) compute(c, sm.st[stg]);
    };
#pragma unroll 1
    for (int c = 0; c < NC; c += kStages) {
        step(c, std::integral_constant<int, 0>{});
        if (c + 1 < NC) step(c + 1, std::integral_constant<int, 1>{});
        if (c + 2 < NC) step(c + 2, std::integral_constant<int, 2>{});
    }
    tile_epilogue<GU, false>(a, sm, grp, acc, r0, col, live);
}

// One expert tile of a 2-bit (Q2_256) matrix, K = H (gate/up) or F (down).
// A 16-weight subblock of a row holds codes q in 0..3 with a 4-bit scale s
// and a 4-bit min m, its 256-weight superblock an fp16 d and dmin; the
// weight is d*s*q - dmin*m.  Against a 32-block b of the activation (codes x,
// scale ad_b) the row's sum is
//   ad_b * d * SP_b - ad_b * dmin * SM_b,
//   SP_b = sum over the block of (s*q) * x: one int8 MFMA, the codes being
//          expanded to the bytes s*q <= 45 as the operand is formed (a
//          v_perm_b32 lookup in the table {0, s, 2s, 3s});
//   SM_b = sum over the block's two subblocks of m * (sum of x over it).
// The first term is scaled as in the Q8 GEMM (outer product ad x d, one
// conversion and one fma per output and block); the second is one
// v_mfma_f32_32x32x2_f32 per block, (ad_b * xsum) x (-dmin * m) (the latter
// exact in fp32).  The two terms largely cancel, so both go, block after
// block, into a partial sum of the chunk's four blocks that starts at zero,
// and the tile's accumulator takes one addition per chunk: its rounding
// errors stay relative to the result, not to the terms.
//
// Ring loads per wave and chunk (three each):
//   every wave   activation codes of tile rows 8w .. 8w+7 (as in the Q8 GEMM)
//   waves 0-3    packed codes of B rows 32w .. +31; activation scales of pairs 16w .. +15
//   waves 4-7    scale/min bytes of B rows 32(w-4) .. +31
//   waves 4, 5   activation code sums of pairs 32(w-4) .. +31
//   waves 6, 7   (d, dmin) of B rows 64(w-6) .. +63
template <int K, bool GU, bool DUMP>
__device__ __forceinline__ void expert_gemm_q2(const LayerArgs &a, RingSmem &sm, int4 grp) {
    constexpr int NB = K / 32, NC = NB / kKC;
    static_assert(NC >= 2 && K % 256 == 0, "K chunks");
    const Dims &d = a.d;
    setup_tile(a, sm, grp, false, !GU);
    const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, n = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int which = wave >> 2, wm = (wave >> 1) & 1, wn = wave & 1;
    const int R = GU ? d.F : d.H;  // rows of each weight matrix
    const uint32_t mat_bytes = (uint32_t)q2_bytes(R, K);
    const uint8_t *m0, *m1;  // matrices of B rows 0..63 and 64..127
    if constexpr (GU) {
        m0 = a.wt.gate + grp.x * q2_bytes(R, K);
        m1 = a.wt.up + grp.x * q2_bytes(R, K);
    } else {
        m0 = m1 = a.wt.down + grp.x * q2_bytes(R, K);
    }
    const int r0 = GU ? blockIdx.x * (kTB / 2) : blockIdx.x * kTB;
    const int r1 = GU ? r0 : r0 + kTB / 2;
    const int8_t *act = GU ? a.ws.xq : a.ws.hq;
    const float *ascale = GU ? a.ws.xd : a.ws.hd;
    const int32_t *asum = GU ? a.ws.xs16 : a.ws.hs16;
    const int64_t act_rows = GU ? d.T : d.P;
    const uint32_t sm_plane = (uint32_t)R * (K / 4), dd_plane = sm_plane + (uint32_t)R * (K / 16);

    const __amdgpu_buffer_rsrc_t r_act = buf_rsrc(act, (uint32_t)(act_rows * K));
    const __amdgpu_buffer_rsrc_t r_b0 = buf_rsrc(m0, mat_bytes), r_b1 = buf_rsrc(m1, mat_bytes);
    const int lrow = 8 * wave + (lane >> 3), piece = (lane & 7) ^ (lane >> 3);
    const uint32_t off_a = (uint32_t)sm.arow[lrow] * K + 16 * piece;
    const int v = wave & 3;                                  // B rows 32v .. +31 for the code / scale-min loads
    const int grow = (v < 2 ? r0 : r1) + 32 * (v & 1) + (lane >> 1);  // matrix row of this lane's B row
    const __amdgpu_buffer_rsrc_t r_bx = v < 2 ? r_b0 : r_b1;
    uint32_t off_1, off_2;
    __amdgpu_buffer_rsrc_t r_2;
    if (wave < 4) {
        off_1 = (uint32_t)grow * (K / 4) + 16 * (lane & 1);
        r_2 = buf_rsrc(ascale, (uint32_t)(act_rows * (K / 32) * 4));
        off_2 = ((uint32_t)sm.arow[16 * wave + (lane >> 2)] * (K / 32) + (lane & 3)) * 4;
    } else {
        off_1 = sm_plane + (uint32_t)grow * (K / 16) + 4 * (lane & 1);
        if (wave < 6) {
            r_2 = buf_rsrc(asum, (uint32_t)(act_rows * (K / 16) * 4));
            off_2 = ((uint32_t)sm.arow[32 * (wave - 4) + (lane >> 1)] * (K / 16) + 4 * (lane & 1)) * 4;
        } else {
            r_2 = wave == 6 ? r_b0 : r_b1;
            off_2 = dd_plane + (uint32_t)((wave == 6 ? r0 : r1) + lane) * (K / 256) * 4;
        }
    }
    auto issue = [&](int c, int stg) {
        RingStageQ2 &S = sm.q2[stg];
        dma16(r_act, &S.A[wave * 1024], off_a + c * kRow);
        if (wave < 4) {
            dma16(r_bx, &S.Bq[wave * 256], off_1 + c * 32);
            dma4(r_2, &S.sa[wave * 64], off_2 + c * (kKC * 4));
        } else {
            dma4(r_bx, &S.Bsm[(wave - 4) * 64], off_1 + c * 8);
            if (wave < 6) dma16(r_2, &S.as16[(wave - 4) * 256], off_2 + c * 32);
            else dma4(r_2, &S.dd[(wave - 6) * 64], off_2 + (c >> 1) * 4);
        }
    };

    const int am = wm * 32 + n, bj = which * (kTB / 2) + wn * 32 + n;
    uint32_t slot[kKC];
#pragma unroll
    for (int kb = 0; kb < kKC; ++kb) slot[kb] = 16 * ((2 * kb + half) ^ (n & 7));
    const int col = GU ? r0 + wn * 32 + n : r0 + bj;
    const bool live = wm * 32 < grp.z;
    constexpr uint32_t kLo2 = 0x03030303u;
    const uint32_t keep0 = half ? 0u : ~0u;  // dumps: subblock 2kb (lower half lanes) / 2kb+1
    float acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.0f;

    issue(0, 0);
    issue(1, 1);
    auto compute = [&](int c, const RingStageQ2 &S) {
        const uint32_t ddw = S.dd[bj];
        const float dw = f16_to_f32((uint16_t)(ddw & 0xffffu));
        const float nmin = -f16_to_f32((uint16_t)(ddw >> 16));
        const float4 sav = *reinterpret_cast<const float4 *>(&S.sa[am * kKC]);
        const float sa_k[kKC] = {sav.x, sav.y, sav.z, sav.w};
        const uint2 smw = *reinterpret_cast<const uint2 *>(&S.Bsm[bj * 2]);
        // a row's 8 code words (and a pair's 8 sums) as two 16-byte reads; this
        // lane's subblocks are 2kb + half
        const i32x4 bq0 = *reinterpret_cast<const i32x4 *>(&S.Bq[bj * 8]);
        const i32x4 bq1 = *reinterpret_cast<const i32x4 *>(&S.Bq[bj * 8 + 4]);
        const i32x4 xs0 = *reinterpret_cast<const i32x4 *>(&S.as16[am * 8]);
        const i32x4 xs1 = *reinterpret_cast<const i32x4 *>(&S.as16[am * 8 + 4]);
        const uint32_t cw[kKC] = {(uint32_t)(half ? bq0.y : bq0.x), (uint32_t)(half ? bq0.w : bq0.z),
                                  (uint32_t)(half ? bq1.y : bq1.x), (uint32_t)(half ? bq1.w : bq1.z)};
        const int32_t xs[kKC] = {half ? xs0.y : xs0.x, half ? xs0.w : xs0.z, half ? xs1.y : xs1.x,
                                 half ? xs1.w : xs1.z};
        // scale/min byte of this lane's subblock 2kb + half
        auto smbyte = [&](int kb) { return ((kb < 2 ? smw.x : smw.y) >> (8 * (2 * (kb & 1)) + 8 * half)) & 0xffu; };
        auto a_op = [&](int kb) { return *reinterpret_cast<const i32x4 *>(&S.A[am * kRow + slot[kb]]); };
        auto block_mfma = [&](int kb) {
            const uint32_t tbl = ((smbyte(kb) & 15u) * 0x030201u) << 8;  // bytes 0, s, 2s, 3s
            const uint32_t w = cw[kb];
            const i32x4 bv = {(int)__builtin_amdgcn_perm(0u, tbl, w & kLo2),
                              (int)__builtin_amdgcn_perm(0u, tbl, (w >> 2) & kLo2),
                              (int)__builtin_amdgcn_perm(0u, tbl, (w >> 4) & kLo2),
                              (int)__builtin_amdgcn_perm(0u, tbl, (w >> 6) & kLo2)};
            const v16i zero = {};
            return __builtin_amdgcn_mfma_i32_32x32x32_i8(a_op(kb), bv, zero, 0, 0, 0);
        };
        v16i cnext = block_mfma(0);
        v16f t = {};  // the chunk's partial sum
#pragma unroll
        for (int kb = 0; kb < kKC; kb += 2) {
            const float dx = half ? sa_k[kb + 1] : sa_k[kb];
            const v32f pz = {};
            const v32f ps = __builtin_amdgcn_mfma_f32_32x32x1f32(dx, dw, pz, 0, 0, 0);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int kj = kb + j, b = c * kKC + kj;
                const v16i cv = cnext;
                if (kj + 1 < kKC) cnext = block_mfma(kj + 1);
                const float xa = __fmul_rn(sa_k[kj], (float)xs[kj]);
                const float mb = __fmul_rn(nmin, (float)(smbyte(kj) >> 4));
                t = __builtin_amdgcn_mfma_f32_32x32x2f32(xa, mb, t, 0, 0, 0);
#pragma unroll
                for (int i = 0; i < 16; ++i) t[i] = __fmaf_rn((float)cv[i], ps[16 * j + i], t[i]);
                if constexpr (DUMP) {
                    // exact subblock sums sum(q * x) of subblocks 2b and 2b+1
                    const uint32_t w = cw[kj];
                    const uint32_t e[4] = {w & kLo2, (w >> 2) & kLo2, (w >> 4) & kLo2, (w >> 6) & kLo2};
                    const i32x4 q0 = {(int)(e[0] & keep0), (int)(e[1] & keep0), (int)(e[2] & keep0),
                                      (int)(e[3] & keep0)};
                    const i32x4 q1 = {(int)(e[0] & ~keep0), (int)(e[1] & ~keep0), (int)(e[2] & ~keep0),
                                      (int)(e[3] & ~keep0)};
                    const v16i zero = {};
                    const v16i p0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a_op(kj), q0, zero, 0, 0, 0);
                    const v16i p1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a_op(kj), q1, zero, 0, 0, 0);
                    if (col % a.dump.stride == 0) {
                        int32_t *dst = GU ? (which ? a.dump.up_sums : a.dump.gate_sums) : a.dump.down_sums;
                        const int pitch = GU ? a.dump.pitch_gu : a.dump.pitch_dn;
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            const int m = wm * 32 + acc_row(i, lane);
                            if (m < grp.z) {
                                int32_t *o = dst + ((int64_t)sm.pair[m] * (R / a.dump.stride) + col / a.dump.stride) * pitch;
                                o[2 * b] = p0[i];
                                o[2 * b + 1] = p1[i];
                            }
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] = __fadd_rn(acc[i], t[i]);
    };
    auto step = [&](int c, auto stg_c) {
        constexpr int stg = decltype(stg_c)::value;
        if (c + 1 < NC) wait_vm<3>();
        else wait_vm<0>();
        lds_barrier();
        if (c + 2 < NC) issue(c + 2, (stg + 2) % kStages);
        if (live) compute(c, sm.q2[stg]);
    };
#pragma unroll 1
    for (int c = 0; c < NC; c += kStages) {
        step(c, std::integral_constant<int, 0>{});
        if (c + 1 < NC) step(c + 1, std::integral_constant<int, 1>{});
        if (c + 2 < NC) step(c + 2, std::integral_constant<int, 2>{});
    }
    tile_epilogue<GU, GU>(a, sm, grp, acc, r0, col, live);
}

// Work-list entry of this workgroup; entries past the device-side count exit.
// Q2 layers: the shared expert (Q8) and routed experts (2-bit) share a launch.
template <int H, int FMT, bool DUMP>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4))) void gateup_mfma_kernel(LayerArgs a) {
    __shared__ __attribute__((aligned(16))) RingSmem sm;
    if ((int)blockIdx.y >= a.ws.ctl[kCtlGroups]) return;
    const int4 grp = a.ws.groups[blockIdx.y];
    const bool shared = grp.x == a.d.E;
    if constexpr (FMT == kFmtQ2) {
        if (!shared) {
            expert_gemm_q2<H, true, DUMP>(a, sm, grp);
            return;
        }
    }
    expert_gemm<H, true, DUMP>(a, sm, grp, shared);
}
template <int F, int FMT, bool DUMP>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4))) void down_mfma_kernel(LayerArgs a) {
    __shared__ __attribute__((aligned(16))) RingSmem sm;
    if ((int)blockIdx.y >= a.ws.ctl[kCtlGroups]) return;
    const int4 grp = a.ws.groups[blockIdx.y];
    const bool shared = grp.x == a.d.E;
    if constexpr (FMT == kFmtQ2) {
        if (!shared) {
            expert_gemm_q2<F, false, DUMP>(a, sm, grp);
            return;
        }
    }
    expert_gemm<F, false, DUMP>(a, sm, grp, shared);
}

// ------------------------------------------------------------- launchers
template <bool GU, int FMT, bool DUMP, int K>
static void gemm_launch_k(const LayerArgs &a, dim3 grid, hipStream_t s) {
    if constexpr (GU) klaunch(gateup_mfma_kernel<K, FMT, DUMP>, grid, 512, s, a);
    else klaunch(down_mfma_kernel<K, FMT, DUMP>, grid, 512, s, a);
}
template <bool GU, int FMT, bool DUMP>
static hipError_t gemm_launch(const LayerArgs &a, int K, dim3 grid, hipStream_t s) {
    switch (K) {
        case 256: gemm_launch_k<GU, FMT, DUMP, 256>(a, grid, s); break;
        case 512: gemm_launch_k<GU, FMT, DUMP, 512>(a, grid, s); break;
        case 1024: gemm_launch_k<GU, FMT, DUMP, 1024>(a, grid, s); break;
        case 2048: gemm_launch_k<GU, FMT, DUMP, 2048>(a, grid, s); break;
        case 4096: gemm_launch_k<GU, FMT, DUMP, 4096>(a, grid, s); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}
template <bool GU>
static hipError_t gemm_dispatch(const LayerArgs &a, int K, dim3 grid, bool dump, hipStream_t s) {
    if (a.d.fmt == kFmtQ2)
        return dump ? gemm_launch<GU, kFmtQ2, true>(a, K, grid, s) : gemm_launch<GU, kFmtQ2, false>(a, K, grid, s);
    return dump ? gemm_launch<GU, kFmtQ8, true>(a, K, grid, s) : gemm_launch<GU, kFmtQ8, false>(a, K, grid, s);
}

hipError_t launch_gateup_mfma(const LayerArgs &a, int max_tiles, bool dump, hipStream_t s) {
    if (a.d.F % (kTB / 2) || a.d.H < 256) return hipErrorInvalidValue;
    return gemm_dispatch<true>(a, a.d.H, dim3(a.d.F / (kTB / 2), max_tiles), dump, s);
}

hipError_t launch_down_mfma(const LayerArgs &a, int max_tiles, bool dump, hipStream_t s) {
    if (a.d.H % kTB || a.d.F < 256) return hipErrorInvalidValue;
    return gemm_dispatch<false>(a, a.d.F, dim3(a.d.H / kTB, max_tiles), dump, s);
}

}  // namespace qrmoe
