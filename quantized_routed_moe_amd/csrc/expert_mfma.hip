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
// Tile = 64 pairs x 64 columns.  K runs in chunks of KC blocks staged in LDS
// (padded rows), the next chunk's global loads held in registers meanwhile.
// The scale products of two consecutive blocks come from one 2-block outer
// product (lanes 0..31 supply block b, lanes 32..63 block b+1).
//
//  gate/up  8 waves: (gate | up) x 2 (pairs) x 2 (columns), each wave one
//           32 x 32 tile of one matrix (fewer registers per wave, so more
//           waves hide the epilogue's latency); after K, the up waves pass
//           their sums through LDS and the gate waves apply SwiGLU and the
//           per-32-column quantization of h (a wave's 32 columns = one block).
//  down     4 waves: 2 (pairs) x 2 (output rows); y = w_pair * acc, combined
//           afterwards in ascending expert id by the combine kernel.
#include <utility>

#include "dev_vec.hpp"

namespace qrmoe {

constexpr int kTM = 64;                  // pairs per tile
constexpr int kTN = 64;                  // columns per tile
// K chunk staged per step of the down GEMM: 8 blocks (twice the compute
// between a chunk's request and its use).
constexpr int kKCDown = 8;
template <int KC>
constexpr int row_bytes() { return KC * 32 + 16; }  // padded LDS row (bytes)

typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v32f __attribute__((ext_vector_type(32)));

template <int NBR, int KC>
struct GemmSmem {
    static constexpr int kKC = KC;
    alignas(16) int8_t A[kTM][row_bytes<KC>()];    // activation codes of the chunk
    alignas(16) int8_t B[NBR][row_bytes<KC>()];    // weight codes of the chunk
    float sa[KC][kTM];                             // activation block scales of the chunk
    uint32_t sw[NBR][KC / 2];                      // weight block scales of the chunk (fp16 pairs)
    int32_t arow[kTM];                   // activation row of each tile row
    int32_t pair[kTM];
    float w[kTM];
};

__device__ __forceinline__ i32x4 g16(const void *p) { return *reinterpret_cast<const i32x4 *>(p); }
__device__ __forceinline__ i32x4 g16nt(const void *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const i32x4 *>(p));
}
__device__ __forceinline__ int acc_row(int i, int lane) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); }

// Staging of one K chunk (kKC blocks) by NT threads: 16-byte activation and
// weight code pieces, activation block scales and pairs of fp16 weight block
// scales, spread evenly over the threads.  The global addresses of a thread's
// pieces do not change from chunk to chunk and are set up once; the compute
// phase reads only LDS, so no value loaded for a later chunk is waited for
// early (a wave waits for its loads in issue order).
template <int NT, int NBR, int kKC>
struct Stage {
    static constexpr int PR = kKC * 2;                   // 16-byte pieces per row and chunk
    static constexpr int NA = kTM * PR / NT;
    static constexpr int NW = NBR * PR / NT;
    static constexpr int NS = (kKC * kTM + NT - 1) / NT;           // activation scales per thread
    static constexpr int NWS = (NBR * (kKC / 2) + NT - 1) / NT;    // fp16 weight-scale pairs per thread
    static_assert(NA >= 1 && NW >= 1 && kTM * PR % NT == 0 && NBR * PR % NT == 0, "staging geometry");
    const int8_t *pa[NA];
    const uint8_t *pb[NW];
    const float *ps[NS];
    const uint32_t *pw[NWS];
    i32x4 a[NA];
    i32x4 b[NW];
    float s[NS];
    uint32_t w[NWS];

    // bmat(j): weight matrix of B staging row j; brow0(j): its first row index
    template <int K, class BRow>
    __device__ __forceinline__ void setup(const GemmSmem<NBR, kKC> &sm, const int8_t *__restrict__ act,
                                          const float *__restrict__ ascale, int64_t R, BRow brow) {
        const int tid = threadIdx.x;
#pragma unroll
        for (int i = 0; i < NA; ++i) {
            const int idx = tid + NT * i, row = idx / PR, piece = idx % PR;
            pa[i] = act + (int64_t)sm.arow[row] * K + piece * 16;
        }
#pragma unroll
        for (int i = 0; i < NW; ++i) {
            const int idx = tid + NT * i, row = idx / PR, piece = idx % PR;
            pb[i] = brow(row).first + (int64_t)brow(row).second * K + piece * 16;
        }
        // (scale slots past the chunk's count point at slot 0 and load nothing)
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            const int idx = tid + NT * i < kKC * kTM ? tid + NT * i : 0;
            const int m = idx & 63, kb = idx >> 6;
            ps[i] = ascale + (int64_t)sm.arow[m] * (K / 32) + kb;
        }
#pragma unroll
        for (int i = 0; i < NWS; ++i) {
            const int idx = tid + NT * i < NBR * (kKC / 2) ? tid + NT * i : 0;
            const int wr = idx / (kKC / 2), wh = idx % (kKC / 2);
            pw[i] = reinterpret_cast<const uint32_t *>(brow(wr).first + R * K) +
                    ((int64_t)brow(wr).second * (K / 32)) / 2 + wh;
        }
    }
    __device__ __forceinline__ void load(int c) {
        const int tid = threadIdx.x;
#pragma unroll
        for (int i = 0; i < NA; ++i) a[i] = g16(pa[i] + c * (kKC * 32));
#pragma unroll
        for (int i = 0; i < NW; ++i) b[i] = g16nt(pb[i] + c * (kKC * 32));
#pragma unroll
        for (int i = 0; i < NS; ++i)
            if (tid + NT * i < kKC * kTM) s[i] = ps[i][c * kKC];
#pragma unroll
        for (int i = 0; i < NWS; ++i)
            if (tid + NT * i < NBR * (kKC / 2)) w[i] = pw[i][c * (kKC / 2)];
    }
    __device__ __forceinline__ void store(GemmSmem<NBR, kKC> &sm) const {
        const int tid = threadIdx.x;
#pragma unroll
        for (int i = 0; i < NA; ++i) {
            const int idx = tid + NT * i, row = idx / PR, piece = idx % PR;
            *reinterpret_cast<i32x4 *>(&sm.A[row][piece * 16]) = a[i];
        }
#pragma unroll
        for (int i = 0; i < NW; ++i) {
            const int idx = tid + NT * i, row = idx / PR, piece = idx % PR;
            *reinterpret_cast<i32x4 *>(&sm.B[row][piece * 16]) = b[i];
        }
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            const int idx = tid + NT * i;
            if (idx < kKC * kTM) sm.sa[idx >> 6][idx & 63] = s[i];
        }
#pragma unroll
        for (int i = 0; i < NWS; ++i) {
            const int idx = tid + NT * i;
            if (idx < NBR * (kKC / 2)) sm.sw[idx / (kKC / 2)][idx % (kKC / 2)] = w[i];
        }
    }
};

// Tile setup: pairs, activation rows (token for x, pair for h) and weights.
template <class Smem>
__device__ __forceinline__ void setup_tile(const LayerArgs &a, Smem &sm, int4 grp, bool shared,
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

// fp16 weight scale of block kb (0..kKC-1) of staged weight row r
template <class Smem>
__device__ __forceinline__ float wscale(const Smem &sm, int r, int kb) {
    const uint32_t v = sm.sw[r][kb >> 1];
    return f16_to_f32((uint16_t)((kb & 1) ? (v >> 16) : (v & 0xffff)));
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

// ------------------------------------------------------------- gate / up
// One workgroup: 64 pairs x 64 columns of gate and of up (128 weight rows),
// 8 waves, (gate | up) x 2 (pairs) x 2 (columns), each wave one 32 x 32 tile
// of one matrix.  K runs in chunks of 4 blocks through a 3-stage LDS ring:
// chunk c+2 streams in while chunk c is computed, one barrier per chunk.
// A row holds a chunk's 128 code bytes as 8 16-byte slots, slot q of row r
// holding piece q ^ (r & 7), so the MFMA operand reads (8 consecutive rows
// at one piece) fall on 8 different bank groups.
constexpr int kGuKC = 4;       // blocks per chunk
constexpr int kGuStages = 3;   // LDS ring depth
constexpr int kGuRow = kGuKC * 32;
struct GuStage {
    int8_t A[kTM * kGuRow];        // activation codes of the chunk (swizzled rows)
    int8_t B[2 * kTN * kGuRow];    // gate rows 0..63, up rows 64..127 (swizzled)
    float sa[kTM * kGuKC];         // activation block scales [pair][block]
    uint16_t sw[2 * kTN * kGuKC];  // weight block scales [row][block], fp16
};
struct GuSmem {
    GuStage st[kGuStages];
    int32_t arow[kTM];
    int32_t pair[kTM];
    float w[kTM];
};
static_assert(sizeof(GuStage) % 16 == 0, "stage alignment");
static_assert(kTM * kTN * 4 <= (int)sizeof(GuStage), "SwiGLU exchange fits in one stage");

template <int H, bool DUMP>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4))) void gateup_mfma_kernel(LayerArgs a) {
    constexpr int NB = H / 32, NC = NB / kGuKC;
    static_assert(NC >= 2 && NB % kGuKC == 0, "K chunks");
    __shared__ __attribute__((aligned(16))) GuSmem sm;
    const int g = blockIdx.y;
    if (g >= a.ws.ctl[kCtlGroups]) return;
    const int4 grp = a.ws.groups[g];
    const bool shared = grp.x == a.d.E;
    const Dims &d = a.d;
    setup_tile(a, sm, grp, shared, false);
    const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, n = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int which = wave >> 2, wm = (wave >> 1) & 1, wn = wave & 1;  // which: 0 gate, 1 up
    const uint8_t *gmat = shared ? a.wt.sh_gate : a.wt.gate + grp.x * q8_bytes(d.F, H);
    const uint8_t *umat = shared ? a.wt.sh_up : a.wt.up + grp.x * q8_bytes(d.F, H);
    const int c0 = blockIdx.x * kTN;
    const uint32_t mat_bytes = (uint32_t)q8_bytes(d.F, H);

    // ---- this wave's four loads per chunk (byte offsets at chunk 0)
    const __amdgpu_buffer_rsrc_t r_xq = buf_rsrc(a.ws.xq, (uint32_t)((int64_t)d.T * H));
    const __amdgpu_buffer_rsrc_t r_gate = buf_rsrc(gmat, mat_bytes), r_up = buf_rsrc(umat, mat_bytes);
    const int lrow = 8 * wave + (lane >> 3), piece = (lane & 7) ^ (lane >> 3);
    const uint32_t off_a = (uint32_t)sm.arow[lrow] * H + 16 * piece;          // activation row lrow
    const uint32_t off_w = (uint32_t)(c0 + lrow) * H + 16 * piece;            // gate / up row lrow
    __amdgpu_buffer_rsrc_t r_s;
    uint32_t off_s;
    if (wave < 4) {  // activation scales: pairs 16 wave .. +15, 4 blocks each
        r_s = buf_rsrc(a.ws.xd, (uint32_t)((int64_t)d.T * (H / 32) * 4));
        off_s = ((uint32_t)sm.arow[16 * wave + (lane >> 2)] * (H / 32) + (lane & 3)) * 4;
    } else {         // weight scales: rows 32 (wave-4) .. +31 of B, two dwords (4 fp16) each
        const int row = 32 * (wave - 4) + (lane >> 1);
        r_s = wave < 6 ? r_gate : r_up;
        off_s = (uint32_t)d.F * H + (uint32_t)(c0 + (row & (kTN - 1))) * (H / 32) * 2 + 4 * (lane & 1);
    }
    auto issue = [&](int c, int stg) {
        GuStage &S = sm.st[stg];
        dma16(r_xq, &S.A[wave * 1024], off_a + c * kGuRow);
        dma16(r_gate, &S.B[wave * 1024], off_w + c * kGuRow);
        dma16(r_up, &S.B[kTN * kGuRow + wave * 1024], off_w + c * kGuRow);
        if (wave < 4) dma4(r_s, &S.sa[wave * 64], off_s + c * (kGuKC * 4));
        else dma4(r_s, &S.sw[(wave - 4) * 128], off_s + c * (kGuKC * 2));
    };

    // ---- this lane's LDS reads: operand rows and the swizzled slot of each block half
    const int am = wm * 32 + n, bj = which * kTN + wn * 32 + n;
    uint32_t slot[kGuKC];
#pragma unroll
    for (int kb = 0; kb < kGuKC; ++kb) slot[kb] = 16 * ((2 * kb + half) ^ (n & 7));
    const int col = c0 + wn * 32 + n;  // this lane's h column (gate/up row)
    const bool live = wm * 32 < grp.z;  // this wave's 32 pairs hold at least one real pair
    float acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.0f;

    issue(0, 0);
    issue(1, 1);
    auto compute = [&](int c, const GuStage &S) {
        auto block_mfma = [&](int kb) {
            const i32x4 av = *reinterpret_cast<const i32x4 *>(&S.A[am * kGuRow + slot[kb]]);
            const i32x4 bv = *reinterpret_cast<const i32x4 *>(&S.B[bj * kGuRow + slot[kb]]);
            const v16i zero = {};
            return __builtin_amdgcn_mfma_i32_32x32x32_i8(av, bv, zero, 0, 0, 0);
        };
        v16i cnext = block_mfma(0);
#pragma unroll
        for (int kb = 0; kb < kGuKC; kb += 2) {
            // scale products of blocks kb (registers 0..15) and kb+1 (16..31)
            const float dx = S.sa[am * kGuKC + kb + half];
            const float dw = f16_to_f32(S.sw[bj * kGuKC + kb + half]);
            const v32f pz = {};
            const v32f ps = __builtin_amdgcn_mfma_f32_32x32x1f32(dx, dw, pz, 0, 0, 0);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int b = c * kGuKC + kb + j;
                const v16i cv = cnext;
                if (kb + j + 1 < kGuKC) cnext = block_mfma(kb + j + 1);
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[i] = __fmaf_rn((float)cv[i], ps[16 * j + i], acc[i]);
                if (DUMP && (col % a.dump.stride == 0)) {
                    int32_t *dst = which ? a.dump.up_sums : a.dump.gate_sums;
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int m = wm * 32 + acc_row(i, lane);
                        if (m < grp.z)
                            dst[((int64_t)sm.pair[m] * (d.F / a.dump.stride) + col / a.dump.stride) * a.dump.pitch_gu +
                                b] = cv[i];
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
        if (c + 2 < NC) issue(c + 2, (stg + 2) % kGuStages);
        if (live) compute(c, sm.st[stg]);
    };
#pragma unroll 1
    for (int c = 0; c < NC; c += kGuStages) {
        step(c, std::integral_constant<int, 0>{});
        if (c + 1 < NC) step(c + 1, std::integral_constant<int, 1>{});
        if (c + 2 < NC) step(c + 2, std::integral_constant<int, 2>{});
    }
    // the up waves hand their sums to the gate waves through LDS (the ring is
    // drained: the last chunk waited for every load): SwiGLU, then quantize
    // each pair's 32 columns (the 32 lanes of a half-wave)
    __syncthreads();
    float *hx = reinterpret_cast<float *>(&sm.st[0]);  // [64 pairs][64 columns]
    if (which == 1) {
#pragma unroll
        for (int i = 0; i < 16; ++i) hx[(wm * 32 + acc_row(i, lane)) * kTN + wn * 32 + n] = acc[i];
    }
    __syncthreads();
    if (which == 0 && live) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int m = wm * 32 + acc_row(i, lane);
            const float hv = swiglu(acc[i], hx[m * kTN + wn * 32 + n]);
            const float amax = group_max<32>(fabsf(hv));
            const float dsc = quant_scale(amax);
            const float inv = dsc > 0.0f ? 1.0f / dsc : 0.0f;
            if (m < grp.z) {
                const int64_t p = sm.pair[m];
                a.ws.hq[p * d.F + col] = (int8_t)quant_code(hv, inv);
                if (n == 0) a.ws.hd[p * (d.F / 32) + col / 32] = dsc;
            }
        }
    }
}

// ------------------------------------------------------------------ down
template <int F, bool DUMP>
__global__ __launch_bounds__(256) void down_mfma_kernel(LayerArgs a) {
    constexpr int kKC = kKCDown, NB = F / 32, NC = NB / kKC, NBR = kTN;
    static_assert(NC >= 1 && NB % kKC == 0, "K chunks");
    __shared__ GemmSmem<NBR, kKC> sm;
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
    auto brow = [&](int j) { return std::make_pair(dmat, r0 + j); };
    const int row = r0 + wn * 32 + n;  // this lane's output row
    const int brow_lds = wn * 32 + n;
    float acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
    Stage<256, NBR, kKC> st;
    st.template setup<F>(sm, a.ws.hq, a.ws.hd, d.H, brow);
    st.load(0);
#pragma unroll 1
    for (int c = 0; c < NC; ++c) {
        __syncthreads();
        st.store(sm);
        __syncthreads();
        if (c + 1 < NC) st.load(c + 1);
#pragma unroll
        for (int kb = 0; kb < kKC; kb += 2) {
            // scale products of blocks kb (registers 0..15) and kb+1 (16..31)
            const float dh = sm.sa[kb + half][wm * 32 + n];
            const float dw = wscale(sm, brow_lds, kb + half);
            const v32f pz = {};
            const v32f ps = __builtin_amdgcn_mfma_f32_32x32x1f32(dh, dw, pz, 0, 0, 0);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int b = c * kKC + kb + j;
                const i32x4 av = *reinterpret_cast<const i32x4 *>(&sm.A[wm * 32 + n][(kb + j) * 32 + 16 * half]);
                const i32x4 wv = *reinterpret_cast<const i32x4 *>(&sm.B[wn * 32 + n][(kb + j) * 32 + 16 * half]);
                const v16i zero = {};
                const v16i cv = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, wv, zero, 0, 0, 0);
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[i] = __fmaf_rn((float)cv[i], ps[16 * j + i], acc[i]);
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
        case 256: klaunch(gateup_mfma_kernel<256, DUMP>, grid, 512, s, a); break;
        case 512: klaunch(gateup_mfma_kernel<512, DUMP>, grid, 512, s, a); break;
        case 1024: klaunch(gateup_mfma_kernel<1024, DUMP>, grid, 512, s, a); break;
        case 2048: klaunch(gateup_mfma_kernel<2048, DUMP>, grid, 512, s, a); break;
        case 4096: klaunch(gateup_mfma_kernel<4096, DUMP>, grid, 512, s, a); break;
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
