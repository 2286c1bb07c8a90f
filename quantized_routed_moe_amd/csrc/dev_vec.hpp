// Device helpers of the VALU expert kernels: lane geometry, weight-row
// registers, int8 x int8 block dot products (v_dot4c_i32_i8) with the two
// block scales, activation staging, SwiGLU and the h quantizer.
#pragma once

#include "common.hpp"

namespace qrmoe {

// LDS of one workgroup: quantized activations of up to NTOK tokens, their
// block scales, (2-bit weights) their 16-subblock code sums, h of 32 rows.
template <int K, int NTOK>
struct VecSmem {
    alignas(16) int8_t aq[NTOK][K];
    float ad[NTOK][K / 32];
    int32_t as16[NTOK][K / 16];
    float h[NTOK][2 * kVecRows];  // up to 64 rows of h per workgroup
    int32_t pair[NTOK];
    int32_t row[NTOK];
    float w[NTOK];
};

// Default lanes per weight row: Q8 rows are cut in 16-byte chunks (half
// blocks), Q2 rows in 64-weight pieces (16 code bytes, 4 subblocks).
template <int K, int FMT>
struct DefLpr {
    static constexpr int v = FMT == kFmtQ8 ? (K / 16 < 64 ? K / 16 : 64) : (K / 64 < 64 ? K / 64 : 64);
};

template <int K, int FMT, int LPR = DefLpr<K, FMT>::v>
struct Geo {
    static constexpr int L = LPR;
    static constexpr int J = FMT == kFmtQ8 ? K / (16 * LPR) : K / (64 * LPR);  // chunks per lane
    static constexpr int RPW = 64 / LPR;                                       // rows per wave pass
    static_assert(J >= 1 && LPR <= 64 && (FMT == kFmtQ8 || J == 1), "lane geometry");
};

// One lane's part of one weight row.  Q8: chunk j is 16 code bytes at
// 16*(seg + LPR*j) with the fp16 scale of its 32-block.  Q2: 64 weights at
// 64*seg: 16 code bytes, 4 scale/min bytes, and the superblock's d, dmin.
template <int K, int FMT, int LPR>
struct RowRegs;

// Scales stay as raw fp16 bits until the dot product uses them: converting at
// load time would make the wave wait for the loads it has just issued (loads
// retire in order), which turns a prefetch into a synchronous read.
template <int K, int LPR>
struct RowRegs<K, kFmtQ8, LPR> {
    static constexpr int J = Geo<K, kFmtQ8, LPR>::J;
    int4 c[J];
    uint32_t s16[J];  // one zero-extended fp16 per register (no packing, which would wait for the load)
    __device__ __forceinline__ void load(const uint8_t *__restrict__ mat, int64_t R, int64_t r, int seg) {
        const int4 *codes = reinterpret_cast<const int4 *>(mat + r * K);
        const uint16_t *sc = reinterpret_cast<const uint16_t *>(mat + R * K) + r * (K / 32);
#pragma unroll
        for (int j = 0; j < J; ++j) {
            c[j] = load_stream16(codes + seg + LPR * j);
            s16[j] = sc[(seg + LPR * j) >> 1];
        }
    }
    // the empty asm keeps the conversion (and so the wait for the load) at the use
    __device__ __forceinline__ float scale(int j) const {
        uint32_t v = s16[j];
        asm volatile("" : "+v"(v));
        return f16_to_f32((uint16_t)v);
    }
};

template <int K, int LPR>
struct RowRegs<K, kFmtQ2, LPR> {
    int4 c;
    uint32_t sm;
    uint32_t dd;  // fp16 d (low half), fp16 dmin (high half)
    __device__ __forceinline__ void load(const uint8_t *__restrict__ mat, int64_t R, int64_t r, int seg) {
        c = load_stream16(reinterpret_cast<const int4 *>(mat + r * (K / 4)) + seg);
        sm = *reinterpret_cast<const uint32_t *>(mat + R * K / 4 + r * (K / 16) + 4 * seg);
        dd = *reinterpret_cast<const uint32_t *>(mat + R * K / 4 + R * K / 16 + (r * (K / 256) + seg / 4) * 4);
    }
    __device__ __forceinline__ uint32_t raw() const {
        uint32_t v = dd;
        asm volatile("" : "+v"(v));  // keeps the conversion (and the wait for the load) at the use
        return v;
    }
    __device__ __forceinline__ float d() const { return f16_to_f32((uint16_t)(raw() & 0xffff)); }
    __device__ __forceinline__ float dmin() const { return f16_to_f32((uint16_t)(raw() >> 16)); }
};

// Partial dot of one lane's part of a row with a quantized activation row
// (floating-point steps written with explicit rounding intrinsics so that
// every kernel inlining this computes bit-identical partials)
// (aq: K int8 codes, ad: K/32 scales, as16: K/16 subblock code sums, all in
// LDS).  With dump != nullptr the exact int32 block sums are written: per
// 32-block (Q8; the two halves of a block sit in lanes seg, seg^1) or per
// 16-weight subblock (Q2).
template <int K, int LPR>
__device__ __forceinline__ float lane_dot(const RowRegs<K, kFmtQ8, LPR> &w, const int8_t *aq, const float *ad,
                                          const int32_t *, int seg, int32_t *dump) {
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < Geo<K, kFmtQ8, LPR>::J; ++j) {
        const int chunk = seg + LPR * j;
        const int4 x = *reinterpret_cast<const int4 *>(aq + chunk * 16);
        int I = sdot4(w.c[j].x, x.x, 0);
        I = sdot4(w.c[j].y, x.y, I);
        I = sdot4(w.c[j].z, x.z, I);
        I = sdot4(w.c[j].w, x.w, I);
        acc = __fmaf_rn((float)I, __fmul_rn(w.scale(j), ad[chunk >> 1]), acc);
        if (dump) {
            const int full = I + __shfl_xor(I, 1);
            if ((seg & 1) == 0) dump[chunk >> 1] = full;
        }
    }
    return acc;
}

template <int K, int LPR>
__device__ __forceinline__ float lane_dot(const RowRegs<K, kFmtQ2, LPR> &w, const int8_t *aq, const float *ad,
                                          const int32_t *as16, int seg, int32_t *dump) {
    const int4 *xp = reinterpret_cast<const int4 *>(aq + 64 * seg);
    const int words[4] = {w.c.x, w.c.y, w.c.z, w.c.w};
    int SP[2] = {0, 0}, SM[2] = {0, 0};
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
        const int4 x = xp[jj];
        const uint32_t wv = (uint32_t)words[jj];
        int P = sdot4((int)(wv & 0x03030303u), x.x, 0);
        P = sdot4((int)((wv >> 2) & 0x03030303u), x.y, P);
        P = sdot4((int)((wv >> 4) & 0x03030303u), x.z, P);
        P = sdot4((int)((wv >> 6) & 0x03030303u), x.w, P);
        const int s = (int)((w.sm >> (8 * jj)) & 15u), m = (int)((w.sm >> (8 * jj + 4)) & 15u);
        // 24-bit multiplies (full rate): s, m < 16, |P| <= 16*3*127 and
        // |as16| <= 16*127, so every product is exact in 24 bits
        SP[jj >> 1] += __mul24(s, P);
        SM[jj >> 1] += __mul24(m, as16[4 * seg + jj]);
        if (dump) dump[4 * seg + jj] = P;
    }
    // explicit roundings: the same value in every kernel that inlines this
    const float wd = w.d(), wm = w.dmin();
    const float b0 = __fsub_rn(__fmul_rn(wd, (float)SP[0]), __fmul_rn(wm, (float)SM[0]));
    const float b1 = __fsub_rn(__fmul_rn(wd, (float)SP[1]), __fmul_rn(wm, (float)SM[1]));
    return __fadd_rn(__fmul_rn(ad[2 * seg], b0), __fmul_rn(ad[2 * seg + 1], b1));
}

// Copy the quantized rows `rows[0..cnt)` of (q, dq, s16) into LDS slots 0..cnt.
// Each iteration requests its code chunk, scale and subblock sum together
// before storing them, so a wave waits for its loads once per iteration.
template <int K, int NTOK, bool S16>
__device__ __forceinline__ void stage_rows(VecSmem<K, NTOK> &sm, const int8_t *__restrict__ q,
                                           const float *__restrict__ dq, const int32_t *__restrict__ s16, int cnt) {
    for (int i = threadIdx.x; i < cnt * (K / 16); i += 256) {
        const int tok = i / (K / 16), c = i % (K / 16);
        const int4 v = reinterpret_cast<const int4 *>(q + (int64_t)sm.row[tok] * K)[c];
        const bool has_scale = i < cnt * (K / 32);
        const int stok = i / (K / 32), b = i % (K / 32);
        float sc = 0.0f;
        if (has_scale) sc = dq[(int64_t)sm.row[stok] * (K / 32) + b];
        int32_t sum16 = 0;
        if constexpr (S16) sum16 = s16[(int64_t)sm.row[tok] * (K / 16) + c];
        reinterpret_cast<int4 *>(sm.aq[tok])[c] = v;
        if (has_scale) sm.ad[stok][b] = sc;
        if constexpr (S16) sm.as16[tok][c] = sum16;
    }
}

// Sums of the staged codes over 16-subblocks (for 2-bit weights applied to h).
template <int K, int NTOK>
__device__ __forceinline__ void subblock_sums(VecSmem<K, NTOK> &sm, int cnt) {
    for (int i = threadIdx.x; i < cnt * (K / 16); i += 256) {
        const int tok = i / (K / 16), g = i % (K / 16);
        const int4 v = reinterpret_cast<const int4 *>(sm.aq[tok])[g];
        int s = sdot4(v.x, 0x01010101, 0);
        s = sdot4(v.y, 0x01010101, s);
        s = sdot4(v.z, 0x01010101, s);
        s = sdot4(v.w, 0x01010101, s);
        sm.as16[tok][g] = s;
    }
}

__device__ __forceinline__ float swiglu(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// Ring depth of gate/up rows (row passes held by a wave): the current pass
// and the next two in flight.  (Six for the small 2-bit rows measured
// slower: the one-token 2-bit gate/up is not bound by rows in flight.)
template <int K, int FMT>
struct GuDepth {
    static constexpr int v = 3;
};

// Gate/up of one expert for rows r0..r0+ROWS-1 and the cnt staged tokens,
// then SwiGLU, and the quantization of each token's 32-row h blocks into
// hq/hd.  sm.pair[] names the output pair of each token.
//
// Each wave keeps the rows of the next DEPTH - 1 passes in flight (a ring of
// DEPTH gate and up rows, indexed at compile time).  The first DEPTH - 1 are
// requested before `stage()` (the caller's activation staging, which ends
// with a barrier), so weight streaming starts as soon as the expert is known.
// NW waves per workgroup, whose NW*64 threads cover (at least) NTOK tokens x
// ROWS rows of h (ROWS a multiple of the 32-row h block).
template <int K, int FMT, int NTOK, int ROWS, bool DUMP, int NW = 4, class Stage>
__device__ void gateup_rows(const LayerArgs &a, VecSmem<K, NTOK> &sm, const uint8_t *__restrict__ gmat,
                            const uint8_t *__restrict__ umat, int cnt, int r0, Stage stage) {
    using G = Geo<K, FMT>;
    using RR = RowRegs<K, FMT, G::L>;
    constexpr int PASSES = ROWS / (NW * G::RPW);
    constexpr int DEPTH = GuDepth<K, FMT>::v < PASSES + 1 ? GuDepth<K, FMT>::v : PASSES + 1;
    static_assert(PASSES >= 1 && ROWS % (NW * G::RPW) == 0, "row geometry");
    static_assert(ROWS % kVecRows == 0 && ROWS <= 2 * kVecRows && NW * 64 >= NTOK * ROWS, "h blocks");
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const Dims &d = a.d;
    const int seg = lane % G::L, rsub = lane / G::L;
    auto row_of = [&](int pass) { return (pass * NW + wave) * G::RPW + rsub; };
    RR wg[DEPTH], wu[DEPTH];
#pragma unroll
    for (int q = 0; q < DEPTH - 1; ++q)
        if (q < PASSES) {
            wg[q].load(gmat, d.F, r0 + row_of(q), seg);
            wu[q].load(umat, d.F, r0 + row_of(q), seg);
        }
    stage();
#pragma unroll
    for (int pass = 0; pass < PASSES; ++pass) {
        if (pass + DEPTH - 1 < PASSES) {
            wg[(pass + DEPTH - 1) % DEPTH].load(gmat, d.F, r0 + row_of(pass + DEPTH - 1), seg);
            wu[(pass + DEPTH - 1) % DEPTH].load(umat, d.F, r0 + row_of(pass + DEPTH - 1), seg);
        }
        const RR &g0 = wg[pass % DEPTH], &u0 = wu[pass % DEPTH];
        const int row_local = row_of(pass);
        const int r = r0 + row_local;
        const bool dump_row = DUMP && (r % a.dump.stride == 0);
        for (int tok = 0; tok < cnt; ++tok) {
            int32_t *dg = nullptr, *du = nullptr;
            if (dump_row) {
                const int64_t base =
                    ((int64_t)sm.pair[tok] * (d.F / a.dump.stride) + r / a.dump.stride) * a.dump.pitch_gu;
                dg = a.dump.gate_sums + base;
                du = a.dump.up_sums + base;
            }
            const float gp = group_sum<G::L>(lane_dot<K, G::L>(g0, sm.aq[tok], sm.ad[tok], sm.as16[tok], seg, dg));
            const float up = group_sum<G::L>(lane_dot<K, G::L>(u0, sm.aq[tok], sm.ad[tok], sm.as16[tok], seg, du));
            if (seg == 0) sm.h[tok][row_local] = swiglu(gp, up);
        }
    }
    __syncthreads();
    const int tok = tid / ROWS, i = tid % ROWS;  // 32 consecutive lanes = one h block of one token (tok < NTOK...)
    const float v = tok < cnt ? sm.h[tok][i] : 0.0f;
    const float amax = group_max<32>(fabsf(v));
    if (tok < cnt) {
        const float dsc = quant_scale(amax);
        const float inv = dsc > 0.0f ? 1.0f / dsc : 0.0f;
        const int p = sm.pair[tok];
        a.ws.hq[(int64_t)p * d.F + r0 + i] = (int8_t)quant_code(v, inv);
        if (i % 32 == 0) a.ws.hd[(int64_t)p * (d.F / 32) + (r0 + i) / 32] = dsc;
    }
}

}  // namespace qrmoe
