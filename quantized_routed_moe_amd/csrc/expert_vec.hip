// Expert FFN on the VALU: streams Q8_32 / Q2_256 weight rows from HBM with
// coalesced 16-byte loads and applies each row to up to 8 tokens of one
// expert, int8 x int8 -> int32 block sums with v_dot4c_i32_i8, then the two
// block scales in fp32.  Used for decode-sized batches (the quantized
// matvec path: "DwarfStar (ds4) — ROCm / gfx1151 fork", Performance
// optimizations, moe_gate_up_mid_decode_* / moe_down_sum6_* and the q8_0
// "preq" matvecs) and for 2-bit experts at any batch size.
//
// Work list: groups {expert, first pair, count <= 8}; grid = (row chunks of
// 32 rows) x (groups).  Workgroups beyond the device-side group count exit.
#include "common.hpp"

namespace qrmoe {

template <int K>
struct VecSmem {
    alignas(16) int8_t aq[kVecTok][K];  // quantized activations of the group's tokens
    float ad[kVecTok][K / 32];          // their block scales
    int32_t as16[kVecTok][K / 16];      // sums of the codes over 16-subblocks (2-bit weights)
    float h[kVecTok][kVecRows];
    int32_t pair[kVecTok];
};

// Lane geometry.  Q8: each lane owns J 16-byte chunks (half blocks) of a row,
// chunk j at byte (seg + LPR*j)*16.  Q2: each lane owns 64 weights (16 code
// bytes, 4 subblocks, 2 activation blocks).
template <int K, int FMT>
struct Geo {
    static constexpr int LPR = FMT == kFmtQ8 ? (K / 16 < 64 ? K / 16 : 64) : (K / 64 < 64 ? K / 64 : 64);
    static constexpr int J = FMT == kFmtQ8 ? K / (16 * LPR) : 1;
    static constexpr int RPW = 64 / LPR;
    static constexpr int PASSES = kVecRows / (4 * RPW);
    static_assert(PASSES >= 1 && kVecRows % (4 * RPW) == 0, "row geometry");
};

// Row data of one matrix row held by one lane.
template <int K, int FMT>
struct RowRegs;

template <int K>
struct RowRegs<K, kFmtQ8> {
    int4 c[Geo<K, kFmtQ8>::J];
    float s[Geo<K, kFmtQ8>::J];
    __device__ __forceinline__ void load(const uint8_t *__restrict__ mat, int64_t R, int64_t r, int seg) {
        constexpr int LPR = Geo<K, kFmtQ8>::LPR;
        const int4 *codes = reinterpret_cast<const int4 *>(mat + r * K);
        const uint16_t *sc = reinterpret_cast<const uint16_t *>(mat + R * K) + r * (K / 32);
#pragma unroll
        for (int j = 0; j < Geo<K, kFmtQ8>::J; ++j) {
            c[j] = load_stream16(codes + seg + LPR * j);
            s[j] = f16_to_f32(sc[(seg + LPR * j) >> 1]);
        }
    }
};

template <int K>
struct RowRegs<K, kFmtQ2> {
    int4 c;
    uint32_t sm;
    float d, dmin;
    __device__ __forceinline__ void load(const uint8_t *__restrict__ mat, int64_t R, int64_t r, int seg) {
        c = load_stream16(reinterpret_cast<const int4 *>(mat + r * (K / 4)) + seg);
        sm = *reinterpret_cast<const uint32_t *>(mat + R * K / 4 + r * (K / 16) + 4 * seg);
        const uint32_t dd = *reinterpret_cast<const uint32_t *>(mat + R * K / 4 + R * K / 16 + (r * (K / 256) + seg / 4) * 4);
        d = f16_to_f32((uint16_t)(dd & 0xffff));
        dmin = f16_to_f32((uint16_t)(dd >> 16));
    }
};

// Partial dot product of one lane's part of a row with one token's quantized
// activation (in LDS).  Writes exact integer block sums when dump != nullptr.
template <int K>
__device__ __forceinline__ float lane_dot(const RowRegs<K, kFmtQ8> &w, const VecSmem<K> &sm, int tok, int seg,
                                          int32_t *dump) {
    constexpr int LPR = Geo<K, kFmtQ8>::LPR;
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < Geo<K, kFmtQ8>::J; ++j) {
        const int chunk = seg + LPR * j;
        const int4 x = *reinterpret_cast<const int4 *>(&sm.aq[tok][chunk * 16]);
        int I = sdot4(w.c[j].x, x.x, 0);
        I = sdot4(w.c[j].y, x.y, I);
        I = sdot4(w.c[j].z, x.z, I);
        I = sdot4(w.c[j].w, x.w, I);
        acc += (float)I * (w.s[j] * sm.ad[tok][chunk >> 1]);
        if (dump) {
            const int full = I + __shfl_xor(I, 1);  // the two halves of the 32-block sit in lanes seg, seg^1
            if ((seg & 1) == 0) dump[chunk >> 1] = full;
        }
    }
    return acc;
}

template <int K>
__device__ __forceinline__ float lane_dot(const RowRegs<K, kFmtQ2> &w, const VecSmem<K> &sm, int tok, int seg,
                                          int32_t *dump) {
    const int4 *xp = reinterpret_cast<const int4 *>(&sm.aq[tok][64 * seg]);
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
        SP[jj >> 1] += s * P;
        SM[jj >> 1] += m * sm.as16[tok][4 * seg + jj];
        if (dump) dump[4 * seg + jj] = P;
    }
    return sm.ad[tok][2 * seg] * (w.d * (float)SP[0] - w.dmin * (float)SM[0]) +
           sm.ad[tok][2 * seg + 1] * (w.d * (float)SP[1] - w.dmin * (float)SM[1]);
}

// Stage the quantized activations of `cnt` tokens into LDS.
template <int K, int FMT>
__device__ __forceinline__ void stage_acts(VecSmem<K> &sm, const int8_t *__restrict__ q, const float *__restrict__ dq,
                                           const int32_t *__restrict__ s16, const int *rows, int cnt) {
    const int tid = threadIdx.x;
    for (int i = tid; i < cnt * (K / 16); i += 256) {
        const int tok = i / (K / 16), c = i % (K / 16);
        reinterpret_cast<int4 *>(sm.aq[tok])[c] = reinterpret_cast<const int4 *>(q + (int64_t)rows[tok] * K)[c];
    }
    for (int i = tid; i < cnt * (K / 32); i += 256) {
        const int tok = i / (K / 32), b = i % (K / 32);
        sm.ad[tok][b] = dq[(int64_t)rows[tok] * (K / 32) + b];
    }
    if constexpr (FMT == kFmtQ2) {
        for (int i = tid; i < cnt * (K / 16); i += 256) {
            const int tok = i / (K / 16), g = i % (K / 16);
            sm.as16[tok][g] = s16[(int64_t)rows[tok] * (K / 16) + g];
        }
    }
}

__device__ __forceinline__ float swiglu(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// ------------------------------------------------------------- gate / up
template <int K, int FMT, bool DUMP>
__device__ void gateup_body(const LayerArgs &a, VecSmem<K> &sm, const uint8_t *__restrict__ gmat,
                            const uint8_t *__restrict__ umat, int4 grp, bool shared) {
    using G = Geo<K, FMT>;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const Dims &d = a.d;
    const int cnt = grp.z;
    const int r0 = blockIdx.x * kVecRows;
    __shared__ int tok_rows[kVecTok];
    if (tid < cnt) {
        const int p = shared ? d.T * d.k + grp.y + tid : a.ws.perm[grp.y + tid];
        sm.pair[tid] = p;
        tok_rows[tid] = shared ? grp.y + tid : p / d.k;
    }
    __syncthreads();
    stage_acts<K, FMT>(sm, a.ws.xq, a.ws.xd, a.ws.xs16, tok_rows, cnt);
    __syncthreads();
    const int seg = lane % G::LPR, rsub = lane / G::LPR;
    RowRegs<K, FMT> wg, wu;
    int row_local = wave * G::RPW + rsub;
    wg.load(gmat, d.F, r0 + row_local, seg);
    wu.load(umat, d.F, r0 + row_local, seg);
#pragma unroll 1
    for (int pass = 0; pass < G::PASSES; ++pass) {
        RowRegs<K, FMT> ng, nu;
        const int next_local = ((pass + 1) * 4 + wave) * G::RPW + rsub;
        if (pass + 1 < G::PASSES) {
            ng.load(gmat, d.F, r0 + next_local, seg);
            nu.load(umat, d.F, r0 + next_local, seg);
        }
        const int r = r0 + row_local;
        const bool dump_row = DUMP && (r % a.dump.stride == 0);
        for (int tok = 0; tok < cnt; ++tok) {
            int32_t *dg = nullptr, *du = nullptr;
            if (dump_row) {
                const int64_t base = ((int64_t)sm.pair[tok] * (d.F / a.dump.stride) + r / a.dump.stride) * a.dump.pitch_gu;
                dg = a.dump.gate_sums + base;
                du = a.dump.up_sums + base;
            }
            const float gp = group_sum<G::LPR>(lane_dot<K>(wg, sm, tok, seg, dg));
            const float up = group_sum<G::LPR>(lane_dot<K>(wu, sm, tok, seg, du));
            if (seg == 0) sm.h[tok][row_local] = swiglu(gp, up);
        }
        if (pass + 1 < G::PASSES) {
            wg = ng;
            wu = nu;
            row_local = next_local;
        }
    }
    __syncthreads();
    // quantize the 32-row h block of every token
    const int tok = tid >> 5, i = tid & 31;
    const float v = tok < cnt ? sm.h[tok][i] : 0.0f;
    const float amax = group_max<32>(fabsf(v));
    if (tok < cnt) {
        const float dsc = quant_scale(amax);
        const float inv = dsc > 0.0f ? 1.0f / dsc : 0.0f;
        const int p = sm.pair[tok];
        a.ws.hq[(int64_t)p * d.F + r0 + i] = (int8_t)quant_code(v, inv);
        if (i == 0) a.ws.hd[(int64_t)p * (d.F / 32) + r0 / 32] = dsc;
    }
}

template <int K, int FMT, bool DUMP>
__global__ __launch_bounds__(256) void gateup_vec_kernel(LayerArgs a) {
    __shared__ VecSmem<K> sm;
    const int g = blockIdx.y;
    if (g >= a.ws.ctl[kCtlGroups]) return;
    const int4 grp = a.ws.groups[g];
    if (grp.x == a.d.E) {
        gateup_body<K, kFmtQ8, DUMP>(a, sm, a.wt.sh_gate, a.wt.sh_up, grp, true);
    } else {
        const int64_t mb = mat_bytes(FMT, a.d.F, K);
        gateup_body<K, FMT, DUMP>(a, sm, a.wt.gate + grp.x * mb, a.wt.up + grp.x * mb, grp, false);
    }
}

// ------------------------------------------------------------------ down
// y[p][r] = w_p * (down row r . h_p).  The combine kernel then writes
// out[t][r] = sum over t's experts in ascending id of y + the shared expert's y.
__device__ __forceinline__ void combine_rows(const LayerArgs &a, int r0, int nrows, int t0, int t1) {
    const Dims &d = a.d;
    for (int idx = threadIdx.x; idx < (t1 - t0) * nrows; idx += 256) {
        const int t = t0 + idx / nrows, r = r0 + idx % nrows;
        const int32_t *ids = a.ws.ids + t * d.k;
        float acc = 0.0f;
        int prev = -1;
        for (int step = 0; step < d.k; ++step) {
            int best = 0x7fffffff, bj = 0;
            for (int j = 0; j < d.k; ++j) {
                const int e = ids[j];
                if (e > prev && e < best) {
                    best = e;
                    bj = j;
                }
            }
            if (best == 0x7fffffff) break;  // repeated expert ids (unchecked table): each id counted once per step
            acc += a.ws.y[(int64_t)(t * d.k + bj) * d.H + r];
            prev = best;
        }
        if (d.has_shared) acc += a.ws.y[(int64_t)(d.T * d.k + t) * d.H + r];
        a.out[(int64_t)t * d.H + r] = acc;
    }
}

template <int K, int FMT, bool DUMP>
__device__ void down_body(const LayerArgs &a, VecSmem<K> &sm, const uint8_t *__restrict__ dmat, int4 grp,
                          bool shared) {
    using G = Geo<K, FMT>;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const Dims &d = a.d;
    const int cnt = grp.z;
    const int r0 = blockIdx.x * kVecRows;
    __shared__ int prow[kVecTok];
    __shared__ float pw[kVecTok];
    if (tid < cnt) {
        const int p = shared ? d.T * d.k + grp.y + tid : a.ws.perm[grp.y + tid];
        sm.pair[tid] = p;
        prow[tid] = p;
        pw[tid] = shared ? 1.0f : a.ws.w[p];
    }
    __syncthreads();
    stage_acts<K, kFmtQ8>(sm, a.ws.hq, a.ws.hd, nullptr, prow, cnt);
    if constexpr (FMT == kFmtQ2) {
        __syncthreads();
        for (int i = tid; i < cnt * (K / 16); i += 256) {
            const int tok = i / (K / 16), g = i % (K / 16);
            int s = 0;
#pragma unroll
            for (int c = 0; c < 16; ++c) s += sm.aq[tok][16 * g + c];
            sm.as16[tok][g] = s;
        }
    }
    __syncthreads();
    const int seg = lane % G::LPR, rsub = lane / G::LPR;
    RowRegs<K, FMT> wr;
    int row_local = wave * G::RPW + rsub;
    wr.load(dmat, d.H, r0 + row_local, seg);
#pragma unroll 1
    for (int pass = 0; pass < G::PASSES; ++pass) {
        RowRegs<K, FMT> nr;
        const int next_local = ((pass + 1) * 4 + wave) * G::RPW + rsub;
        if (pass + 1 < G::PASSES) nr.load(dmat, d.H, r0 + next_local, seg);
        const int r = r0 + row_local;
        const bool dump_row = DUMP && (r % a.dump.stride == 0);
        for (int tok = 0; tok < cnt; ++tok) {
            int32_t *dd = nullptr;
            if (dump_row)
                dd = a.dump.down_sums + ((int64_t)sm.pair[tok] * (d.H / a.dump.stride) + r / a.dump.stride) * a.dump.pitch_dn;
            const float y = group_sum<G::LPR>(lane_dot<K>(wr, sm, tok, seg, dd));
            if (seg == 0) a.ws.y[(int64_t)sm.pair[tok] * d.H + r] = pw[tok] * y;
        }
        if (pass + 1 < G::PASSES) {
            wr = nr;
            row_local = next_local;
        }
    }
}

template <int K, int FMT, bool DUMP>
__global__ __launch_bounds__(256) void down_vec_kernel(LayerArgs a) {
    __shared__ VecSmem<K> sm;
    const int g = blockIdx.y;
    if (g >= a.ws.ctl[kCtlGroups]) return;
    const int4 grp = a.ws.groups[g];
    if (grp.x == a.d.E) {
        down_body<K, kFmtQ8, DUMP>(a, sm, a.wt.sh_down, grp, true);
    } else {
        const int64_t mb = mat_bytes(FMT, a.d.H, K);
        down_body<K, FMT, DUMP>(a, sm, a.wt.down + grp.x * mb, grp, false);
    }
}

// Batched combine: workgroup (x, y) covers 32 output rows x 8 tokens.
__global__ __launch_bounds__(256) void combine_kernel(LayerArgs a) {
    const int t0 = blockIdx.y * 8;
    combine_rows(a, blockIdx.x * kVecRows, kVecRows, t0, min(t0 + 8, a.d.T));
}

// ------------------------------------------------------------- launchers
template <int FMT, bool DUMP>
static hipError_t gateup_k(const LayerArgs &a, dim3 grid, hipStream_t s) {
    switch (a.d.H) {
        case 128: if constexpr (FMT == kFmtQ8) { gateup_vec_kernel<128, FMT, DUMP><<<grid, 256, 0, s>>>(a); break; } return hipErrorInvalidValue;
        case 256: if constexpr (FMT == kFmtQ8) { gateup_vec_kernel<256, FMT, DUMP><<<grid, 256, 0, s>>>(a); break; } return hipErrorInvalidValue;
        case 512: gateup_vec_kernel<512, FMT, DUMP><<<grid, 256, 0, s>>>(a); break;
        case 1024: gateup_vec_kernel<1024, FMT, DUMP><<<grid, 256, 0, s>>>(a); break;
        case 2048: gateup_vec_kernel<2048, FMT, DUMP><<<grid, 256, 0, s>>>(a); break;
        case 4096: gateup_vec_kernel<4096, FMT, DUMP><<<grid, 256, 0, s>>>(a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_gateup_vec(const LayerArgs &a, int max_groups, bool dump, hipStream_t s) {
    dim3 grid(a.d.F / kVecRows, max_groups);
    if (a.d.fmt == kFmtQ8) return dump ? gateup_k<kFmtQ8, true>(a, grid, s) : gateup_k<kFmtQ8, false>(a, grid, s);
    return dump ? gateup_k<kFmtQ2, true>(a, grid, s) : gateup_k<kFmtQ2, false>(a, grid, s);
}

template <int FMT, bool DUMP>
static hipError_t down_k(const LayerArgs &a, dim3 grid, hipStream_t s) {
    switch (a.d.F) {
        case 128: if constexpr (FMT == kFmtQ8) { down_vec_kernel<128, FMT, DUMP><<<grid, 256, 0, s>>>(a); break; } return hipErrorInvalidValue;
        case 256: if constexpr (FMT == kFmtQ8) { down_vec_kernel<256, FMT, DUMP><<<grid, 256, 0, s>>>(a); break; } return hipErrorInvalidValue;
        case 512: down_vec_kernel<512, FMT, DUMP><<<grid, 256, 0, s>>>(a); break;
        case 1024: down_vec_kernel<1024, FMT, DUMP><<<grid, 256, 0, s>>>(a); break;
        case 2048: down_vec_kernel<2048, FMT, DUMP><<<grid, 256, 0, s>>>(a); break;
        case 4096: down_vec_kernel<4096, FMT, DUMP><<<grid, 256, 0, s>>>(a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_down_vec(const LayerArgs &a, int max_groups, bool dump, hipStream_t s) {
    dim3 grid(a.d.H / kVecRows, max_groups);
    if (a.d.fmt == kFmtQ8) return dump ? down_k<kFmtQ8, true>(a, grid, s) : down_k<kFmtQ8, false>(a, grid, s);
    return dump ? down_k<kFmtQ2, true>(a, grid, s) : down_k<kFmtQ2, false>(a, grid, s);
}

hipError_t launch_combine(const LayerArgs &a, hipStream_t s) {
    combine_kernel<<<dim3(a.d.H / kVecRows, (a.d.T + 7) / 8), dim3(256), 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace qrmoe
