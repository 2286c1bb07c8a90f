// Expert FFN on the VALU for batches served from a work list: streams
// Q8_32 / Q2_256 weight rows from HBM with coalesced 16-byte loads and
// applies each row to up to 8 tokens of one expert, int8 x int8 -> int32
// block sums with v_dot4c_i32_i8, then the two block scales in fp32 (the
// quantized matvec path of "DwarfStar (ds4) — ROCm / gfx1151 fork",
// Performance optimizations: moe_gate_up_mid_* / moe_down_* and the q8_0
// "preq" matvecs).  Used for batches of 2..32 tokens (2-bit experts: up to
// 63), and for shapes below the MFMA GEMMs' minimum.
//
// Work list: groups {expert (E = shared), first index, count <= 8}; grid =
// (row chunks of 32 rows) x (groups).  Workgroups beyond the device-side
// group count exit at once.
#include "dev_vec.hpp"

namespace qrmoe {

template <int K, int FMT, bool DUMP>
__global__ __launch_bounds__(256) void gateup_vec_kernel(LayerArgs a) {
    __shared__ VecSmem<K, kVecTok> sm;
    const int g = blockIdx.y;
    const int ngroups = a.ws.ctl[kCtlGroups];
    const int4 grp = a.ws.groups[g];  // in the allocation for every g of the grid; used only when g < ngroups
    if (g >= ngroups) return;
    const bool shared = grp.x == a.d.E;
    const int tid = threadIdx.x;
    const int r0 = blockIdx.x * kVecRows;
    // the group's pairs are requested before the weight rows (a wave waits for
    // loads in issue order); their x rows are staged while the rows stream in
    int p = 0;
    if (tid < grp.z) p = shared ? a.d.T * a.d.k + grp.y + tid : a.ws.perm[grp.y + tid];
    auto stage = [&](bool s16) {
        if (tid < grp.z) {
            sm.pair[tid] = p;
            sm.row[tid] = shared ? grp.y + tid : p / a.d.k;
        }
        __syncthreads();
        if (s16) stage_rows<K, kVecTok, true>(sm, a.ws.xq, a.ws.xd, a.ws.xs16, grp.z);
        else stage_rows<K, kVecTok, false>(sm, a.ws.xq, a.ws.xd, nullptr, grp.z);
        __syncthreads();
    };
    if (shared) {
        gateup_rows<K, kFmtQ8, kVecTok, kVecRows, DUMP>(a, sm, a.wt.sh_gate, a.wt.sh_up, grp.z, r0,
                                                             [&] { stage(false); });
    } else {
        const int64_t mb = mat_bytes(FMT, a.d.F, K);
        gateup_rows<K, FMT, kVecTok, kVecRows, DUMP>(a, sm, a.wt.gate + grp.x * mb, a.wt.up + grp.x * mb, grp.z,
                                                          r0, [&] { stage(FMT == kFmtQ2); });
    }
}

// y[p][r] = w_p * (down row r . h_p) for rows r0..r0+31 of one expert.  The
// lane geometry L is the routed format's for every expert (the shared Q8
// expert included), the same one the one-token down kernel uses, so a token's
// y values do not depend on the batch it is served in.  Rows of the next two
// passes stay in flight; the first two are requested before `stage()` (the
// caller's staging of h, ending with a barrier).
template <int K, int FMT, int L, bool DUMP, class Stage>
__device__ void down_rows(const LayerArgs &a, VecSmem<K, kVecTok> &sm, const uint8_t *__restrict__ dmat, int cnt,
                          int r0, Stage stage) {
    using G = Geo<K, FMT, L>;
    using RR = RowRegs<K, FMT, G::L>;
    constexpr int PASSES = kVecRows / (4 * G::RPW);
    static_assert(PASSES >= 1 && kVecRows % (4 * G::RPW) == 0, "row geometry");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const Dims &d = a.d;
    const int seg = lane % G::L, rsub = lane / G::L;
    auto row_of = [&](int pass) { return (pass * 4 + wave) * G::RPW + rsub; };
    RR w0, w1;
    w0.load(dmat, d.H, r0 + row_of(0), seg);
    if (PASSES > 1) w1.load(dmat, d.H, r0 + row_of(1), seg);
    stage();
#pragma unroll
    for (int pass = 0; pass < PASSES; ++pass) {
        RR nw;
        if (pass + 2 < PASSES) nw.load(dmat, d.H, r0 + row_of(pass + 2), seg);
        const int r = r0 + row_of(pass);
        const bool dump_row = DUMP && (r % a.dump.stride == 0);
        for (int tok = 0; tok < cnt; ++tok) {
            int32_t *dd = nullptr;
            if (dump_row)
                dd = a.dump.down_sums +
                     ((int64_t)sm.pair[tok] * (d.H / a.dump.stride) + r / a.dump.stride) * a.dump.pitch_dn;
            const float y = group_sum<G::L>(lane_dot<K, G::L>(w0, sm.aq[tok], sm.ad[tok], sm.as16[tok], seg, dd));
            if (seg == 0) a.ws.y[(int64_t)sm.pair[tok] * d.H + r] = __fmul_rn(sm.w[tok], y);
        }
        w0 = w1;
        w1 = nw;
    }
}

template <int K, int FMT, bool DUMP>
__global__ __launch_bounds__(256) void down_vec_kernel(LayerArgs a) {
    __shared__ VecSmem<K, kVecTok> sm;
    const int g = blockIdx.y;
    const int ngroups = a.ws.ctl[kCtlGroups];
    const int4 grp = a.ws.groups[g];  // in the allocation for every g of the grid; used only when g < ngroups
    if (g >= ngroups) return;
    const bool shared = grp.x == a.d.E;
    const int tid = threadIdx.x;
    const int r0 = blockIdx.x * kVecRows;
    constexpr int L = DefLpr<K, FMT>::v;
    // pairs and combine weights are requested before the weight rows
    int p = 0;
    if (tid < grp.z) p = shared ? a.d.T * a.d.k + grp.y + tid : a.ws.perm[grp.y + tid];
    float wp = 1.0f;
    if (tid < grp.z && !shared) wp = a.ws.w[p];
    auto stage = [&](bool sums) {
        if (tid < grp.z) {
            sm.pair[tid] = p;
            sm.row[tid] = p;  // h is stored per pair
            sm.w[tid] = wp;
        }
        __syncthreads();
        stage_rows<K, kVecTok, false>(sm, a.ws.hq, a.ws.hd, nullptr, grp.z);
        __syncthreads();
        if (sums) {
            subblock_sums(sm, grp.z);
            __syncthreads();
        }
    };
    if (shared) {
        down_rows<K, kFmtQ8, L, DUMP>(a, sm, a.wt.sh_down, grp.z, r0, [&] { stage(false); });
    } else {
        const int64_t mb = mat_bytes(FMT, a.d.H, K);
        down_rows<K, FMT, L, DUMP>(a, sm, a.wt.down + grp.x * mb, grp.z, r0, [&] { stage(FMT == kFmtQ2); });
    }
}

// out[t][r] = sum over t's experts in ascending id of y[t*k + j][r], then the
// shared expert's y.  Workgroup (x, t): rows [1024x, 1024x + 1024) of token t,
// 4 consecutive rows per thread; the token's order of experts is found once.
__global__ __launch_bounds__(256) void combine_kernel(LayerArgs a) {
    const Dims &d = a.d;
    const int t = blockIdx.y;
    const int r = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (r >= d.H) return;
    int e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = j < d.k ? a.ws.ids[t * d.k + j] : 0x7fffffff;
    float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    auto add = [&](int64_t pair) {
        const float4 v = *reinterpret_cast<const float4 *>(a.ws.y + pair * d.H + r);
        acc.x = __fadd_rn(acc.x, v.x);
        acc.y = __fadd_rn(acc.y, v.y);
        acc.z = __fadd_rn(acc.z, v.z);
        acc.w = __fadd_rn(acc.w, v.w);
    };
    int prev = -1;
    for (int step = 0; step < d.k; ++step) {
        int best = 0x7fffffff, bj = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (e[j] > prev && e[j] < best) {
                best = e[j];
                bj = j;
            }
        if (best == 0x7fffffff) break;  // a repeated id (unchecked hash table) is summed once
        add((int64_t)t * d.k + bj);
        prev = best;
    }
    if (d.has_shared) add((int64_t)d.T * d.k + t);
    *reinterpret_cast<float4 *>(a.out + (int64_t)t * d.H + r) = acc;
}

// ------------------------------------------------------------- launchers
template <int FMT, bool DUMP>
static hipError_t gateup_k(const LayerArgs &a, dim3 grid, hipStream_t s) {
    switch (a.d.H) {
        case 128: if constexpr (FMT == kFmtQ8) { klaunch(gateup_vec_kernel<128, FMT, DUMP>, grid, 256, s, a); break; } return hipErrorInvalidValue;
        case 256: if constexpr (FMT == kFmtQ8) { klaunch(gateup_vec_kernel<256, FMT, DUMP>, grid, 256, s, a); break; } return hipErrorInvalidValue;
        case 512: klaunch(gateup_vec_kernel<512, FMT, DUMP>, grid, 256, s, a); break;
        case 1024: klaunch(gateup_vec_kernel<1024, FMT, DUMP>, grid, 256, s, a); break;
        case 2048: klaunch(gateup_vec_kernel<2048, FMT, DUMP>, grid, 256, s, a); break;
        case 4096: klaunch(gateup_vec_kernel<4096, FMT, DUMP>, grid, 256, s, a); break;
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
        case 128: if constexpr (FMT == kFmtQ8) { klaunch(down_vec_kernel<128, FMT, DUMP>, grid, 256, s, a); break; } return hipErrorInvalidValue;
        case 256: if constexpr (FMT == kFmtQ8) { klaunch(down_vec_kernel<256, FMT, DUMP>, grid, 256, s, a); break; } return hipErrorInvalidValue;
        case 512: klaunch(down_vec_kernel<512, FMT, DUMP>, grid, 256, s, a); break;
        case 1024: klaunch(down_vec_kernel<1024, FMT, DUMP>, grid, 256, s, a); break;
        case 2048: klaunch(down_vec_kernel<2048, FMT, DUMP>, grid, 256, s, a); break;
        case 4096: klaunch(down_vec_kernel<4096, FMT, DUMP>, grid, 256, s, a); break;
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
    klaunch(combine_kernel, dim3((a.d.H + 1023) / 1024, a.d.T), dim3(256), s, a);
    return hipGetLastError();
}

}  // namespace qrmoe
