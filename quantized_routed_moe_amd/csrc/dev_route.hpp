// Device helpers of the routing stage: activation quantizer, fp64 pairwise
// router logits, top-k and hash selection (see route.hip for the definitions
// they implement).
#pragma once

#include <climits>
#include <cmath>

#include "common.hpp"

namespace qrmoe {

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

// Score and selection key of one (token, expert): s = sigmoid(l) (fp64,
// rounded once), key = s + bias (one fp32 add).
__device__ __forceinline__ void score_key(float l, const float *bias, int e, float *score, float *key) {
    const float sc = score_of(l);
    *score = sc;
    *key = sc + (bias ? bias[e] : 0.0f);
}

// Order-preserving image of an fp32 key in the unsigned integers (IEEE total
// order on finite values; -0 maps with +0).  Every finite key maps above 0.
__device__ __forceinline__ uint32_t key_order(float key) {
    const uint32_t u = __float_as_uint(key == 0.0f ? 0.0f : key);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One wave selects the top-k (k <= 8 <= E) experts of one token from its keys
// (larger key first, equal keys: smaller expert id) and weights them by
// score / sum of the selected scores, summed in rank order.
//  1. tau = the k-th largest key image, found bit by bit from the top: a bit
//     is kept when at least k keys are >= the threshold with it set (ballot
//     counts, uniform scalar work).
//  2. selected = keys above tau, then keys equal to tau in ascending expert id
//     until k are taken.
//  3. each selected expert's rank = number of keys ordered before it; lane
//     `rank` keeps its id and score, lanes 0..k-1 write the result.
//  PER candidate slots per lane (64 * PER >= E); slots past E sort below
//  every key and are never counted or selected.
template <int PER>
__device__ void select_keys_per(const float *__restrict__ krow, const float *__restrict__ srow, int E, int k,
                                int32_t *ids_out, float *w_out, int lane) {
    uint32_t u[PER];
    float s[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = lane + 64 * i;
        const bool ok = e < E;
        u[i] = ok ? key_order(krow[e]) : 0u;  // absent candidates sort below every key
        s[i] = ok ? srow[e] : 0.0f;
    }
    uint32_t tau = 0;
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t c = tau | (1u << bit);
        int n = 0;
#pragma unroll
        for (int i = 0; i < PER; ++i)
            n += __popcll(__ballot(u[i] >= c));
        if (n >= k) tau = c;
    }
    uint64_t selb[PER];
    int need = k;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        selb[i] = __ballot(u[i] > tau);
        need -= __popcll(selb[i]);
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        uint64_t eq = __ballot(u[i] == tau);
        while (eq && need > 0) {  // lowest lane = smallest id within the slot
            const uint64_t low = eq & (~eq + 1ull);
            selb[i] |= low;
            eq ^= low;
            --need;
        }
    }
    int my_id = 0;
    float my_s = 0.0f;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        uint64_t m = selb[i];
        while (m) {
            const int l = __builtin_ctzll(m);
            m &= m - 1;
            const uint32_t ux = __builtin_amdgcn_readlane(u[i], l);
            const float sx = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s[i]), l));
            const int ex = l + 64 * i;
            int rank = 0;
#pragma unroll
            for (int j = 0; j < PER; ++j)
                rank += __popcll(__ballot(u[j] > ux || (u[j] == ux && lane + 64 * j < ex)));
            if (lane == rank) {
                my_id = ex;
                my_s = sx;
            }
        }
    }
    float S = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
        if (j < k) S += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_s), j));
    if (lane < k) {
        ids_out[lane] = my_id;
        w_out[lane] = my_s / S;
    }
}

__device__ __forceinline__ void select_keys_wave(const float *__restrict__ krow, const float *__restrict__ srow, int E,
                                                 int k, int32_t *ids_out, float *w_out, int lane) {
    if (E <= 64) select_keys_per<1>(krow, srow, E, k, ids_out, w_out, lane);
    else if (E <= 128) select_keys_per<2>(krow, srow, E, k, ids_out, w_out, lane);
    else if (E <= 256) select_keys_per<4>(krow, srow, E, k, ids_out, w_out, lane);
    else if (E <= 512) select_keys_per<8>(krow, srow, E, k, ids_out, w_out, lane);
    else select_keys_per<16>(krow, srow, E, k, ids_out, w_out, lane);
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

}  // namespace qrmoe
