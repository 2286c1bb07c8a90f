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

// Selection order as one integer: larger key first, equal keys smaller
// expert id first.  The fp32 key's bits are mapped to an order-preserving
// unsigned integer (IEEE total order on finite values), the id is stored
// complemented in the low word.
__device__ __forceinline__ uint64_t sel_code(float key, int e) {
    uint32_t u = __float_as_uint(key == 0.0f ? 0.0f : key);  // -0 ties with +0
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)u << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e);
}

__device__ __forceinline__ void cas_desc(uint64_t &a, uint64_t &b) {
    const uint64_t hi = a > b ? a : b, lo = a > b ? b : a;
    a = hi;
    b = lo;
}

// Sort 8 codes descending (bitonic network).
__device__ __forceinline__ void sort8_desc(uint64_t v[8]) {
#pragma unroll
    for (int k = 2; k <= 8; k <<= 1)
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int l = i ^ j;
                if (l > i) {
                    if ((i & k) == 0) cas_desc(v[i], v[l]);
                    else cas_desc(v[l], v[i]);
                }
            }
}

// One wave selects the top-k (k <= 8) experts of one token from its keys
// (larger key first, equal keys: smaller expert id) and weights them by
// score / sum of the selected scores (summed in rank order).  Each lane sorts
// its own candidates, then an xor butterfly merges the lanes' top-8 lists:
// at each level a lane keeps the top 8 of its list and its partner's.
__device__ void select_keys_wave(const float *__restrict__ krow, const float *__restrict__ srow, int E, int k,
                                 int32_t *ids_out, float *w_out, int lane) {
    constexpr int MAXPER = 16;  // E <= 1024
    const int per = (E + 63) / 64;
    uint64_t top[8];
    float my_s[MAXPER];
#pragma unroll
    for (int i = 0; i < MAXPER; ++i) {
        const int e = lane + 64 * i;
        my_s[i] = (i < per && e < E) ? srow[e] : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) top[i] = 0;  // below every real code
    // fold this lane's candidates into a sorted top-8 list, 8 at a time
#pragma unroll
    for (int base = 0; base < MAXPER; base += 8) {
        if (base >= per) break;
        uint64_t c[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int e = lane + 64 * (base + i);
            c[i] = (base + i < per && e < E) ? sel_code(krow[e], e) : 0;
        }
        sort8_desc(c);
#pragma unroll
        for (int i = 0; i < 8; ++i) {  // top 8 of two sorted lists form a bitonic sequence
            const uint64_t m = c[7 - i] > top[i] ? c[7 - i] : top[i];
            top[i] = m;
        }
        sort8_desc(top);
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        uint64_t other[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t lo = __shfl_xor((uint32_t)top[i], o), hi = __shfl_xor((uint32_t)(top[i] >> 32), o);
            other[i] = ((uint64_t)hi << 32) | lo;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) top[i] = other[7 - i] > top[i] ? other[7 - i] : top[i];
        sort8_desc(top);
    }
    // every lane holds the same list; fetch each selected score from its owner lane
    int sel[8];
    float sc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        sel[j] = (int)(0xFFFFFFFFu - (uint32_t)top[j]);
        float mine = 0.0f;
        const int slot = (sel[j] >> 6) & (MAXPER - 1);
#pragma unroll
        for (int i = 0; i < MAXPER; ++i)
            if (i == slot) mine = my_s[i];
        sc[j] = __shfl(mine, sel[j] & 63);
    }
    if (lane == 0) {
        float S = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (j < k) S += sc[j];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (j < k) {
                ids_out[j] = sel[j];
                w_out[j] = sc[j] / S;
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

}  // namespace qrmoe
