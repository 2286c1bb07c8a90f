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
    return (float)wave_sum_f64(segment_tree<SEG>(xrow + lane * SEG, wrow + lane * SEG));
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
// score / sum of the selected scores, summed in rank order.  k rounds, each
// on the vector ALUs without branches: the wave maximum m of the remaining
// key images (xor butterfly), the smallest expert id holding m (a per-lane
// minimum over its candidate slots, then a butterfly minimum), whose slot is
// then cleared; its score is read from the owning lane.  Lane `rank` keeps
// the id and score of that rank; lanes 0..k-1 write the result.
//  PER candidate slots per lane (64 * PER >= E), expert id lane + 64*slot;
//  slots past E hold 0, below every key image, and are never taken.
template <int PER>
struct KeyRegs {
    uint32_t u[PER];
    float s[PER];
    __device__ __forceinline__ void load(const float *__restrict__ krow, const float *__restrict__ srow, int E,
                                         int lane) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = lane + 64 * i;
            const bool ok = e < E;
            u[i] = ok ? key_order(krow[e]) : 0u;
            s[i] = ok ? srow[e] : 0.0f;
        }
    }
};

template <int PER>
__device__ void select_keys_from(KeyRegs<PER> r, int k, int &my_id, float &my_w, int lane) {
    auto umax = [](uint32_t a, uint32_t b) { return a > b ? a : b; };
    auto umin = [](uint32_t a, uint32_t b) { return a < b ? a : b; };
    my_id = 0;
    float my_s = 0.0f, S = 0.0f;
    for (int rank = 0; rank < k; ++rank) {
        uint32_t lm = r.u[0];
#pragma unroll
        for (int i = 1; i < PER; ++i) lm = umax(lm, r.u[i]);
        const uint32_t m = group_reduce<64>(lm, umax);
        uint32_t cid = 0xffffffffu;
#pragma unroll
        for (int i = 0; i < PER; ++i) cid = umin(cid, r.u[i] == m ? (uint32_t)(lane + 64 * i) : 0xffffffffu);
        const uint32_t id = group_reduce<64>(cid, umin);  // the same in every lane
        float sl = 0.0f;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const bool hit = (uint32_t)(lane + 64 * i) == id;
            sl = hit ? r.s[i] : sl;
            r.u[i] = hit ? 0u : r.u[i];
        }
        const float sx = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sl), (int)(id & 63u)));
        S += sx;
        if (lane == rank) {
            my_id = (int)id;
            my_s = sx;
        }
    }
    my_w = my_s / S;
}

template <int PER>
__device__ __forceinline__ void select_keys_per(const float *__restrict__ krow, const float *__restrict__ srow, int E,
                                                int k, int &my_id, float &my_w, int lane) {
    KeyRegs<PER> r;
    r.load(krow, srow, E, lane);
    select_keys_from<PER>(r, k, my_id, my_w, lane);
}

// Lane r < k of the calling wave receives the rank-r expert id and weight.
__device__ __forceinline__ void select_keys_regs(const float *__restrict__ krow, const float *__restrict__ srow, int E,
                                                 int k, int &id, float &w, int lane) {
    if (E <= 64) select_keys_per<1>(krow, srow, E, k, id, w, lane);
    else if (E <= 128) select_keys_per<2>(krow, srow, E, k, id, w, lane);
    else if (E <= 256) select_keys_per<4>(krow, srow, E, k, id, w, lane);
    else if (E <= 512) select_keys_per<8>(krow, srow, E, k, id, w, lane);
    else select_keys_per<16>(krow, srow, E, k, id, w, lane);
}

__device__ __forceinline__ void select_keys_wave(const float *__restrict__ krow, const float *__restrict__ srow, int E,
                                                 int k, int32_t *ids_out, float *w_out, int lane) {
    int id;
    float w;
    select_keys_regs(krow, srow, E, k, id, w, lane);
    if (lane < k) {
        ids_out[lane] = id;
        w_out[lane] = w;
    }
}

// Lane j < k receives the j-th entry of the token's table row (rows of
// row_k >= k entries; clamped and flagged when out of range) and its weight:
// 1/k, or with srow (the token's sigmoid scores) the score renormalised over
// the k kept experts, S summed in table order (lane order).
__device__ __forceinline__ void select_hash_regs(const int32_t *__restrict__ token_ids, const int32_t *__restrict__ table,
                                                 int t, int vocab, int row_k, int E, int k, int &id_out, float &w_out,
                                                 int32_t *flags, const float *__restrict__ srow, int lane) {
    int id = token_ids[t];
    if (id < 0 || id >= vocab) {
        if (lane == 0) atomicOr(flags, 1);
        id = 0;
    }
    id_out = 0;
    w_out = 0.0f;
    if (lane < k) {
        int e = table[(int64_t)id * row_k + lane];
        if (e < 0 || e >= E) {
            atomicOr(flags, 2);
            e = 0;
        }
        id_out = e;
        w_out = 1.0f / (float)k;
    }
    // A kept row that names one expert twice (after clamping) is flagged: the
    // layer then weights that expert once, where the row asks for it twice.
    bool dup = false;
#pragma unroll
    for (int j = 0; j < 8; ++j)
        if (j < k) dup |= lane < k && j < lane && __builtin_amdgcn_readlane(id_out, j) == id_out;
    if (__ballot(dup) != 0 && lane == 0) atomicOr(flags, 4);
    if (srow) {
        const float sc = lane < k ? srow[id_out] : 0.0f;
        float S = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (j < k) S += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sc), j));
        if (lane < k) w_out = sc / S;
    }
}

// Hash routing of several tokens per wave, eight lanes per token: lane j < k
// of token t's group takes entry j of the token's table row and its weight,
// with the same clamping, flags and arithmetic as select_hash_regs (S summed
// in table order, the group's lane order).  scores, when given, is [T][E].
__device__ __forceinline__ void select_hash_group8(const int32_t *__restrict__ token_ids,
                                                   const int32_t *__restrict__ table, int t, bool valid, int vocab,
                                                   int row_k, int E, int k, int &id_out, float &w_out,
                                                   int32_t *flags, const float *__restrict__ scores, int lane) {
    const int j = lane & 7;
    int id = valid ? token_ids[t] : 0;
    if (id < 0 || id >= vocab) {
        if (j == 0) atomicOr(flags, 1);
        id = 0;
    }
    const bool mine = valid && j < k;
    int e = 0;
    if (mine) {
        e = table[(int64_t)id * row_k + j];
        if (e < 0 || e >= E) {
            atomicOr(flags, 2);
            e = 0;
        }
    }
    id_out = e;
    w_out = mine ? 1.0f / (float)k : 0.0f;
    const int base = lane & ~7;
    bool dup = false;  // an expert repeated within the kept row, flagged as in select_hash_regs
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int ei = __shfl(e, base + i);
        dup |= mine && i < j && ei == e;
    }
    if (dup) atomicOr(flags, 4);
    if (scores) {
        const float sc = mine ? scores[(int64_t)t * E + e] : 0.0f;
        float S = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (i < k) S += __shfl(sc, base + i);
        if (mine) w_out = sc / S;
    }
}

__device__ void select_hash_wave(const int32_t *__restrict__ token_ids, const int32_t *__restrict__ table, int t,
                                 int vocab, int row_k, int E, int k, int32_t *ids_out, float *w_out, int32_t *flags,
                                 const float *__restrict__ srow, int lane) {
    int id;
    float w;
    select_hash_regs(token_ids, table, t, vocab, row_k, E, k, id, w, flags, srow, lane);
    if (lane < k) {
        ids_out[lane] = id;
        w_out[lane] = w;
    }
}

}  // namespace qrmoe
