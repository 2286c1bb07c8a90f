// Decode-sized batches (T <= 32 tokens).
//
//  front   quantize x and compute the router logits, scores and selection
//          keys (learned layers: one workgroup per logit, the four waves each
//          sum a quarter of the adjacent-pair tree).
//  select  one workgroup: top-k or hash selection, sort, work list.
//  gateup  T == 1: below.  T > 1: gate/up + SwiGLU + h quantization of the
//          routed and shared groups of the work list (expert_vec.hip).
//  down    T == 1: one kernel computes every output row from all selected
//          experts at once (each wave holds the row of every expert in
//          registers, requested before anything else) and sums w * y in
//          ascending expert id, shared last, with the same rounding steps as
//          the batched down + combine.  T > 1: per-group down rows into y,
//          then the combine kernel (expert_vec.hip).
//
// Stage boundaries are kernel boundaries: no device-scope fences, which on
// this multi-XCD part write back and invalidate L2.
#include "dev_route.hpp"
#include "dev_vec.hpp"

namespace qrmoe {

// ------------------------------------------------------------------ front
template <int H>
__global__ __launch_bounds__(256) void decode_front_kernel(LayerArgs a, int n_lead) {
    __shared__ double part[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const Dims &d = a.d;
    const int nblk = d.T * (H / 32);
    for (int b = blockIdx.x * 256 + tid; b < nblk; b += n_lead * 256)
        quant_one_block(a.x, a.ws.xq, a.ws.xd, d.fmt == kFmtQ2 ? a.ws.xs16 : nullptr, b);
    if (d.route == kRouteHash) return;  // no router
    // every (token, expert) logit, or with table_logits the (token, entry j)
    // ones of the table's first k entries (clamped as the selection clamps
    // them; an expert named twice is computed twice, with the same bits)
    const int nlog = d.table_logits ? d.T * d.k : d.T * d.E;
    auto pair_of = [&](int le, int &t, int &e) {
        if (d.table_logits) {
            t = le / d.k;
            int id = a.token_ids[t];
            if (id < 0 || id >= d.vocab) id = 0;
            e = a.wt.table[(int64_t)id * d.table_k + le % d.k];
            if (e < 0 || e >= d.E) e = 0;
        } else {
            t = le / d.E;
            e = le % d.E;
        }
    };
    if constexpr (H >= 256) {
        // one logit per workgroup; wave w sums elements [w*H/4, (w+1)*H/4)
        constexpr int SEG = H / 256;
        for (int le = blockIdx.x; le < nlog; le += n_lead) {
            int t, e;
            pair_of(le, t, e);
            const int off = wave * (H / 4) + lane * SEG;
            const double v =
                wave_sum_f64(segment_tree<SEG>(a.x + (int64_t)t * H + off, a.wt.router_w + (int64_t)e * H + off));
            if (lane == 0) part[wave] = v;
            __syncthreads();
            if (tid == 0) {
                const float l = (float)((part[0] + part[1]) + (part[2] + part[3]));
                const int64_t i = (int64_t)t * d.E + e;
                a.ws.logits[i] = l;
                score_key(l, a.wt.router_b, e, a.ws.scores + i, a.ws.keys + i);
            }
            __syncthreads();
        }
    } else {
        for (int le = blockIdx.x * 4 + wave; le < nlog; le += n_lead * 4) {
            int t, e;
            pair_of(le, t, e);
            const float l = wave_logit<H>(a.x + (int64_t)t * H, a.wt.router_w + (int64_t)e * H, lane);
            if (lane == 0) {
                const int64_t i = (int64_t)t * d.E + e;
                a.ws.logits[i] = l;
                score_key(l, a.wt.router_b, e, a.ws.scores + i, a.ws.keys + i);
            }
        }
    }
}

// ----------------------------------------------------------------- select
// One workgroup: top-k (or hash lookup) of every token, stable sort of the
// P = T*k <= 256 pairs by expert (rank = number of pairs with a smaller
// expert, or the same expert and a smaller pair index), and the work list
// (the shared expert's token runs, then each expert's pairs cut into runs
// of at most kVecTok, experts ascending).
struct SelectSmem {
    alignas(16) int32_t ids[kDecodeMaxT * 8];  // padded to a multiple of 4 with INT_MAX (counted nowhere)
    float w[kDecodeMaxT * 8];
    int32_t perm[kDecodeMaxT * 8];
    int32_t gpos[kDecodeMaxT * 8 + 1];
    int32_t tmp[4];
    int32_t ngroups;
};

// Learned routing, one token per wave at a time: the wave's next token's keys
// and scores are requested before the current token is selected.
template <int PER>
__device__ void select_learned_tokens(const LayerArgs &a, SelectSmem &rs, int wave, int lane) {
    const Dims &d = a.d;
    KeyRegs<PER> cur;
    if (wave < d.T) cur.load(a.ws.keys + (int64_t)wave * d.E, a.ws.scores + (int64_t)wave * d.E, d.E, lane);
    for (int t = wave; t < d.T; t += 4) {
        KeyRegs<PER> nxt;
        if (t + 4 < d.T) nxt.load(a.ws.keys + (int64_t)(t + 4) * d.E, a.ws.scores + (int64_t)(t + 4) * d.E, d.E, lane);
        int id;
        float w;
        select_keys_from<PER>(cur, d.k, id, w, lane);
        if (lane < d.k) {
            rs.ids[t * d.k + lane] = id;
            rs.w[t * d.k + lane] = w;
        }
        cur = nxt;
    }
}

__global__ __launch_bounds__(256) void decode_select_kernel(LayerArgs a) {
    __shared__ SelectSmem rs;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const Dims &d = a.d;
    const int P = d.T * d.k;
    if (d.route == kRouteLearned) {
        if (d.E <= 64) select_learned_tokens<1>(a, rs, wave, lane);
        else if (d.E <= 128) select_learned_tokens<2>(a, rs, wave, lane);
        else if (d.E <= 256) select_learned_tokens<4>(a, rs, wave, lane);
        else if (d.E <= 512) select_learned_tokens<8>(a, rs, wave, lane);
        else select_learned_tokens<16>(a, rs, wave, lane);
    } else {
        // eight lanes per token: the workgroup routes 32 tokens per pass
        for (int t0 = 0; t0 < d.T; t0 += 32) {
            const int t = t0 + wave * 8 + lane / 8, j = lane & 7;
            const bool valid = t < d.T;
            int id;
            float w;
            select_hash_group8(a.token_ids, a.wt.table, valid ? t : 0, valid, d.vocab, d.table_k, d.E, d.k, id, w,
                               a.ws.ctl + kCtlFlags, d.route == kRouteHashScored ? a.ws.scores : nullptr, lane);
            if (valid && j < d.k) {
                rs.ids[t * d.k + j] = id;
                rs.w[t * d.k + j] = w;
            }
        }
    }
    const int P4 = (P + 3) & ~3;
    if (tid >= P && tid < P4) rs.ids[tid] = 0x7fffffff;
    __syncthreads();
    const int4 *__restrict__ ids4 = reinterpret_cast<const int4 *>(rs.ids);
    if (tid < P) {
        const int e = rs.ids[tid];
        int rank = 0;
#pragma unroll 4
        for (int q4 = 0; q4 < P4 / 4; ++q4) {
            const int4 f = ids4[q4];
            const int q = 4 * q4;
            rank += (f.x < e) || (f.x == e && q < tid);
            rank += (f.y < e) || (f.y == e && q + 1 < tid);
            rank += (f.z < e) || (f.z == e && q + 2 < tid);
            rank += (f.w < e) || (f.w == e && q + 3 < tid);
        }
        rs.perm[rank] = tid;
        a.ws.ids[tid] = e;
        a.ws.w[tid] = rs.w[tid];
    }
    __syncthreads();
    int flag = 0;
    if (tid < P) {
        const int e = rs.ids[rs.perm[tid]];
        int start = tid;
        while (start > 0 && rs.ids[rs.perm[start - 1]] == e) --start;
        flag = ((tid - start) % kVecTok) == 0;
        a.ws.perm[tid] = rs.perm[tid];
    }
    int inc = flag;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(inc, o);
        if (lane >= o) inc += v;
    }
    if (lane == 63) rs.tmp[wave] = inc;
    __syncthreads();
    for (int w = 0; w < wave; ++w) inc += rs.tmp[w];
    if (flag) rs.gpos[inc - 1] = tid;
    if (tid == 255) rs.ngroups = inc;
    __syncthreads();
    // the shared expert's token runs first: their workgroups carry the most
    // tokens, so they start with the kernel instead of forming its tail
    const int G = rs.ngroups;
    const int ns = d.has_shared ? (d.T + kVecTok - 1) / kVecTok : 0;
    for (int j = tid; j < ns; j += 256)
        a.ws.groups[j] = make_int4(d.E, j * kVecTok, min(kVecTok, d.T - j * kVecTok), P + j * kVecTok);
    for (int g = tid; g < G; g += 256) {
        const int gs = rs.gpos[g], ge = g + 1 < G ? rs.gpos[g + 1] : P;
        a.ws.groups[ns + g] = make_int4(rs.ids[rs.perm[gs]], gs, ge - gs, rs.perm[gs]);
    }
    if (tid == 0) {
        a.ws.ctl[kCtlGroups] = G + ns;
        a.ws.offsets[d.E] = P;
    }
    for (int e = tid; e < d.E; e += 256) {
        int c = 0, below = 0;
#pragma unroll 4
        for (int q4 = 0; q4 < P4 / 4; ++q4) {
            const int4 f = ids4[q4];
            c += (f.x == e) + (f.y == e) + (f.z == e) + (f.w == e);
            below += (f.x < e) + (f.y < e) + (f.z < e) + (f.w < e);
        }
        a.ws.counts[e] = c;
        a.ws.offsets[e] = below;
    }
}

// ---------------------------------------------------- gate/up, one token
// T == 1: the selection is repeated in every workgroup instead of running in
// a kernel of its own (it costs each workgroup about as much as its first
// weight request, and saves a dependent launch).  blockIdx.y is the slot: the
// position of the workgroup's expert among the distinct selected experts in
// ascending id; the slots after the last routed one are the shared expert's,
// whose gate/up rows stream from the start.  Workgroup (0, 0) publishes the routing for the down
// kernel and the debug copies: ids and w in rank order, perm (pairs by
// expert, then slot), counts, offsets and the work list.
struct Sel1Smem {
    int32_t ids[8];
    float w[8];
    int32_t pairs[8];  // rank slots ordered by (expert, slot)
    int32_t uniq[8];   // distinct selected experts, ascending
    int32_t first[8];  // position in `pairs` of each distinct expert's first pair
    int32_t nuniq;
    int32_t flags;     // hash-path flags of workgroups other than (0, 0)
};

// Two workgroup shapes: 64 rows (two h blocks) x 8 waves while the grid
// holds at most one workgroup per CU, else 32 rows (one h block) x 4 waves,
// whose smaller workgroups share CUs (at top-8 of 384 experts the wide grid
// needs a second round).
constexpr int kG1Rows = 64, kG1Waves = 8;
constexpr int kG1RowsNarrow = 32, kG1WavesNarrow = 4;
constexpr int kG1OneRound = 256;  // workgroups of one round of the wide shape (one per CU)
// Rows of a shared-expert workgroup: one h block where a wave pass allows it,
// so the shared expert's rows spread over more workgroups (one slot per 32
// rows of each column); the shared expert is Q8 even when the routed experts
// are 2-bit, and with one slot its workgroups would stream three times the
// bytes of a 2-bit routed one.
constexpr int kMaxSelList = 9;  // work-list entries the one-token down kernel reads (top_k <= 8, shared)
template <int K, int NW>
constexpr int g1_shared_rows() {
    return NW * Geo<K, kFmtQ8>::RPW > 32 ? NW * Geo<K, kFmtQ8>::RPW : 32;
}

template <int K, int FMT, bool DUMP, int ROWS, int NW>
__global__ __launch_bounds__(512) void decode_gateup1_kernel(LayerArgs a) {
    __shared__ VecSmem<K, kVecTok> sm;
    __shared__ Sel1Smem ss;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const Dims &d = a.d;
    const int slot = blockIdx.y;
    if (slot >= d.k) {  // shared expert (pair k): needs no routing, streams while the others select
        constexpr int SR = g1_shared_rows<K, NW>();
        if (tid == 0) {
            sm.pair[0] = d.k;
            sm.row[0] = 0;
        }
        gateup_rows<K, kFmtQ8, kVecTok, SR, DUMP, NW>(
            a, sm, a.wt.sh_gate, a.wt.sh_up, 1, ((slot - d.k) * gridDim.x + blockIdx.x) * SR, [&] {
                for (int i = tid; i < K / 16; i += 64 * NW) {
                    reinterpret_cast<int4 *>(sm.aq[0])[i] = reinterpret_cast<const int4 *>(a.ws.xq)[i];
                    if (i < K / 32) sm.ad[0][i] = a.ws.xd[i];
                }
                __syncthreads();
            });
        return;
    }
    const bool publish = blockIdx.x == 0 && slot == 0;
    if (wave == 0) {
        int id;
        float w;
        if (d.route == kRouteLearned)
            select_keys_regs(a.ws.keys, a.ws.scores, d.E, d.k, id, w, lane);
        else
            select_hash_regs(a.token_ids, a.wt.table, 0, d.vocab, d.table_k, d.E, d.k, id, w,
                             publish ? a.ws.ctl + kCtlFlags : &ss.flags,
                             d.route == kRouteHashScored ? a.ws.scores : nullptr, lane);
        // lane j < k holds rank slot j: order the slots by (expert, slot) in
        // registers, then the distinct experts in ascending id
        const int k = d.k;
        const int e = lane < k ? id : 0x7fffffff;
        int rank = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (i < k) {
                const int f = __builtin_amdgcn_readlane(e, i);
                rank += (f < e) || (f == e && i < lane);
            }
        int src = 0;  // slot at sorted position `lane`
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (j < k && __builtin_amdgcn_readlane(rank, j) == lane) src = j;
        const int ej = __shfl(e, src);
        const int eprev = __shfl_up(ej, 1);
        const bool is_first = lane < k && (lane == 0 || eprev != ej);
        const uint64_t firsts = __ballot(is_first);
        if (lane < k) {
            ss.ids[lane] = id;
            ss.w[lane] = w;
            ss.pairs[lane] = src;
        }
        if (is_first) {
            const int u = __popcll(firsts & ((1ull << lane) - 1ull));
            ss.uniq[u] = ej;
            ss.first[u] = lane;
        }
        if (lane == 0) ss.nuniq = __popcll(firsts);
    } else {
        // meanwhile the token's quantized x goes to LDS slot 0
        for (int i = tid - 64; i < K / 16; i += 64 * (NW - 1)) {
            reinterpret_cast<int4 *>(sm.aq[0])[i] = reinterpret_cast<const int4 *>(a.ws.xq)[i];
            if (i < K / 32) sm.ad[0][i] = a.ws.xd[i];
            if (FMT == kFmtQ2) sm.as16[0][i] = a.ws.xs16[i];
        }
    }
    __syncthreads();
    const int nuniq = ss.nuniq;
    if (publish) {
        const int k = d.k;
        if (tid < k) {
            a.ws.ids[tid] = ss.ids[tid];
            a.ws.w[tid] = ss.w[tid];
            a.ws.perm[tid] = ss.pairs[tid];
        }
        for (int e = tid; e < d.E; e += 64 * NW) {
            int c = 0, below = 0;
            for (int i = 0; i < k; ++i) {
                c += ss.ids[i] == e;
                below += ss.ids[i] < e;
            }
            a.ws.counts[e] = c;
            a.ws.offsets[e] = below;
        }
        if (tid < nuniq) {
            const int f = ss.first[tid], n = (tid + 1 < nuniq ? ss.first[tid + 1] : k) - f;
            a.ws.groups[tid] = make_int4(ss.uniq[tid], f, n, ss.pairs[f]);
        } else if (tid >= nuniq + d.has_shared && tid < kMaxSelList) {
            a.ws.groups[tid] = make_int4(0, 0, 0, 0);  // entries past the list name group 0's pair
        }
        if (tid == 0) {
            a.ws.offsets[d.E] = k;
            if (d.has_shared) a.ws.groups[nuniq] = make_int4(d.E, 0, 1, k);
            a.ws.ctl[kCtlGroups] = nuniq + d.has_shared;
        }
    }
    if (slot >= nuniq) return;  // fewer distinct experts than k (a repeated hash-table id)
    const int e = ss.uniq[slot], f = ss.first[slot];
    const int cnt = (slot + 1 < nuniq ? ss.first[slot + 1] : d.k) - f;
    if (tid < cnt) {
        sm.pair[tid] = ss.pairs[f + tid];
        sm.row[tid] = 0;
    }
    // a repeated expert (cnt > 1) applies to the same x: copy slot 0
    for (int i = tid; i < (cnt - 1) * (K / 16); i += 64 * NW) {
        const int tok = 1 + i / (K / 16), c = i % (K / 16);
        reinterpret_cast<int4 *>(sm.aq[tok])[c] = reinterpret_cast<const int4 *>(sm.aq[0])[c];
        if (c < K / 32) sm.ad[tok][c] = sm.ad[0][c];
        if (FMT == kFmtQ2) sm.as16[tok][c] = sm.as16[0][c];
    }
    const int64_t mb = mat_bytes(FMT, d.F, K);
    gateup_rows<K, FMT, kVecTok, ROWS, DUMP, NW>(a, sm, a.wt.gate + e * mb, a.wt.up + e * mb, cnt,
                                                               blockIdx.x * ROWS, [&] { __syncthreads(); });
}

// -------------------------------------------------------- down, one token
// Rows of the output: each wave pass covers RPW rows (LPR lanes per row, the
// routed format's geometry; the shared Q8 expert reuses it with more chunks
// per lane).  Every selected expert's row is requested before h is staged.
constexpr int kMaxSel = kMaxSelList;  // top_k <= 8 plus the shared expert
constexpr int kD1Waves = 8;           // waves of a one-token down workgroup (they share the staged h)

// NR routed row slots per lane (top_k <= NR); every slot is loaded and
// reduced, the ones past the routed groups are dropped at the combine.
template <int F, int FMT, bool DUMP, int NR>
// (4096-wide Q8 rows hold 4 chunks a lane per expert: those run at 2 waves per SIMD)
__global__ __launch_bounds__(64 * kD1Waves, (F == 4096 && FMT == kFmtQ8) ? 2 : 4) void decode_down1_kernel(LayerArgs a) {
    constexpr int L = DefLpr<F, FMT>::v;
    constexpr int RPW = 64 / L;
    constexpr int NT = 64 * kD1Waves;
    constexpr int NS = ((NR + 1) * (F / 32) + NT - 1) / NT;  // h block scales per thread (G <= NR + 1)
    constexpr int NH = ((NR + 1) * (F / 16) + NT - 1) / NT;  // 16-byte h code chunks per thread
    __shared__ VecSmem<F, kMaxSel> sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const Dims &d = a.d;
    const int seg = lane % L, r = (blockIdx.x * kD1Waves + wave) * RPW + lane / L;
    // Loads are issued in the order their results are needed, because a wave
    // waits for loads in issue order: the shared expert's row (needs no
    // routing), the work list, the h rows and combine weights of the groups,
    // then the routed rows; h is written to LDS while the rows still stream.
    RowRegs<F, kFmtQ8, L> rsh;
    if (d.has_shared) rsh.load(a.wt.sh_down, d.H, r, seg);
    // k routed groups in ascending id, then the shared expert (the list holds at least kMaxSel entries)
    const int4 *__restrict__ glist = a.ws.groups;
    int gx[kMaxSel], gp[kMaxSel];
#pragma unroll
    for (int i = 0; i < kMaxSel; ++i) {
        const int4 g = glist[i];
        gx[i] = g.x;
        gp[i] = g.w;  // first (only) pair of the group
    }
    const int G = a.ws.ctl[kCtlGroups];
    const int nr = d.has_shared ? G - 1 : G;
    // pair of group `i` by a chain of selects (constant register indices)
#define QRMOE_PAIR_OF(out, i)                                      \
    int out = gp[0];                                               \
    _Pragma("unroll") for (int j_ = 1; j_ < kMaxSel; ++j_) out = (i) == j_ ? gp[j_] : out
    QRMOE_PAIR_OF(pown, tid);
    // work-list entries past the G groups were never written: their pairs
    // index nothing, so threads past the routed groups read group 0's weight
    const float wraw = a.ws.w[tid < nr ? pown : gp[0]];
    // h block scales: loads now, LDS after the rows are requested
    float hdv[NS];
#pragma unroll
    for (int u = 0; u < NS; ++u) {
        const int idx = tid + NT * u;
        const bool ok = idx < G * (F / 32);
        QRMOE_PAIR_OF(p, ok ? idx / (F / 32) : 0);
        hdv[u] = a.ws.hd[(int64_t)p * (F / 32) + (ok ? idx % (F / 32) : 0)];
    }
    // h codes of the G pairs: loads now (in registers), LDS after the rows
    // are requested, so the wave waits for h and then for each row in turn
    // instead of for all of them at once.  Chunks past the G pairs re-read
    // pair 0's row and are not stored.
    typedef int v4i __attribute__((ext_vector_type(4)));
    v4i hv[NH];
#pragma unroll
    for (int u = 0; u < NH; ++u) {
        const int idx = tid + NT * u;
        const bool ok = idx < G * (F / 16);
        QRMOE_PAIR_OF(p, ok ? idx / (F / 16) : 0);
        hv[u] = reinterpret_cast<const v4i *>(a.ws.hq + (int64_t)p * F)[ok ? idx % (F / 16) : 0];
    }
#undef QRMOE_PAIR_OF
    // The compiler may not move the loads above below the rows (a wave's loads
    // return in issue order, so each would then wait for every row).
    __builtin_amdgcn_sched_barrier(0);
    // Every slot loads without a branch (a slot past the routed groups re-reads
    // group 0's row, served by the cache), so nothing is sunk below the rows.
    const int64_t mb = mat_bytes(FMT, d.H, F);
    RowRegs<F, FMT, L> rr[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) rr[i].load(a.wt.down + (int64_t)(i < nr ? gx[i] : gx[0]) * mb, d.H, r, seg);
    if (tid < G) {
        sm.pair[tid] = pown;
        sm.w[tid] = tid < nr ? wraw : 1.0f;
    }
#pragma unroll
    for (int u = 0; u < NS; ++u) {
        const int idx = tid + NT * u;
        if (idx < G * (F / 32)) sm.ad[idx / (F / 32)][idx % (F / 32)] = hdv[u];
    }
    // Every thread stores each chunk it loaded (chunks past the G pairs go to
    // a junk slot in the h area, which this kernel does not use otherwise):
    // a store under a branch would let the compiler sink its load below the
    // rows.  2-bit weights also need h's 16-code subblock sums: a chunk is
    // one subblock.
    v4i *junk = reinterpret_cast<v4i *>(&sm.h[0][0]) + (tid & 127);
    static_assert(sizeof(sm.h) >= 128 * sizeof(v4i), "junk slots");
#pragma unroll
    for (int u = 0; u < NH; ++u) {
        const int idx = tid + NT * u;
        const bool ok = idx < G * (F / 16);
        v4i *dst = ok ? reinterpret_cast<v4i *>(sm.aq[idx / (F / 16)]) + idx % (F / 16) : junk;
        *dst = hv[u];
        if constexpr (FMT == kFmtQ2) {
            int sub = sdot4(hv[u][0], 0x01010101, 0);
            sub = sdot4(hv[u][1], 0x01010101, sub);
            sub = sdot4(hv[u][2], 0x01010101, sub);
            sub = sdot4(hv[u][3], 0x01010101, sub);
            if (ok) sm.as16[idx / (F / 16)][idx % (F / 16)] = sub;
        }
    }
    __syncthreads();
    // Same arithmetic per expert as the batched down + combine: y = w * (sum
    // over lanes), summed in ascending expert id, the shared expert last.
    // The shared expert's row was requested first, so it is reduced first.
    const bool dump_row = DUMP && (r % a.dump.stride == 0);
    float ysh = 0.0f;
    if (d.has_shared) {
        int32_t *dd = dump_row ? a.dump.down_sums +
                                     ((int64_t)sm.pair[nr] * (d.H / a.dump.stride) + r / a.dump.stride) *
                                         a.dump.pitch_dn
                               : nullptr;
        ysh = group_sum<L>(lane_dot<F, L>(rsh, sm.aq[nr], sm.ad[nr], sm.as16[nr], seg, dd));
    }
    // The routed slots are reduced without branches; slots past the routed
    // groups read LDS rows nobody wrote and are dropped here.
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        int32_t *dd = dump_row && i < nr ? a.dump.down_sums +
                                               ((int64_t)sm.pair[i] * (d.H / a.dump.stride) + r / a.dump.stride) *
                                                   a.dump.pitch_dn
                                         : nullptr;
        const float y = group_sum<L>(lane_dot<F, L>(rr[i], sm.aq[i], sm.ad[i], sm.as16[i], seg, dd));
        const float t = __fadd_rn(acc, __fmul_rn(sm.w[i], y));
        acc = i < nr ? t : acc;
    }
    if (d.has_shared) acc = __fadd_rn(acc, __fmul_rn(1.0f, ysh));
    if (seg == 0) a.out[r] = acc;
}

// ------------------------------------------------------------- launchers
template <int H>
static hipError_t front_h(const LayerArgs &a, hipStream_t s) {
    const Dims &d = a.d;
    const int nq = (d.T * (H / 32) + 255) / 256;
    int n_lead = nq;
    if (d.route != kRouteHash) {
        const int n = d.table_logits ? d.T * d.k : d.T * d.E;
        const int nl = H >= 256 ? n : (n + 3) / 4;
        n_lead = nl > nq ? nl : nq;
    }
    if (n_lead > 4096) n_lead = 4096;
    klaunch(decode_front_kernel<H>, dim3(n_lead), dim3(256), s, a, n_lead);
    return hipGetLastError();
}

hipError_t launch_decode_front(const LayerArgs &a, hipStream_t s) {
    switch (a.d.H) {
        case 128: return front_h<128>(a, s);
        case 256: return front_h<256>(a, s);
        case 512: return front_h<512>(a, s);
        case 1024: return front_h<1024>(a, s);
        case 2048: return front_h<2048>(a, s);
        case 4096: return front_h<4096>(a, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode_select(const LayerArgs &a, hipStream_t s) {
    klaunch(decode_select_kernel, dim3(1), dim3(256), s, a);
    return hipGetLastError();
}

// grid: (F / ROWS columns) x (k routed slots + the shared expert's slots)
template <int K, int FMT, bool DUMP, int ROWS, int NW>
static void gateup1_grid(const LayerArgs &a, hipStream_t s) {
    const int nsh = a.d.has_shared ? ROWS / g1_shared_rows<K, NW>() : 0;
    klaunch(decode_gateup1_kernel<K, FMT, DUMP, ROWS, NW>, dim3(a.d.F / ROWS, a.d.k + nsh), dim3(64 * NW), s, a);
}

template <int K, int FMT, bool DUMP>
static void gateup1_launch(const LayerArgs &a, hipStream_t s) {
    const int nsh = a.d.has_shared ? kG1Rows / g1_shared_rows<K, kG1Waves>() : 0;
    if ((a.d.F / kG1Rows) * (a.d.k + nsh) <= kG1OneRound)
        gateup1_grid<K, FMT, DUMP, kG1Rows, kG1Waves>(a, s);
    else
        gateup1_grid<K, FMT, DUMP, kG1RowsNarrow, kG1WavesNarrow>(a, s);
}

template <int FMT, bool DUMP>
static hipError_t gateup1_f(const LayerArgs &a, hipStream_t s) {
    switch (a.d.H) {
        case 128: if constexpr (FMT == kFmtQ8) { gateup1_launch<128, FMT, DUMP>(a, s); break; } return hipErrorInvalidValue;
        case 256: if constexpr (FMT == kFmtQ8) { gateup1_launch<256, FMT, DUMP>(a, s); break; } return hipErrorInvalidValue;
        case 512: gateup1_launch<512, FMT, DUMP>(a, s); break;
        case 1024: gateup1_launch<1024, FMT, DUMP>(a, s); break;
        case 2048: gateup1_launch<2048, FMT, DUMP>(a, s); break;
        case 4096: gateup1_launch<4096, FMT, DUMP>(a, s); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_decode_gateup1(const LayerArgs &a, bool dump, hipStream_t s) {
    if (a.d.T != 1) return hipErrorInvalidValue;
    if (a.d.fmt == kFmtQ8) return dump ? gateup1_f<kFmtQ8, true>(a, s) : gateup1_f<kFmtQ8, false>(a, s);
    return dump ? gateup1_f<kFmtQ2, true>(a, s) : gateup1_f<kFmtQ2, false>(a, s);
}

template <int F, int FMT, bool DUMP>
static hipError_t down1_h(const LayerArgs &a, hipStream_t s) {
    constexpr int RPW = 64 / DefLpr<F, FMT>::v;
    const dim3 grid(a.d.H / (kD1Waves * RPW)), block(64 * kD1Waves);
    if (a.d.k <= 2) klaunch(decode_down1_kernel<F, FMT, DUMP, 2>, grid, block, s, a);
    else if (a.d.k <= 6) klaunch(decode_down1_kernel<F, FMT, DUMP, 6>, grid, block, s, a);
    else klaunch(decode_down1_kernel<F, FMT, DUMP, kMaxSel - 1>, grid, block, s, a);
    return hipGetLastError();
}

template <int FMT, bool DUMP>
static hipError_t down1_f(const LayerArgs &a, hipStream_t s) {
    switch (a.d.F) {
        case 128: if constexpr (FMT == kFmtQ8) return down1_h<128, FMT, DUMP>(a, s); return hipErrorInvalidValue;
        case 256: if constexpr (FMT == kFmtQ8) return down1_h<256, FMT, DUMP>(a, s); return hipErrorInvalidValue;
        case 512: return down1_h<512, FMT, DUMP>(a, s);
        case 1024: return down1_h<1024, FMT, DUMP>(a, s);
        case 2048: return down1_h<2048, FMT, DUMP>(a, s);
        case 4096: return down1_h<4096, FMT, DUMP>(a, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode_down1(const LayerArgs &a, bool dump, hipStream_t s) {
    if (a.d.fmt == kFmtQ8) return dump ? down1_f<kFmtQ8, true>(a, s) : down1_f<kFmtQ8, false>(a, s);
    return dump ? down1_f<kFmtQ2, true>(a, s) : down1_f<kFmtQ2, false>(a, s);
}

}  // namespace qrmoe
