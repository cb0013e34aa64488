// Steps 1-2 of the MoE FFN forward: top-K softmax routing and fixed-capacity
// drop-and-pad slot selection.
//
// [FC] "feat(cuda-graphs): capture fixed-capacity MoE execution", Design notes:
//      every expert gets exactly C = ceil(N*K*F/E) slots; the real
//      assignments are chosen by routing probability.
// [PF] "Permute-Free Grouped GEMM for MoE (bf16, gfx950)", section 4
//      (route_counts / route_within): per-expert counts and within-expert
//      ranks from one scan.
#include <math.h>

#include <initializer_list>

#include "moe_common.h"

namespace moe {
namespace {

// ---------------------------------------------------------------------------
// route_topk: a group of LPT lanes per token (16, 32 or 64, so a wave routes
// 64/LPT tokens).  Each lane holds VPL logits (expert v*LPT + lane); K rounds
// of a group-wide arg-max (ties -> lower expert) pick the experts in
// descending-logit order.  Lane k of the group keeps round k's winner, then
// the K-way softmax runs in float64: exp(l_k - l_0), a sum in k order that
// every lane forms identically through shuffles, one division, one rounding
// to float32.
// ---------------------------------------------------------------------------
constexpr int kTopkThreads = 256;

// DPP lane exchanges inside a 16-lane row (no LDS round trip).
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i within each half row
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i within the row
constexpr int kDppShr1 = 0x111;       // lane i <- lane i-1 within the row

template <int CTRL>
__device__ __forceinline__ int dpp(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(dpp<CTRL>(__float_as_int(v)));
}
template <int CTRL>
__device__ __forceinline__ double dpp(double v) {
    const long long b = __double_as_longlong(v);
    const int lo = dpp<CTRL>(static_cast<int>(b)), hi = dpp<CTRL>(static_cast<int>(b >> 32));
    return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<uint32_t>(lo));
}

// (value, expert) arg-max step: the partner wins if its value is larger, or
// equal with a lower expert index; INT32_MAX marks "no candidate".
__device__ __forceinline__ void argmax_step(float& bv, int& bi, float ov, int oi) {
    const bool better = oi != INT32_MAX && (bi == INT32_MAX || ov > bv || (ov == bv && oi < bi));
    if (better) { bv = ov; bi = oi; }
}

template <int LPT, int VPL>
__global__ __launch_bounds__(kTopkThreads) void route_topk_kernel(
    const float* __restrict__ logits, int N, int E, int K, int* __restrict__ topk_ids,
    float* __restrict__ topk_probs, int* __restrict__ zero_count, const int* __restrict__ n_live) {
    constexpr int TPB = kTopkThreads / LPT;   // tokens per block
    const int g = threadIdx.x % LPT;          // lane within the token's group
    const int t = blockIdx.x * TPB + threadIdx.x / LPT;
    // n_live (optional, device data, clamped to [0, N]): tokens at or past it
    // route nowhere -- expert -1, probability 0 -- and their logits are not read
    const int nl = n_live ? min(max(n_live[0], 0), N) : N;
    const bool live_token = t < nl;           // whole groups share t, so exchanges stay in-group
    const float* row = logits + static_cast<size_t>(live_token ? t : 0) * E;
    float v[VPL];
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
        const int e = j * LPT + g;
        v[j] = (live_token && e < E) ? row[e] : 0.0f;
    }
    uint32_t taken = 0;
    float my_logit = 0.0f;
    int my_id = 0;
    for (int k = 0; k < K; ++k) {
        float bv = 0.0f;
        int bi = INT32_MAX;
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
            const int e = j * LPT + g;
            const bool live = e < E && !((taken >> j) & 1u);
            if (live && (bi == INT32_MAX || v[j] > bv)) { bv = v[j]; bi = e; }
        }
        // all-reduce over the 16-lane row with DPP, then across rows
        argmax_step(bv, bi, dpp<kDppXor1>(bv), dpp<kDppXor1>(bi));
        argmax_step(bv, bi, dpp<kDppXor2>(bv), dpp<kDppXor2>(bi));
        argmax_step(bv, bi, dpp<kDppHalfMirror>(bv), dpp<kDppHalfMirror>(bi));
        argmax_step(bv, bi, dpp<kDppMirror>(bv), dpp<kDppMirror>(bi));
#pragma unroll
        for (int off = 16; off < LPT; off <<= 1)
            argmax_step(bv, bi, __shfl_xor(bv, off, LPT), __shfl_xor(bi, off, LPT));
        if (bi % LPT == g) taken |= 1u << (bi / LPT);
        if (g == k) { my_logit = bv; my_id = bi; }
    }
    const double top = static_cast<double>(__shfl(my_logit, 0, LPT));
    const double ex = g < K ? exp(static_cast<double>(my_logit) - top) : 0.0;
    // denominator: e_0 + e_1 + ... + e_{K-1} in k order.  In a 16-lane row,
    // K-1 rounds of s <- s(lane-1) + e leave lane K-1 holding the ordered sum.
    double denom;
    if (LPT == 16) {
        double s = ex;
        for (int it = 1; it < K; ++it) {
            const double prev = dpp<kDppShr1>(s);
            s = g == 0 ? ex : prev + ex;
        }
        denom = __shfl(s, K - 1, LPT);
    } else {
        denom = 0.0;
        for (int k = 0; k < K; ++k) denom += __shfl(ex, k, LPT);
    }
    if (t < N && g < K) {
        topk_ids[static_cast<size_t>(t) * K + g] = live_token ? my_id : -1;
        topk_probs[static_cast<size_t>(t) * K + g] = live_token ? static_cast<float>(ex / denom) : 0.0f;
    }
    // the fused align counts kept routes per token with atomics: start at 0
    if (zero_count && t < N && g == 0) zero_count[t] = 0;
}

// ---------------------------------------------------------------------------
// capacity_select: one 1024-thread workgroup per expert.
//  1. Compaction: scan topk_ids in route order (t*K + k, i.e. token order),
//     per-thread match masks over 32 routes + a block prefix scan, and append
//     this expert's candidate route indices to LDS.  If load <= C every
//     candidate is kept in that order and the kernel is done.
//  2. Else gather the candidates' probabilities (bit patterns) in one batch.
//     Up to 2048 candidates: rank each one by counting those that beat it and
//     keep ranks < C.  Beyond that: radix-select (4 x 8-bit digits, LDS
//     histograms) the C-th
//     largest probability T and how many candidates equal to T still fit.
//     Probabilities are positive floats, so their bit patterns order like
//     their values.
//  3. Keep key > T, plus the first `need` candidates with key == T in token
//     order; a second block scan numbers the kept routes 0..count-1 in token
//     order.  Every route_slot entry of this expert gets exactly one write.
// ---------------------------------------------------------------------------
constexpr int kSelThreads = 1024;
constexpr int kSelChunk = 32;   // routes per thread per compaction pass
constexpr int kRankMax = 2048;  // rank counting up to this load, radix select above

// Step 3's outputs, when the selection writes them itself (the fused
// route + capacity + align call).  Expert e's workgroup owns its segment of
// the route list and every route whose top-K pick is e, so each element has
// exactly one writer; the per-token kept counts are the one shared output
// (integer atomics on counters the top-K kernel zeroed).
struct AlignOut {
    int* sorted_slot_ids;      // null: selection only
    float* slot_probs;
    int* expert_ids;
    int* block_start;
    int* token_routes;
    int* token_route_count;
    int* num_tokens_post_padded;
    int N, K, E, Cp;
};

// One candidate's outcome: route r (= t*K + k) of expert e is kept in `slot`
// (>= 0) or dropped (-1); `prob` is its routing probability.
__device__ __forceinline__ void emit_route(const AlignOut& ao, int e, int r, int slot, float prob) {
    if (!ao.sorted_slot_ids) return;
    if (slot >= 0) {
        const int s = e * ao.Cp + slot;
        ao.sorted_slot_ids[s] = r / ao.K;
        ao.slot_probs[s] = prob;
        ao.token_routes[r] = s;
        atomicAdd(&ao.token_route_count[r / ao.K], 1);
    } else {
        ao.token_routes[r] = -1;
    }
}

// The rest of expert e's segment once `kept` slots are taken: pad slots
// (sentinel row N, probability +0), the blocks' owner, the first block, and
// (expert 0) the padded extent.
__device__ __forceinline__ void emit_segment(const AlignOut& ao, int e, int kept, int tid) {
    if (!ao.sorted_slot_ids) return;
    for (int j = kept + tid; j < ao.Cp; j += kSelThreads) {
        ao.sorted_slot_ids[e * ao.Cp + j] = ao.N;
        ao.slot_probs[e * ao.Cp + j] = 0.0f;
    }
    const int blocks = ao.Cp / kBlockM;
    for (int b = tid; b < blocks; b += kSelThreads) ao.expert_ids[e * blocks + b] = e;
    if (tid == 0) {
        ao.block_start[e] = e * blocks;
        if (e == 0) ao.num_tokens_post_padded[0] = ao.E * ao.Cp;
    }
}

__global__ __launch_bounds__(kSelThreads) void capacity_select_kernel(
    const int* __restrict__ ids, const float* __restrict__ probs, int NK, int C,
    int* __restrict__ route_slot, int* __restrict__ expert_count, AlignOut ao) {
    __shared__ uint32_t s_route[kMaxN];
    __shared__ __attribute__((aligned(16))) uint32_t s_key[kMaxN];
    __shared__ int s_scan[kSelThreads / kWave];
    __shared__ int s_hist[256];
    __shared__ uint32_t s_pick[2];
    const int e = blockIdx.x;
    const int tid = threadIdx.x;

    // 1. compaction of this expert's route indices, in route (= token) order
    int load = 0;
    for (int base = 0; base < NK; base += kSelThreads * kSelChunk) {
        const int start = base + tid * kSelChunk;
        uint32_t mask = 0;
        if (start + kSelChunk <= NK) {
            const int4* p = reinterpret_cast<const int4*>(ids + start);
            int4 v[kSelChunk / 4];
#pragma unroll
            for (int q = 0; q < kSelChunk / 4; ++q) v[q] = p[q];   // all loads in flight at once
#pragma unroll
            for (int q = 0; q < kSelChunk / 4; ++q) {
                mask |= (v[q].x == e ? 1u : 0u) << (4 * q + 0);
                mask |= (v[q].y == e ? 1u : 0u) << (4 * q + 1);
                mask |= (v[q].z == e ? 1u : 0u) << (4 * q + 2);
                mask |= (v[q].w == e ? 1u : 0u) << (4 * q + 3);
            }
        } else {
            for (int j = 0; j < kSelChunk; ++j)
                if (start + j < NK && ids[start + j] == e) mask |= 1u << j;
        }
        int total = 0;
        int pos = load + block_exclusive_scan(__popc(mask), s_scan, &total);
        while (mask) {
            const int j = __ffs(mask) - 1;
            mask &= mask - 1;
            if (pos < kMaxN) s_route[pos] = static_cast<uint32_t>(start + j);   // load <= N <= kMaxN
            ++pos;
        }
        load += total;
    }
    load = min(load, static_cast<int>(kMaxN));
    __syncthreads();

    if (load <= C) {   // every candidate fits: slot = position in token order
        for (int i = tid; i < load; i += kSelThreads) {
            const int r = static_cast<int>(s_route[i]);
            route_slot[r] = i;
            if (ao.sorted_slot_ids) emit_route(ao, e, r, i, probs[r]);
        }
        emit_segment(ao, e, load, tid);
        if (tid == 0) expert_count[e] = load;
        return;
    }
    // over capacity: gather the candidates' probabilities (one batch of loads);
    // keys past `load` up to a multiple of 16 are zero (a zero key never beats
    // a probability, which is > 0)
    const int padded = (load + 15) & ~15;
    for (int i = tid; i < padded; i += kSelThreads)
        s_key[i] = i < load ? __float_as_uint(probs[s_route[i]]) : 0u;
    __syncthreads();

    if (load <= kRankMax) {
        // 2'. rank counting: candidate i is kept iff fewer than C candidates
        // beat it (a larger key, or an equal key and a lower token, which in
        // this token-ordered list means a lower position).  Both rules fold
        // into one 64-bit key, (key << 32) | (2^32 - 1 - position): j beats i
        // iff its 64-bit key is larger.  Wave w counts, for the 64 candidates
        // of group w % G, the beaters among the P-th part w / G of the list
        // (G groups, P = waves / G parts), and the parts add up in LDS.  All
        // lanes of a wave read the same key at once (an LDS broadcast), so
        // there is no contention, unlike histogram atomics on the few exponent
        // digits the probabilities share.  Ranks live past the keys
        // (s_key[kRankMax..]), the 64-bit keys past those; kept flags go to
        // bit 31 of s_route.  Keys past `load` are zero and never beat a
        // probability, which is > 0.
        uint32_t* s_rank = s_key + kRankMax;
        uint64_t* s_k64 = reinterpret_cast<uint64_t*>(s_key + 2 * kRankMax);
        for (int i = tid; i < padded; i += kSelThreads) {
            if (i < load) s_rank[i] = 0;
            s_k64[i] = i < load ? (static_cast<uint64_t>(s_key[i]) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(i))
                                : 0ull;
        }
        __syncthreads();
        constexpr int kWaves = kSelThreads / kWave;
        const int groups = (load + kWave - 1) / kWave;             // waves take turns when > kWaves
        const int wave = tid / kWave, lane = tid % kWave;
        for (int task = wave; task < groups * max(1, kWaves / groups); task += kWaves) {
            const int parts = max(1, kWaves / groups);
            const int g = task % groups, part = task / groups;
            const int chunk = (padded / 16 + parts - 1) / parts * 16;   // keys per part
            const int j0 = part * chunk, j1 = min(padded, j0 + chunk);
            const int i = g * kWave + lane;
            const uint64_t ki = i < load ? s_k64[i] : ~0ull;
            int rank = 0;
            const ulonglong2* k2 = reinterpret_cast<const ulonglong2*>(s_k64);
            for (int j = j0; j < j1; j += 16) {   // 8 independent 16-byte reads per trip
                ulonglong2 q[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) q[u] = k2[j / 2 + u];
#pragma unroll
                for (int u = 0; u < 8; ++u) rank += (q[u].x > ki) + (q[u].y > ki);
            }
            if (i < load && rank) atomicAdd(&s_rank[i], static_cast<uint32_t>(rank));
        }
        __syncthreads();
        for (int i = tid; i < load; i += kSelThreads)
            if (s_rank[i] < static_cast<uint32_t>(C)) s_route[i] |= 0x80000000u;
        __syncthreads();
        const int per = (load + kSelThreads - 1) / kSelThreads;
        const int lo = min(load, tid * per), hi = min(load, lo + per);
        int kept = 0;
        for (int i = lo; i < hi; ++i) kept += static_cast<int>(s_route[i] >> 31);
        int tot = 0;
        int slot = block_exclusive_scan(kept, s_scan, &tot);
        for (int i = lo; i < hi; ++i) {
            const uint32_t r = s_route[i];
            const int sl = (r >> 31) ? slot++ : -1;
            route_slot[r & 0x7FFFFFFFu] = sl;
            emit_route(ao, e, static_cast<int>(r & 0x7FFFFFFFu), sl, __uint_as_float(s_key[i]));
        }
        emit_segment(ao, e, C, tid);
        if (tid == 0) expert_count[e] = C;
        return;
    }

    // 2. radix select of the C-th largest key
    uint32_t prefix = 0, prefix_mask = 0;
    int remaining = C;   // rank still to locate among keys that match prefix
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int i = tid; i < 256; i += kSelThreads) s_hist[i] = 0;
        __syncthreads();
        for (int i = tid; i < load; i += kSelThreads) {
            const uint32_t k = s_key[i];
            if ((k & prefix_mask) == prefix) atomicAdd(&s_hist[(k >> shift) & 255u], 1);
        }
        __syncthreads();
        if (tid < kWave) {
            // lane l owns digits 255-4l .. 252-4l (descending)
            int h[4], own = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) { h[j] = s_hist[255 - 4 * tid - j]; own += h[j]; }
            const int inc = wave_inclusive_scan(own);
            const unsigned long long hit = __ballot(inc >= remaining);
            const int L = __ffsll(static_cast<long long>(hit)) - 1;   // first lane reaching the rank
            if (tid == L) {
                int above = inc - own;   // keys with a larger digit
                int d = 255 - 4 * tid;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (above + h[j] >= remaining) { d = 255 - 4 * tid - j; break; }
                    above += h[j];
                }
                s_pick[0] = static_cast<uint32_t>(d);
                s_pick[1] = static_cast<uint32_t>(remaining - above);
            }
        }
        __syncthreads();
        prefix |= s_pick[0] << shift;
        prefix_mask |= 255u << shift;
        remaining = static_cast<int>(s_pick[1]);
        __syncthreads();
    }
    const uint32_t T = prefix;
    const int need = remaining;   // candidates with key == T that are kept

    // 3. keep and number in token order (contiguous chunks keep the order)
    const int per = (load + kSelThreads - 1) / kSelThreads;
    const int lo = min(load, tid * per), hi = min(load, lo + per);
    int gt = 0, eq = 0;
    for (int i = lo; i < hi; ++i) {
        const uint32_t k = s_key[i];
        gt += k > T;
        eq += k == T;
    }
    int tot = 0;
    const int eq_base = block_exclusive_scan(eq, s_scan, &tot);
    const int eq_keep = max(0, min(eq, need - eq_base));
    int slot = block_exclusive_scan(gt + eq_keep, s_scan, &tot);
    int eq_seen = eq_base;
    for (int i = lo; i < hi; ++i) {
        const uint32_t k = s_key[i];
        bool keep = k > T;
        if (k == T) { keep = eq_seen < need; ++eq_seen; }
        const int sl = keep ? slot++ : -1;
        route_slot[s_route[i]] = sl;
        emit_route(ao, e, static_cast<int>(s_route[i]), sl, __uint_as_float(k));
    }
    emit_segment(ao, e, C, tid);
    if (tid == 0) expert_count[e] = C;
}

template <int LPT, int VPL>
void launch_topk(const float* logits, int N, int E, int K, int* ids, float* probs, int* zero_count,
                 const int* n_live, hipStream_t s) {
    constexpr int TPB = kTopkThreads / LPT;
    const int blocks = (N + TPB - 1) / TPB;
    route_topk_kernel<LPT, VPL><<<blocks, kTopkThreads, 0, s>>>(logits, N, E, K, ids, probs, zero_count,
                                                                n_live);
}

// Lanes per token: enough for K (lane k finishes route k) and for E in at
// most 8 logits per lane when it fits, else all 64 lanes.
void dispatch_topk(const float* logits, int N, int E, int K, int* ids, float* probs, int* zero_count,
                   hipStream_t s, const int* n_live = nullptr) {
    if (K <= 16 && E <= 128) {
        if (E <= 32) launch_topk<16, 2>(logits, N, E, K, ids, probs, zero_count, n_live, s);
        else if (E <= 64) launch_topk<16, 4>(logits, N, E, K, ids, probs, zero_count, n_live, s);
        else launch_topk<16, 8>(logits, N, E, K, ids, probs, zero_count, n_live, s);
    } else if (E <= 256) {
        if (E <= 128) launch_topk<32, 4>(logits, N, E, K, ids, probs, zero_count, n_live, s);
        else launch_topk<32, 8>(logits, N, E, K, ids, probs, zero_count, n_live, s);
    } else if (E <= 512) {
        launch_topk<64, 8>(logits, N, E, K, ids, probs, zero_count, n_live, s);
    } else {
        launch_topk<64, 16>(logits, N, E, K, ids, probs, zero_count, n_live, s);
    }
}

}  // namespace
}  // namespace moe

namespace moe {
namespace {

int check_route_ptrs(std::initializer_list<const void*> ptrs) {
    for (const void* q : ptrs) {
        if (!q) return MOE_ERR_INVALID_ARG;
        if (!aligned16(q)) return MOE_ERR_MISALIGNED;
    }
    return MOE_OK;
}

}  // namespace
}  // namespace moe

extern "C" int moe_route_capacity(const float* logits, int64_t N, int32_t E, int32_t K, int64_t C,
                                  int32_t* topk_ids, float* topk_probs, int32_t* route_slot,
                                  int32_t* expert_count, hipStream_t stream) {
    using namespace moe;
    int st = check_route_shape(N, E, K, C);
    if (st != MOE_OK) return st;
    if (N == 0) return MOE_OK;
    st = check_route_ptrs({logits, topk_ids, topk_probs, route_slot, expert_count});
    if (st != MOE_OK) return st;
    const int n = static_cast<int>(N);
    dispatch_topk(logits, n, E, K, topk_ids, topk_probs, nullptr, stream);
    capacity_select_kernel<<<E, kSelThreads, 0, stream>>>(topk_ids, topk_probs, n * K,
                                                          static_cast<int>(C), route_slot,
                                                          expert_count, AlignOut{});
    return launch_status();
}

extern "C" int moe_route_capacity_align(const float* logits, int64_t N, int32_t E, int32_t K,
                                        int64_t C, int32_t* topk_ids, float* topk_probs,
                                        int32_t* route_slot, int32_t* expert_count,
                                        int32_t* sorted_slot_ids, float* slot_probs,
                                        int32_t* expert_ids, int32_t* block_start,
                                        int32_t* token_routes, int32_t* token_route_count,
                                        int32_t* num_tokens_post_padded, hipStream_t stream) {
    using namespace moe;
    int st = check_route_shape(N, E, K, C);
    if (st != MOE_OK) return st;
    if (N == 0) return MOE_OK;
    st = check_route_ptrs({logits, topk_ids, topk_probs, route_slot, expert_count, sorted_slot_ids,
                           slot_probs, expert_ids, block_start, token_routes, token_route_count,
                           num_tokens_post_padded});
    if (st != MOE_OK) return st;
    const int n = static_cast<int>(N);
    const AlignOut ao{sorted_slot_ids, slot_probs, expert_ids, block_start, token_routes,
                      token_route_count, num_tokens_post_padded, n, K, E,
                      static_cast<int>(moe_padded_capacity(C))};
    dispatch_topk(logits, n, E, K, topk_ids, topk_probs, token_route_count, stream);
    capacity_select_kernel<<<E, kSelThreads, 0, stream>>>(topk_ids, topk_probs, n * K,
                                                          static_cast<int>(C), route_slot,
                                                          expert_count, ao);
    return launch_status();
}

namespace moe {
namespace {

int route_dropless(const float* logits, int64_t N, int32_t E, int32_t K, const int32_t* n_live,
                   int32_t* topk_ids, float* topk_probs, int32_t* route_within,
                   int32_t* route_counts, int32_t* sorted_slot_ids, float* slot_probs,
                   int32_t* expert_ids, int32_t* block_start, int32_t* token_routes,
                   int32_t* token_route_count, int32_t* num_tokens_post_padded,
                   hipStream_t stream) {
    int st = check_route_shape(N, E, K, N);
    if (st != MOE_OK) return st;
    if (moe_dropless_bound(N, K, E) > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    if (N == 0) return MOE_OK;
    st = check_route_ptrs({logits, topk_ids, topk_probs, route_within, route_counts,
                           sorted_slot_ids, slot_probs, expert_ids, block_start, token_routes,
                           token_route_count, num_tokens_post_padded});
    if (st != MOE_OK) return st;
    const int n = static_cast<int>(N);
    dispatch_topk(logits, n, E, K, topk_ids, topk_probs, nullptr, stream, n_live);
    // A capacity of N never binds (an expert gets at most one route per
    // token): the selection pass then only ranks each expert's routes in
    // token order and counts them.  Routes of tokens past n_live carry
    // expert -1 and match no expert.
    capacity_select_kernel<<<E, kSelThreads, 0, stream>>>(topk_ids, topk_probs, n * K, n,
                                                          route_within, route_counts, AlignOut{});
    st = launch_align_dropless(topk_ids, topk_probs, route_within, route_counts, N, E, K,
                               sorted_slot_ids, slot_probs, expert_ids, block_start, token_routes,
                               token_route_count, num_tokens_post_padded, stream, n_live);
    return st != MOE_OK ? st : launch_status();
}

}  // namespace
}  // namespace moe

extern "C" int moe_route_dropless(const float* logits, int64_t N, int32_t E, int32_t K,
                                  int32_t* topk_ids, float* topk_probs, int32_t* route_within,
                                  int32_t* route_counts, int32_t* sorted_slot_ids,
                                  float* slot_probs, int32_t* expert_ids, int32_t* block_start,
                                  int32_t* token_routes, int32_t* token_route_count,
                                  int32_t* num_tokens_post_padded, hipStream_t stream) {
    return moe::route_dropless(logits, N, E, K, nullptr, topk_ids, topk_probs, route_within,
                               route_counts, sorted_slot_ids, slot_probs, expert_ids, block_start,
                               token_routes, token_route_count, num_tokens_post_padded, stream);
}

extern "C" int moe_route_dropless_live(const float* logits, int64_t N, int32_t E, int32_t K,
                                       const int32_t* n_live, int32_t* topk_ids,
                                       float* topk_probs, int32_t* route_within,
                                       int32_t* route_counts, int32_t* sorted_slot_ids,
                                       float* slot_probs, int32_t* expert_ids,
                                       int32_t* block_start, int32_t* token_routes,
                                       int32_t* token_route_count,
                                       int32_t* num_tokens_post_padded, hipStream_t stream) {
    if (!n_live) return MOE_ERR_INVALID_ARG;
    if (!moe::aligned16(n_live)) return MOE_ERR_MISALIGNED;
    return moe::route_dropless(logits, N, E, K, n_live, topk_ids, topk_probs, route_within,
                               route_counts, sorted_slot_ids, slot_probs, expert_ids, block_start,
                               token_routes, token_route_count, num_tokens_post_padded, stream);
}
