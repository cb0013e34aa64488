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

#include <algorithm>
#include <atomic>
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
//
// The kernel also writes the routing map ([PF] section 4 builds its layout
// from the routing map), expert-major: byte map[e * Np + t] = k + 1 if token
// t's pick k is expert e, else 0 (Np = N rounded up to 16, every byte of
// [0, Np) written each call), and beside it pmap[e * Np + t] = that pick's
// probability (written at the picks only; elsewhere stale and never read).
// A workgroup's TPB tokens form one TPB-byte piece of each expert's map row,
// assembled in LDS and stored whole, so an expert's selection later reads
// only its own rows -- picks and probabilities in one round trip -- instead
// of every pick.
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

// Arg-max key of (logit, expert): the float's bits made monotonic as an
// unsigned integer in the high word (with -0 folded onto +0 first, so equal
// logits stay equal), and ~expert in the low word, so the larger key is the
// larger logit and, between equal logits, the lower expert -- the order the
// routing defines, decided by one unsigned comparison with no branches.  Any
// real logit's key exceeds 2^32; a key with a zero high word has been picked.
__device__ __forceinline__ uint64_t topk_key(float v, int e) {
    const uint32_t b = __float_as_uint(v + 0.0f);
    const uint32_t u = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    return (static_cast<uint64_t>(u) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(e));
}
__device__ __forceinline__ float key_logit(uint64_t key) {
    const uint32_t u = static_cast<uint32_t>(key >> 32);
    return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}
__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }
template <int CTRL>
__device__ __forceinline__ uint64_t dpp64(uint64_t v) {
    const int lo = dpp<CTRL>(static_cast<int>(v)), hi = dpp<CTRL>(static_cast<int>(v >> 32));
    return (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) | static_cast<uint32_t>(lo);
}
__device__ __forceinline__ uint64_t shfl_xor64(uint64_t v, int off, int width) {
    const int lo = __shfl_xor(static_cast<int>(v), off, width);
    const int hi = __shfl_xor(static_cast<int>(v >> 32), off, width);
    return (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) | static_cast<uint32_t>(lo);
}

// Largest E each group width serves (see dispatch_topk), hence the LDS piece
// of the routing map: E rows of TPB bytes.
template <int LPT>
constexpr int topk_max_e() { return LPT == 16 ? 128 : LPT == 32 ? 256 : kMaxE; }

template <int LPT, int VPL>
__global__ __launch_bounds__(kTopkThreads) void route_topk_kernel(
    const float* __restrict__ logits, int N, int E, int K, int* __restrict__ topk_ids,
    float* __restrict__ topk_probs, int* __restrict__ zero_count, const int* __restrict__ n_live,
    uint8_t* __restrict__ map, uint32_t* __restrict__ pmap, int Np) {
    constexpr int TPB = kTopkThreads / LPT;   // tokens per block
    constexpr int MAP_WORDS = topk_max_e<LPT>() * TPB / 4;
    __shared__ uint32_t s_map[MAP_WORDS];
    const int g = threadIdx.x % LPT;          // lane within the token's group
    const int tl = threadIdx.x / LPT;         // token within the block
    const int t = blockIdx.x * TPB + tl;
    for (int i = threadIdx.x; i < E * TPB / 4; i += kTopkThreads) s_map[i] = 0u;
    // n_live (optional, device data, clamped to [0, N]): tokens at or past it
    // route nowhere -- expert -1, probability 0 -- and their logits are not read
    const int nl = n_live ? min(max(n_live[0], 0), N) : N;
    const bool live_token = t < nl;           // whole groups share t, so exchanges stay in-group
    const float* row = logits + static_cast<size_t>(live_token ? t : 0) * E;
    uint64_t key[VPL];                        // 0 = no expert there
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
        const int e = j * LPT + g;
        key[j] = (live_token && e < E) ? topk_key(row[e], e) : 0ull;
    }
    float my_logit = 0.0f;
    int my_id = 0;
    for (int k = 0; k < K; ++k) {
        // the lane's best remaining key (a tree for independent comparisons),
        // then the group's, by DPP inside 16-lane rows and shuffles across them
        uint64_t m[VPL];
#pragma unroll
        for (int j = 0; j < VPL; ++j) m[j] = key[j];
#pragma unroll
        for (int w = 1; w < VPL; w <<= 1)
#pragma unroll
            for (int j = 0; j + w < VPL; j += 2 * w) m[j] = umax64(m[j], m[j + w]);
        uint64_t best = m[0];
        best = umax64(best, dpp64<kDppXor1>(best));
        best = umax64(best, dpp64<kDppXor2>(best));
        best = umax64(best, dpp64<kDppHalfMirror>(best));
        best = umax64(best, dpp64<kDppMirror>(best));
#pragma unroll
        for (int off = 16; off < LPT; off <<= 1) best = umax64(best, shfl_xor64(best, off, LPT));
        // the winner leaves the running: its key keeps only the low word
        const uint32_t won = static_cast<uint32_t>(best);
#pragma unroll
        for (int j = 0; j < VPL; ++j)
            if (static_cast<uint32_t>(key[j]) == won) key[j] = won;
        if (g == k) { my_logit = key_logit(best); my_id = static_cast<int>(0xFFFFFFFFu - won); }
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
    const float prob = static_cast<float>(ex / denom);
    const bool pick = live_token && g < K && static_cast<unsigned>(my_id) < static_cast<unsigned>(E);
    if (t < N && g < K) {
        topk_ids[static_cast<size_t>(t) * K + g] = live_token ? my_id : -1;
        topk_probs[static_cast<size_t>(t) * K + g] = live_token ? prob : 0.0f;
    }
    if (pick) pmap[static_cast<size_t>(my_id) * Np + t] = __float_as_uint(prob);
    // the fused align counts kept routes per token with atomics: start at 0
    if (zero_count && t < N && g == 0) zero_count[t] = 0;
    __syncthreads();                          // the piece is zeroed
    if (pick) reinterpret_cast<uint8_t*>(s_map)[my_id * TPB + tl] = static_cast<uint8_t>(g + 1);
    __syncthreads();
    // expert e's TPB bytes of this block's tokens, one store each
    const size_t col = static_cast<size_t>(blockIdx.x) * TPB;
    for (int e = threadIdx.x; e < E; e += kTopkThreads) {
        uint8_t* dst = map + static_cast<size_t>(e) * Np + col;
        if (TPB == 16) *reinterpret_cast<uint4*>(dst) = reinterpret_cast<const uint4*>(s_map)[e];
        else if (TPB == 8) *reinterpret_cast<uint2*>(dst) = reinterpret_cast<const uint2*>(s_map)[e];
        else *reinterpret_cast<uint32_t*>(dst) = s_map[e];
    }
}

// ---------------------------------------------------------------------------
// capacity_select: one workgroup per expert.
//  1. Compaction: read the expert's rows of the routing map (one 16-byte
//     piece of picks and its 64 bytes of probabilities per thread, in one
//     round trip), one block prefix scan, and append one 64-bit key per
//     candidate to LDS in token order: (probability << 32) | (2^32-1 - r),
//     r = t*K + k the route.  Routes grow with the token, so the larger key
//     is the one kept first -- larger probability, then the lower token --
//     and every key is distinct and names its route.  If load <= C every
//     candidate is kept in that order and the kernel is done.
//  2. Else up to kRankMax candidates: a sample select finds the C-th largest
//     key T exactly.  Beyond that: radix-select (4 x 8-bit digits, LDS
//     histograms) the C-th largest probability and how many candidates equal
//     to it still fit.  Probabilities are positive floats, so their bit
//     patterns order like their values.
//  3. Keep the candidates at or above the threshold (ties in token order); a
//     second block scan numbers the kept routes 0..count-1 in token order.
//     Every route_slot entry of this expert gets exactly one write.
// LDS is sized by N at launch: the keys (N) and, for the sample select, the
// keys of its bracket (up to kRankMax).
// ---------------------------------------------------------------------------
constexpr int kRankMax = 2048;  // sample select up to this load, radix select above

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
__device__ __forceinline__ void emit_segment(const AlignOut& ao, int e, int kept, int tid, int nthreads) {
    if (!ao.sorted_slot_ids) return;
    for (int j = kept + tid; j < ao.Cp; j += nthreads) {
        ao.sorted_slot_ids[e * ao.Cp + j] = ao.N;
        ao.slot_probs[e * ao.Cp + j] = 0.0f;
    }
    const int blocks = ao.Cp / kBlockM;
    for (int b = tid; b < blocks; b += nthreads) ao.expert_ids[e * blocks + b] = e;
    if (tid == 0) {
        ao.block_start[e] = e * blocks;
        if (e == 0) ao.num_tokens_post_padded[0] = ao.E * ao.Cp;
    }
}

// LDS of one selection workgroup, in 32-bit words: two per key for N keys
// rounded up to 16, then two per bracket key for up to kRankMax of them.
inline int round16(int n) { return (n + 15) & ~15; }
inline size_t select_lds_bytes(int N) {
    return static_cast<size_t>(2 * round16(N) + 2 * round16(std::min(N, kRankMax))) * 4u;
}
__device__ __forceinline__ int key_route(uint64_t key) {
    return static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(key));
}
__device__ __forceinline__ uint32_t key_prob(uint64_t key) { return static_cast<uint32_t>(key >> 32); }

// Sum over each 16-lane row, left in every lane of the row (DPP lane moves).
__device__ __forceinline__ int row_sum(int v) {
    v += dpp<kDppXor1>(v);
    v += dpp<kDppXor2>(v);
    v += dpp<kDppHalfMirror>(v);
    v += dpp<kDppMirror>(v);
    return v;
}
// Maximum over the whole wave, uniform: DPP inside the rows, then the four
// row maxima read as scalars.
__device__ __forceinline__ int wave_max(int v) {
    v = max(v, dpp<kDppXor1>(v));
    v = max(v, dpp<kDppXor2>(v));
    v = max(v, dpp<kDppHalfMirror>(v));
    v = max(v, dpp<kDppMirror>(v));
    return max(max(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
               max(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}

// Bytes of a 16-byte map piece that hold a pick: bit j of the result for
// byte j in 1..K (larger values are not trusted) of a token t < N.
__device__ __forceinline__ uint32_t pick_mask(uint4 q, int t0, int N, int K) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const uint32_t b = (w[j >> 2] >> (8 * (j & 3))) & 0xFFu;
        m |= static_cast<uint32_t>(b != 0u && b <= static_cast<uint32_t>(K) && t0 + j < N) << j;
    }
    return m;
}

// NT threads, one 16-byte map piece each: the launch picks the narrowest
// width that covers the map row, since the workgroup's time is the time its
// waves take to issue their instructions on the one CU that holds them.
template <int NT>
__global__ __launch_bounds__(NT) void capacity_select_kernel(
    const uint8_t* __restrict__ map, const uint32_t* __restrict__ pmap, int Np, int N, int K, int C,
    int* __restrict__ route_slot, int* __restrict__ expert_count, AlignOut ao) {
    extern __shared__ __attribute__((aligned(16))) uint64_t s_dyn[];
    uint64_t* s_k64 = s_dyn;                                        // [round16(N)] candidate keys
    uint64_t* s_b = s_dyn + ((N + 15) & ~15);                       // [round16(min(N, kRankMax))] bracket
    constexpr int kSelThreads = NT;
    __shared__ int s_scan[NT / kWave];
    __shared__ int s_hist[256];
    __shared__ uint32_t s_pick[2];
    const int e = blockIdx.x;
    const int tid = threadIdx.x;

    // 1. compaction: thread i holds piece i (tokens 16i .. 16i+15)
    const int pieces = Np / 16;
    uint4 v = make_uint4(0u, 0u, 0u, 0u), pv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) pv[q] = v;
    if (tid < pieces) {   // the piece's picks and their probabilities, in one round trip
        v = reinterpret_cast<const uint4*>(map + static_cast<size_t>(e) * Np)[tid];
        const uint4* prow = reinterpret_cast<const uint4*>(pmap + static_cast<size_t>(e) * Np) + 4 * tid;
#pragma unroll
        for (int q = 0; q < 4; ++q) pv[q] = prow[q];
    }
    const uint32_t m = pick_mask(v, tid * 16, N, K);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    const uint32_t pw[16] = {pv[0].x, pv[0].y, pv[0].z, pv[0].w, pv[1].x, pv[1].y, pv[1].z, pv[1].w,
                             pv[2].x, pv[2].y, pv[2].z, pv[2].w, pv[3].x, pv[3].y, pv[3].z, pv[3].w};
    int load = 0;
    int pos = block_exclusive_scan(__popc(m), s_scan, &load);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        if ((m >> j) & 1u) {
            const int k = static_cast<int>((w[j >> 2] >> (8 * (j & 3))) & 0xFFu) - 1;
            const uint32_t r = static_cast<uint32_t>((tid * 16 + j) * K + k);
            s_k64[pos++] = (static_cast<uint64_t>(pw[j]) << 32) | (0xFFFFFFFFu - r);
        }
    }
    // zero keys past `load` up to a multiple of 16: below every candidate's
    // (whose low word is never 0), so a zero key never counts
    const int padded = (load + 15) & ~15;
    if (tid < padded - load) s_k64[load + tid] = 0ull;
    __syncthreads();

    if (load <= C) {   // every candidate fits: slot = position in token order
        for (int i = tid; i < load; i += kSelThreads) {
            const uint64_t k = s_k64[i];
            route_slot[key_route(k)] = i;
            emit_route(ao, e, key_route(k), i, __uint_as_float(key_prob(k)));
        }
        emit_segment(ao, e, load, tid, NT);
        if (tid == 0) expert_count[e] = load;
        return;
    }

    if (load <= kRankMax) {
        // 2'. sample select of T, the C-th largest key; the kept candidates
        // are exactly those with key >= T.
        //  a. NT/16 splitters (the candidates at positions s*load/S) are ranked
        //     against every key: the 16 lanes of a splitter's row count every
        //     16th key each and add up across the row;
        //  b. hi = the splitter of largest rank <= C-1 (key >= T) and lo = the
        //     one of smallest rank >= C (key < T) bracket T;
        //  c. unless hi is T itself, T is the key strictly inside the bracket
        //     whose rank, hi's rank + 1 + the bracket keys above it, is C-1.
        // The work is one pass over the keys plus the bracket (about load/S
        // keys) squared, instead of every pair of candidates.
        constexpr int S = NT / 16;                                 // splitters (<= 64)
        __shared__ uint64_t s_spl_key[S];
        __shared__ int s_spl_rank[S];
        __shared__ uint64_t s_bracket[3];                          // lo, hi, T
        __shared__ int s_rank_hi, s_bn;
        {
            const int sp = tid / 16, part = tid % 16;
            const uint64_t ks = s_k64[sp * load / S];
            int cnt = 0;
#pragma unroll 4
            for (int j = part; j < padded; j += 16) cnt += s_k64[j] > ks;
            cnt = row_sum(cnt);                                    // the splitter's rank, in its whole row
            if (part == 0) {
                s_spl_key[sp] = ks;
                s_spl_rank[sp] = cnt;
            }
        }
        __syncthreads();
        if (tid < kWave) {
            // lane q < S holds splitter q
            const bool real = tid < S;
            const int r = real ? s_spl_rank[tid] : -1;
            const uint64_t kq = real ? s_spl_key[tid] : 0ull;
            const int rhi = wave_max(real && r <= C - 1 ? r : -1);          // -1: no splitter at or above T
            const int rlo = -wave_max(real && r >= C ? -r : -INT32_MAX);     // INT32_MAX: none below T
            if (tid == 0) {
                s_bracket[0] = 0ull;                               // open ends: below and above every key
                s_bracket[1] = ~0ull;
                s_bracket[2] = ~0ull;                              // T, unless found below (C = 0: none kept)
                s_rank_hi = rhi;
                s_bn = 0;
            }
            // the splitters of those ranks name the bracket (repeated
            // splitters write the same key); a splitter of rank C-1 is T
            if (real && r == rlo) s_bracket[0] = kq;
            if (real && r == rhi) s_bracket[1] = kq;
            if (real && r == rhi && rhi == C - 1) s_bracket[2] = kq;
        }
        __syncthreads();
        const uint64_t klo = s_bracket[0], khi = s_bracket[1];
        const bool search = C > 0 && s_rank_hi != C - 1;          // uniform
        if (search) {
            for (int i = tid; i < load; i += kSelThreads) {
                const uint64_t k = s_k64[i];
                if (k > klo && k < khi) s_b[atomicAdd(&s_bn, 1)] = k;   // order within the bracket is free
            }
        }
        __syncthreads();
        // zero past the bracket's keys to a multiple of 8 (room: nb <= load <= kRankMax)
        const int nb = search ? s_bn : 0;
        const int nb8 = (nb + 7) & ~7;
        if (tid < nb8 - nb) s_b[nb + tid] = 0ull;
        __syncthreads();
        if (search) {
            for (int i = tid; i < nb; i += kSelThreads) {
                const uint64_t k = s_b[i];
                int r = s_rank_hi + 1;
                for (int j = 0; j < nb8; j += 8) {   // 8 reads in flight, then the comparisons
                    uint64_t q[8];
#pragma unroll
                    for (int u = 0; u < 8; ++u) q[u] = s_b[j + u];
#pragma unroll
                    for (int u = 0; u < 8; ++u) r += q[u] > k;
                }
                if (r == C - 1) s_bracket[2] = k;                  // exactly one key has rank C-1
            }
        }
        __syncthreads();
        const uint64_t T = s_bracket[2];
        // 3'. keep key >= T and number the kept routes in token order
        const int per = (load + kSelThreads - 1) / kSelThreads;
        const int lo = min(load, tid * per), hi = min(load, lo + per);
        int kept = 0;
        for (int i = lo; i < hi; ++i) kept += s_k64[i] >= T;
        int tot = 0;
        int slot = block_exclusive_scan(kept, s_scan, &tot);
        for (int i = lo; i < hi; ++i) {
            const uint64_t k = s_k64[i];
            const int sl = k >= T && slot < C ? slot++ : -1;
            route_slot[key_route(k)] = sl;
            emit_route(ao, e, key_route(k), sl, __uint_as_float(key_prob(k)));
        }
        tot = min(tot, max(C, 0));
        emit_segment(ao, e, tot, tid, NT);
        if (tid == 0) expert_count[e] = tot;
        return;
    }

    // 2. radix select of the C-th largest probability
    uint32_t prefix = 0, prefix_mask = 0;
    int remaining = C;   // rank still to locate among keys that match prefix
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int i = tid; i < 256; i += kSelThreads) s_hist[i] = 0;
        __syncthreads();
        for (int i = tid; i < load; i += kSelThreads) {
            const uint32_t k = key_prob(s_k64[i]);
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
    const int need = remaining;   // candidates with probability == T that are kept

    // 3. keep and number in token order (contiguous chunks keep the order)
    const int per = (load + kSelThreads - 1) / kSelThreads;
    const int lo = min(load, tid * per), hi = min(load, lo + per);
    int gt = 0, eq = 0;
    for (int i = lo; i < hi; ++i) {
        const uint32_t k = key_prob(s_k64[i]);
        gt += k > T;
        eq += k == T;
    }
    int tot = 0;
    const int eq_base = block_exclusive_scan(eq, s_scan, &tot);
    const int eq_keep = max(0, min(eq, need - eq_base));
    int slot = block_exclusive_scan(gt + eq_keep, s_scan, &tot);
    int eq_seen = eq_base;
    for (int i = lo; i < hi; ++i) {
        const uint64_t key = s_k64[i];
        const uint32_t k = key_prob(key);
        bool keep = k > T;
        if (k == T) { keep = eq_seen < need; ++eq_seen; }
        const int sl = keep ? slot++ : -1;
        route_slot[key_route(key)] = sl;
        emit_route(ao, e, key_route(key), sl, __uint_as_float(k));
    }
    emit_segment(ao, e, C, tid, NT);
    if (tid == 0) expert_count[e] = C;
}

// The routing map in the workspace: the pick bytes ([E, Np], Np = N rounded
// up to 16), then the pick probabilities ([E, Np] words).
struct RouteMap {
    uint8_t* picks;
    uint32_t* probs;
    int Np;
};

template <int LPT, int VPL>
void launch_topk(const float* logits, int N, int E, int K, int* ids, float* probs, int* zero_count,
                 const int* n_live, const RouteMap& rm, hipStream_t s) {
    constexpr int TPB = kTopkThreads / LPT;
    const int blocks = rm.Np / TPB;               // every byte of the map's rows, tail included
    route_topk_kernel<LPT, VPL><<<blocks, kTopkThreads, 0, s>>>(logits, N, E, K, ids, probs, zero_count,
                                                                n_live, rm.picks, rm.probs, rm.Np);
}

// Lanes per token: enough for K (lane k finishes route k) and for E in at
// most 8 logits per lane when it fits, else all 64 lanes.
void dispatch_topk(const float* logits, int N, int E, int K, int* ids, float* probs, int* zero_count,
                   const RouteMap& rm, hipStream_t s, const int* n_live = nullptr) {
    if (K <= 16 && E <= 128) {
        if (E <= 32) launch_topk<16, 2>(logits, N, E, K, ids, probs, zero_count, n_live, rm, s);
        else if (E <= 64) launch_topk<16, 4>(logits, N, E, K, ids, probs, zero_count, n_live, rm, s);
        else launch_topk<16, 8>(logits, N, E, K, ids, probs, zero_count, n_live, rm, s);
    } else if (E <= 256) {
        if (E <= 128) launch_topk<32, 4>(logits, N, E, K, ids, probs, zero_count, n_live, rm, s);
        else launch_topk<32, 8>(logits, N, E, K, ids, probs, zero_count, n_live, rm, s);
    } else if (E <= 512) {
        launch_topk<64, 8>(logits, N, E, K, ids, probs, zero_count, n_live, rm, s);
    } else {
        launch_topk<64, 16>(logits, N, E, K, ids, probs, zero_count, n_live, rm, s);
    }
}

template <int T>
void launch_select_t(const RouteMap& rm, int N, int E, int K, int C, int* route_slot,
                     int* expert_count, const AlignOut& ao, hipStream_t s) {
    const size_t lds = select_lds_bytes(N);
    // past 64 KB of dynamic LDS the launch needs the kernel's limit raised,
    // once per device (the attribute belongs to the device the call runs on)
    static std::atomic<bool> raised[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    if (lds > 64 * 1024 && (dev >= 64 || !raised[dev].load(std::memory_order_relaxed))) {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(capacity_select_kernel<T>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize,
                                  static_cast<int>(select_lds_bytes(static_cast<int>(kMaxN))));
        if (dev < 64) raised[dev].store(true, std::memory_order_relaxed);
    }
    capacity_select_kernel<T><<<E, T, lds, s>>>(rm.picks, rm.probs, rm.Np, N, K, C, route_slot,
                                                expert_count, ao);
}

// One map piece (16 tokens) per thread: the narrowest width that covers N.
void launch_select(const RouteMap& rm, int N, int E, int K, int C, int* route_slot,
                   int* expert_count, const AlignOut& ao, hipStream_t s) {
    static_assert(kMaxN <= 16 * 1024, "one map piece per thread");
    const int pieces = rm.Np / 16;
    if (pieces <= 256) launch_select_t<256>(rm, N, E, K, C, route_slot, expert_count, ao, s);
    else if (pieces <= 512) launch_select_t<512>(rm, N, E, K, C, route_slot, expert_count, ao, s);
    else launch_select_t<1024>(rm, N, E, K, C, route_slot, expert_count, ao, s);
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

// Row pitch of the routing map: N rounded up to whole 16-byte pieces.
int64_t map_pitch(int64_t N) { return (N + 15) / 16 * 16; }

// Workspace bytes: the pick bytes and the pick probabilities, E rows each.
size_t map_bytes(int64_t N, int32_t E) {
    return static_cast<size_t>(E) * static_cast<size_t>(map_pitch(N)) * 5u;
}

RouteMap route_map(void* ws, int64_t N, int32_t E) {
    const int64_t Np = map_pitch(N);
    uint8_t* picks = static_cast<uint8_t*>(ws);
    return RouteMap{picks, reinterpret_cast<uint32_t*>(picks + static_cast<size_t>(E) * Np),
                    static_cast<int>(Np)};
}

// The routing map lives in the caller's workspace: present, aligned, large enough.
int check_workspace(const void* ws, size_t bytes, int64_t N, int32_t E) {
    if (!ws) return MOE_ERR_INVALID_ARG;
    if (!aligned16(ws)) return MOE_ERR_MISALIGNED;
    if (bytes < map_bytes(N, E)) return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

// Steps 1-2 (align outputs in `ao` when the call also does step 3), once the
// arguments are validated; the routing map goes to the workspace.
void route_capacity_launch(const float* logits, int n, int E, int K, int C, int32_t* topk_ids,
                           float* topk_probs, int32_t* route_slot, int32_t* expert_count,
                           const AlignOut& ao, void* workspace, hipStream_t stream) {
    const RouteMap rm = route_map(workspace, n, E);
    dispatch_topk(logits, n, E, K, topk_ids, topk_probs, ao.token_route_count, rm, stream);
    launch_select(rm, n, E, K, C, route_slot, expert_count, ao, stream);
}

int route_dropless(const float* logits, int64_t N, int32_t E, int32_t K, const int32_t* n_live,
                   int32_t* topk_ids, float* topk_probs, int32_t* route_within,
                   int32_t* route_counts, int32_t* sorted_slot_ids, float* slot_probs,
                   int32_t* expert_ids, int32_t* block_start, int32_t* token_routes,
                   int32_t* token_route_count, int32_t* num_tokens_post_padded, void* workspace,
                   size_t workspace_bytes, hipStream_t stream) {
    int st = check_route_shape(N, E, K, N);
    if (st != MOE_OK) return st;
    if (moe_dropless_bound(N, K, E) > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    if (N == 0) return MOE_OK;
    st = check_route_ptrs({logits, topk_ids, topk_probs, route_within, route_counts,
                           sorted_slot_ids, slot_probs, expert_ids, block_start, token_routes,
                           token_route_count, num_tokens_post_padded});
    if (st != MOE_OK) return st;
    st = check_workspace(workspace, workspace_bytes, N, E);
    if (st != MOE_OK) return st;
    const int n = static_cast<int>(N);
    const RouteMap rm = route_map(workspace, N, E);
    dispatch_topk(logits, n, E, K, topk_ids, topk_probs, nullptr, rm, stream, n_live);
    // A capacity of N never binds (an expert gets at most one route per
    // token): the selection pass then only ranks each expert's routes in
    // token order and counts them.  Tokens past n_live have no picks in the map.
    launch_select(rm, n, E, K, n, route_within, route_counts, AlignOut{}, stream);
    st = launch_align_dropless(topk_ids, topk_probs, route_within, route_counts, N, E, K,
                               sorted_slot_ids, slot_probs, expert_ids, block_start, token_routes,
                               token_route_count, num_tokens_post_padded, stream, n_live);
    return st != MOE_OK ? st : launch_status();
}

}  // namespace
}  // namespace moe

extern "C" size_t moe_route_capacity_workspace_bytes(int64_t N, int32_t E, int32_t K) {
    if (N < 0 || E < 1 || K < 1 || K > E || N > moe::kMaxN || E > moe::kMaxE || K > moe::kMaxK)
        return 0;
    return moe::map_bytes(N, E);
}

extern "C" int moe_route_capacity(const float* logits, int64_t N, int32_t E, int32_t K, int64_t C,
                                  int32_t* topk_ids, float* topk_probs, int32_t* route_slot,
                                  int32_t* expert_count, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream) {
    using namespace moe;
    int st = check_route_shape(N, E, K, C);
    if (st != MOE_OK) return st;
    if (N == 0) return MOE_OK;
    st = check_route_ptrs({logits, topk_ids, topk_probs, route_slot, expert_count});
    if (st != MOE_OK) return st;
    st = check_workspace(workspace, workspace_bytes, N, E);
    if (st != MOE_OK) return st;
    route_capacity_launch(logits, static_cast<int>(N), E, K, static_cast<int>(C), topk_ids,
                          topk_probs, route_slot, expert_count, AlignOut{}, workspace, stream);
    return launch_status();
}

extern "C" int moe_route_capacity_align(const float* logits, int64_t N, int32_t E, int32_t K,
                                        int64_t C, int32_t* topk_ids, float* topk_probs,
                                        int32_t* route_slot, int32_t* expert_count,
                                        int32_t* sorted_slot_ids, float* slot_probs,
                                        int32_t* expert_ids, int32_t* block_start,
                                        int32_t* token_routes, int32_t* token_route_count,
                                        int32_t* num_tokens_post_padded, void* workspace,
                                        size_t workspace_bytes, hipStream_t stream) {
    using namespace moe;
    int st = check_route_shape(N, E, K, C);
    if (st != MOE_OK) return st;
    if (N == 0) return MOE_OK;
    st = check_route_ptrs({logits, topk_ids, topk_probs, route_slot, expert_count, sorted_slot_ids,
                           slot_probs, expert_ids, block_start, token_routes, token_route_count,
                           num_tokens_post_padded});
    if (st != MOE_OK) return st;
    st = check_workspace(workspace, workspace_bytes, N, E);
    if (st != MOE_OK) return st;
    const int n = static_cast<int>(N);
    const AlignOut ao{sorted_slot_ids, slot_probs, expert_ids, block_start, token_routes,
                      token_route_count, num_tokens_post_padded, n, K, E,
                      static_cast<int>(moe_padded_capacity(C))};
    route_capacity_launch(logits, n, E, K, static_cast<int>(C), topk_ids, topk_probs, route_slot,
                          expert_count, ao, workspace, stream);
    return launch_status();
}

extern "C" int moe_route_dropless(const float* logits, int64_t N, int32_t E, int32_t K,
                                  int32_t* topk_ids, float* topk_probs, int32_t* route_within,
                                  int32_t* route_counts, int32_t* sorted_slot_ids,
                                  float* slot_probs, int32_t* expert_ids, int32_t* block_start,
                                  int32_t* token_routes, int32_t* token_route_count,
                                  int32_t* num_tokens_post_padded, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
    return moe::route_dropless(logits, N, E, K, nullptr, topk_ids, topk_probs, route_within,
                               route_counts, sorted_slot_ids, slot_probs, expert_ids, block_start,
                               token_routes, token_route_count, num_tokens_post_padded, workspace,
                               workspace_bytes, stream);
}

extern "C" int moe_route_dropless_live(const float* logits, int64_t N, int32_t E, int32_t K,
                                       const int32_t* n_live, int32_t* topk_ids,
                                       float* topk_probs, int32_t* route_within,
                                       int32_t* route_counts, int32_t* sorted_slot_ids,
                                       float* slot_probs, int32_t* expert_ids,
                                       int32_t* block_start, int32_t* token_routes,
                                       int32_t* token_route_count,
                                       int32_t* num_tokens_post_padded, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream) {
    if (!n_live) return MOE_ERR_INVALID_ARG;
    if (!moe::aligned16(n_live)) return MOE_ERR_MISALIGNED;
    return moe::route_dropless(logits, N, E, K, n_live, topk_ids, topk_probs, route_within,
                               route_counts, sorted_slot_ids, slot_probs, expert_ids, block_start,
                               token_routes, token_route_count, num_tokens_post_padded, workspace,
                               workspace_bytes, stream);
}

// ---------------------------------------------------------------------------
// Allocation-free routing: moe_route_capacity_align with the routing map in a
// library-owned scratch array instead of a caller workspace, for callers that
// cannot allocate.  Each device holds its own copy of the array (until the
// process ends); host code reaches it only through the address
// hipGetSymbolAddress returns on that device, resolved on the first call made
// there and kept per device.  Every call on a device reuses the same array:
// each call overwrites the map rows it reads (nothing must start at zero),
// and calls that overlap on one device race.
// ---------------------------------------------------------------------------
namespace moe {
namespace {

constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// The scratch array's device address on the current device, or null.
void* scratch_on_current_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p) return p;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
    return p;
}

}  // namespace
}  // namespace moe

extern "C" int moe_route_capacity_align_noalloc(const float* logits, int64_t N, int32_t E, int32_t K,
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
    if (map_bytes(N, E) > kScratchBytes) return MOE_ERR_UNSUPPORTED;
    void* ws = scratch_on_current_device();
    if (!ws) return MOE_ERR_LAUNCH;
    return moe_route_capacity_align(logits, N, E, K, C, topk_ids, topk_probs, route_slot, expert_count,
                                    sorted_slot_ids, slot_probs, expert_ids, block_start, token_routes,
                                    token_route_count, num_tokens_post_padded, ws, kScratchBytes,
                                    stream);
}
