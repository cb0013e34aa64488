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

#include "moe_common.h"

namespace moe {
namespace {

// ---------------------------------------------------------------------------
// route_topk: one wavefront per token.  Each lane holds ceil(E/64) logits; K
// rounds of a wave-wide arg-max (ties -> lower expert) pick the experts in
// descending-logit order.  Lane k keeps round k's winner, then the K-way
// softmax runs in float64: exp(l_k - l_0), a sum in k order that every lane
// forms identically through shuffles, one division, one rounding to float32.
// ---------------------------------------------------------------------------
constexpr int kTopkWaves = 4;

template <int VPL>
__global__ __launch_bounds__(kTopkWaves * kWave) void route_topk_kernel(
    const float* __restrict__ logits, int N, int E, int K, int* __restrict__ topk_ids,
    float* __restrict__ topk_probs) {
    const int lane = lane_id();
    const int t = blockIdx.x * kTopkWaves + threadIdx.x / kWave;
    if (t >= N) return;
    const float* row = logits + static_cast<size_t>(t) * E;
    float v[VPL];
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
        const int e = j * kWave + lane;
        v[j] = e < E ? row[e] : 0.0f;
    }
    uint32_t taken = 0;
    float my_logit = 0.0f;
    int my_id = 0;
    for (int k = 0; k < K; ++k) {
        float bv = 0.0f;
        int bi = INT32_MAX;   // INT32_MAX = no candidate on this lane
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
            const int e = j * kWave + lane;
            const bool live = e < E && !((taken >> j) & 1u);
            if (live && (bi == INT32_MAX || v[j] > bv)) { bv = v[j]; bi = e; }
        }
#pragma unroll
        for (int off = kWave / 2; off >= 1; off >>= 1) {
            const float ov = __shfl_xor(bv, off, kWave);
            const int oi = __shfl_xor(bi, off, kWave);
            const bool better = oi != INT32_MAX &&
                                (bi == INT32_MAX || ov > bv || (ov == bv && oi < bi));
            if (better) { bv = ov; bi = oi; }
        }
        if ((bi & (kWave - 1)) == lane) taken |= 1u << (bi / kWave);
        if (lane == k) { my_logit = bv; my_id = bi; }
    }
    const double top = static_cast<double>(__shfl(my_logit, 0, kWave));
    const double ex = lane < K ? exp(static_cast<double>(my_logit) - top) : 0.0;
    double denom = 0.0;
    for (int k = 0; k < K; ++k) denom += __shfl(ex, k, kWave);
    if (lane < K) {
        topk_ids[static_cast<size_t>(t) * K + lane] = my_id;
        topk_probs[static_cast<size_t>(t) * K + lane] = static_cast<float>(ex / denom);
    }
}

// ---------------------------------------------------------------------------
// capacity_select: one 1024-thread workgroup per expert.
//  1. Compaction: scan topk_ids in route order (t*K + k, i.e. token order),
//     ballot-free per-thread masks over 16 routes + a block prefix scan, and
//     append this expert's candidates (route index, probability bits) to LDS.
//  2. If load > C: radix-select (4 x 8-bit digits, LDS histograms) the C-th
//     largest probability T and how many candidates equal to T still fit.
//     Probabilities are positive floats, so their bit patterns order like
//     their values.
//  3. Keep key > T, plus the first `need` candidates with key == T in token
//     order; a second block scan numbers the kept routes 0..count-1 in token
//     order.  Every route_slot entry of this expert gets exactly one write.
// ---------------------------------------------------------------------------
constexpr int kSelThreads = 1024;
constexpr int kSelChunk = 16;   // routes per thread per compaction pass

__global__ __launch_bounds__(kSelThreads) void capacity_select_kernel(
    const int* __restrict__ ids, const float* __restrict__ probs, int NK, int C,
    int* __restrict__ route_slot, int* __restrict__ expert_count) {
    __shared__ uint32_t s_route[kMaxN];
    __shared__ uint32_t s_key[kMaxN];
    __shared__ int s_scan[kSelThreads / kWave];
    __shared__ int s_hist[256];
    __shared__ uint32_t s_pick[2];
    const int e = blockIdx.x;
    const int tid = threadIdx.x;

    // 1. compaction
    int load = 0;
    for (int base = 0; base < NK; base += kSelThreads * kSelChunk) {
        const int start = base + tid * kSelChunk;
        uint32_t mask = 0;
        if (start + kSelChunk <= NK) {
            const int4* p = reinterpret_cast<const int4*>(ids + start);
#pragma unroll
            for (int q = 0; q < kSelChunk / 4; ++q) {
                const int4 v = p[q];
                mask |= (v.x == e ? 1u : 0u) << (4 * q + 0);
                mask |= (v.y == e ? 1u : 0u) << (4 * q + 1);
                mask |= (v.z == e ? 1u : 0u) << (4 * q + 2);
                mask |= (v.w == e ? 1u : 0u) << (4 * q + 3);
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
            const int r = start + j;
            if (pos < kMaxN) {   // a token feeds an expert at most once, so load <= N <= kMaxN
                s_route[pos] = static_cast<uint32_t>(r);
                s_key[pos] = __float_as_uint(probs[r]);
            }
            ++pos;
        }
        load += total;
    }
    load = min(load, static_cast<int>(kMaxN));
    __syncthreads();

    if (load <= C) {   // every candidate fits: slot = position in token order
        for (int i = tid; i < load; i += kSelThreads) route_slot[s_route[i]] = i;
        if (tid == 0) expert_count[e] = load;
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
        route_slot[s_route[i]] = keep ? slot++ : -1;
    }
    if (tid == 0) expert_count[e] = C;
}

template <int VPL>
void launch_topk(const float* logits, int N, int E, int K, int* ids, float* probs, hipStream_t s) {
    const int blocks = (N + kTopkWaves - 1) / kTopkWaves;
    route_topk_kernel<VPL><<<blocks, kTopkWaves * kWave, 0, s>>>(logits, N, E, K, ids, probs);
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
    if (!logits || !topk_ids || !topk_probs || !route_slot || !expert_count) return MOE_ERR_INVALID_ARG;
    if (!aligned16(logits) || !aligned16(topk_ids) || !aligned16(topk_probs) ||
        !aligned16(route_slot) || !aligned16(expert_count))
        return MOE_ERR_MISALIGNED;
    const int n = static_cast<int>(N);
    const int vpl = (E + kWave - 1) / kWave;
    if (vpl <= 1) launch_topk<1>(logits, n, E, K, topk_ids, topk_probs, stream);
    else if (vpl <= 2) launch_topk<2>(logits, n, E, K, topk_ids, topk_probs, stream);
    else if (vpl <= 4) launch_topk<4>(logits, n, E, K, topk_ids, topk_probs, stream);
    else if (vpl <= 8) launch_topk<8>(logits, n, E, K, topk_ids, topk_probs, stream);
    else launch_topk<16>(logits, n, E, K, topk_ids, topk_probs, stream);
    capacity_select_kernel<<<E, kSelThreads, 0, stream>>>(topk_ids, topk_probs, n * K,
                                                          static_cast<int>(C), route_slot,
                                                          expert_count);
    return launch_status();
}
