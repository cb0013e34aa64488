// Step 3 of the MoE FFN forward: the sync-free align pass.
//
// [PF] "Permute-Free Grouped GEMM for MoE (bf16, gfx950)", section 4 (Data
// structures) and section 5 (route_list_align): an expert-sorted,
// block-padded route list (slot -> token row, sentinel N for padding), the
// owning expert of each block, each expert's first block, the token -> slots
// inverse map and the padded extent as a device scalar.
// [FC] "feat(cuda-graphs): capture fixed-capacity MoE execution", Design
// notes: with fixed capacity every expert owns exactly Cp slots, so the
// layout is static and only its contents depend on the routing.
//
// One flat grid, one writer per output element, no atomics:
//   thread i < E*Cp    slot role  : pad slots (j >= expert_count[e]) get (N, +0.0)
//   thread i < N*K     route role : a kept route writes its slot's (t, p) and
//                                   token_routes; a dropped one writes -1
//   thread i < N       token role : token_route_count
//   thread i < E*Cp/BM block role : expert_ids
//   thread i < E       expert role: block_start; thread 0 also the extent
// Kept routes of expert e occupy slots 0..expert_count[e]-1 exactly, so the
// slot and route roles never write the same element.
#include <algorithm>

#include "moe_common.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void align_kernel(
    const int* __restrict__ topk_ids, const float* __restrict__ topk_probs,
    const int* __restrict__ route_slot, const int* __restrict__ expert_count, int N, int E, int K,
    int Cp, int* __restrict__ sorted_slot_ids, float* __restrict__ slot_probs,
    int* __restrict__ expert_ids, int* __restrict__ block_start, int* __restrict__ token_routes,
    int* __restrict__ token_route_count, int* __restrict__ num_tokens_post_padded) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    const int R = E * Cp;
    if (i < R) {
        const int e = i / Cp, j = i - e * Cp;
        if (j >= expert_count[e]) {
            sorted_slot_ids[i] = N;
            slot_probs[i] = 0.0f;
        }
    }
    if (i < N * K) {
        const int j = route_slot[i];
        const int e = topk_ids[i];
        int s = -1;
        if (j >= 0 && j < Cp && e >= 0 && e < E) {   // device data is range-checked, never trusted
            s = e * Cp + j;
            sorted_slot_ids[s] = i / K;
            slot_probs[s] = topk_probs[i];
        }
        token_routes[i] = s;
    }
    if (i < N) {
        int c = 0;
        for (int k = 0; k < K; ++k) c += route_slot[i * K + k] >= 0;
        token_route_count[i] = c;
    }
    if (i < R / kBlockM) expert_ids[i] = i * kBlockM / Cp;
    if (i < E) block_start[i] = i * Cp / kBlockM;
    if (i == 0) num_tokens_post_padded[0] = R;
}

// Dropless form ([PF] sections 4-5): every route is kept, expert e's
// count_e routes fill its segment in token order (their within-expert ranks
// from the selection pass), segments are padded to BM and follow each other
// in expert order.  Each workgroup first forms the exclusive prefix of the
// padded counts in LDS (E <= 1024), then, one writer per element:
//   thread i < N*K     route role : slot s = start[e] + rank -> (t, p), token_routes
//   thread i < R       slot role  : slots past the real extent -> (N, +0.0)
//   thread i < R/BM    block role : owning expert (binary search), -1 past the extent
//   thread i < E       expert role: block_start, and its segment's pad slots
//   thread i < N       token role : token_route_count = K
//   thread 0                      : the extent
constexpr int kDlThreads = 256;

__global__ __launch_bounds__(kDlThreads) void align_dropless_kernel(
    const int* __restrict__ topk_ids, const float* __restrict__ topk_probs,
    const int* __restrict__ route_within, const int* __restrict__ route_counts, int N, int E, int K,
    int R, int* __restrict__ sorted_slot_ids, float* __restrict__ slot_probs,
    int* __restrict__ expert_ids, int* __restrict__ block_start, int* __restrict__ token_routes,
    int* __restrict__ token_route_count, int* __restrict__ num_tokens_post_padded,
    const int* __restrict__ n_live) {
    __shared__ int s_start[kMaxE + 1];   // exclusive prefix of padded counts, s_start[E] = extent
    __shared__ int s_scan[kDlThreads / kWave];
    constexpr int PER = (kMaxE + kDlThreads - 1) / kDlThreads;
    const int tid = threadIdx.x;
    int padded[PER], own = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int e = tid * PER + j;
        const int c = e < E ? route_counts[e] : 0;
        padded[j] = (max(c, 0) + kBlockM - 1) / kBlockM * kBlockM;
        own += padded[j];
    }
    int total = 0;
    int run = block_exclusive_scan(own, s_scan, &total);
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int e = tid * PER + j;
        if (e < E) s_start[e] = run;
        run += padded[j];
    }
    if (tid == 0) s_start[E] = total;
    __syncthreads();
    const int extent = min(total, R);   // counts from this call never exceed the bound

    const int i = blockIdx.x * blockDim.x + tid;
    if (i < N * K) {
        const int e = topk_ids[i];
        const int j = route_within[i];
        int s = -1;
        if (e >= 0 && e < E && j >= 0 && s_start[e] + j < min(s_start[e + 1], extent)) {
            s = s_start[e] + j;
            sorted_slot_ids[s] = i / K;
            slot_probs[s] = topk_probs[i];
        }
        token_routes[i] = s;
    }
    if (i >= extent && i < R) {
        sorted_slot_ids[i] = N;
        slot_probs[i] = 0.0f;
    }
    if (i < R / kBlockM) {
        int owner = -1;
        if (i * kBlockM < extent) {   // last expert whose segment starts at or before this block
            int lo = 0, hi = E - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) / 2;
                if (s_start[mid] <= i * kBlockM) lo = mid; else hi = mid - 1;
            }
            owner = lo;
        }
        expert_ids[i] = owner;
    }
    if (i < E) {
        block_start[i] = s_start[i] / kBlockM;
        const int c = min(max(route_counts[i], 0), s_start[i + 1] - s_start[i]);
        for (int s = s_start[i] + c; s < min(s_start[i + 1], extent); ++s) {
            sorted_slot_ids[s] = N;
            slot_probs[s] = 0.0f;
        }
    }
    // tokens at or past n_live (when given) routed nowhere
    if (i < N) token_route_count[i] = n_live && i >= min(max(n_live[0], 0), N) ? 0 : K;
    if (i == 0) num_tokens_post_padded[0] = extent;
}

}  // namespace
}  // namespace moe

namespace moe {

int launch_align_dropless(const int32_t* topk_ids, const float* topk_probs,
                          const int32_t* route_within, const int32_t* route_counts, int64_t N,
                          int32_t E, int32_t K, int32_t* sorted_slot_ids, float* slot_probs,
                          int32_t* expert_ids, int32_t* block_start, int32_t* token_routes,
                          int32_t* token_route_count, int32_t* num_tokens_post_padded,
                          hipStream_t stream, const int32_t* n_live) {
    const int64_t R = moe_dropless_bound(N, K, E);
    if (R < 0) return static_cast<int>(R);
    const int64_t work = std::max<int64_t>(R, N * K);
    const int blocks = static_cast<int>((work + kDlThreads - 1) / kDlThreads);
    align_dropless_kernel<<<blocks, kDlThreads, 0, stream>>>(
        topk_ids, topk_probs, route_within, route_counts, static_cast<int>(N), E, K,
        static_cast<int>(R), sorted_slot_ids, slot_probs, expert_ids, block_start, token_routes,
        token_route_count, num_tokens_post_padded, n_live);
    return MOE_OK;
}

}  // namespace moe

extern "C" int moe_align(const int32_t* topk_ids, const float* topk_probs, const int32_t* route_slot,
                         const int32_t* expert_count, int64_t N, int32_t E, int32_t K, int64_t C,
                         int32_t* sorted_slot_ids, float* slot_probs, int32_t* expert_ids,
                         int32_t* block_start, int32_t* token_routes, int32_t* token_route_count,
                         int32_t* num_tokens_post_padded, hipStream_t stream) {
    using namespace moe;
    int st = check_route_shape(N, E, K, C);
    if (st != MOE_OK) return st;
    if (N == 0) return MOE_OK;
    const void* ptrs[] = {topk_ids, topk_probs, route_slot, expert_count, sorted_slot_ids,
                          slot_probs, expert_ids, block_start, token_routes, token_route_count,
                          num_tokens_post_padded};
    for (const void* p : ptrs) {
        if (!p) return MOE_ERR_INVALID_ARG;
        if (!aligned16(p)) return MOE_ERR_MISALIGNED;
    }
    const int Cp = static_cast<int>(moe_padded_capacity(C));
    const int64_t work = std::max<int64_t>(static_cast<int64_t>(E) * Cp, N * K);
    const int blocks = static_cast<int>((work + 255) / 256);
    align_kernel<<<blocks, 256, 0, stream>>>(topk_ids, topk_probs, route_slot, expert_count,
                                             static_cast<int>(N), E, K, Cp, sorted_slot_ids,
                                             slot_probs, expert_ids, block_start, token_routes,
                                             token_route_count, num_tokens_post_padded);
    return launch_status();
}
