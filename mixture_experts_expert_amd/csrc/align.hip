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

}  // namespace
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
