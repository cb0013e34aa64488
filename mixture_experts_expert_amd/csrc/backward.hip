// Backward of the MoE FFN layer: the gated-activation recompute + backward
// and the router-logit gradient.
//
// [PF] "Permute-Free Grouped GEMM for MoE (bf16, gfx950)", section 6: only
// the 2I pre-activation [gate | up] persists across the forward/backward
// boundary; the backward re-materialises act = silu(gate) * up * prob from it
// (the F-wide transient the FC2 weight gradient consumes) and computes the
// gradient with respect to the pre-activation and the route probability in
// the same pass.  The probability gradient then flows through the softmax
// over each token's top K to the router logits.
//
// Both kernels are HBM-bound elementwise passes; they read each input once
// with 16-byte loads and write each output once.
#include "gemm_common.h"

namespace moe {
namespace {

typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

// One wave per slot row s: lanes stride the I columns 8 at a time.
//   act    = silu(g) * u * p
//   d_gate = d_act * p * u * s * (1 + g * (1 - s)),  s = sigmoid(g)
//   d_up   = d_act * p * silu(g)
//   d_prob = sum over the row of d_act * silu(g) * u     (wave reduction)
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const uint16_t* __restrict__ preact,
                                                         const uint16_t* __restrict__ d_act,
                                                         const float* __restrict__ probs, int R,
                                                         int I, uint16_t* __restrict__ act,
                                                         uint16_t* __restrict__ d_pre,
                                                         float* __restrict__ d_prob) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t s = static_cast<int64_t>(blockIdx.x) * (blockDim.x / kWave) + threadIdx.x / kWave;
    if (s >= R) return;
    const float p = probs[s];
    const uint16_t* hg = preact + s * 2 * I;
    const uint16_t* hu = hg + I;
    const uint16_t* da = d_act + s * I;
    float dp = 0.0f;
    for (int c = lane * 8; c < I; c += kWave * 8) {
        const u16x8 g8 = *reinterpret_cast<const u16x8*>(hg + c);
        const u16x8 u8 = *reinterpret_cast<const u16x8*>(hu + c);
        const u16x8 d8 = *reinterpret_cast<const u16x8*>(da + c);
        u16x8 a8, dg8, du8;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float g = bf16_to_f32(g8[j]), u = bf16_to_f32(u8[j]), d = bf16_to_f32(d8[j]);
            const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-g * 1.4426950408889634f));
            const float sl = g * sg;
            a8[j] = f32_to_bf16(sl * u * p);
            dg8[j] = f32_to_bf16(d * p * u * (sg * (1.0f + g * (1.0f - sg))));
            du8[j] = f32_to_bf16(d * p * sl);
            dp += d * sl * u;
        }
        *reinterpret_cast<u16x8*>(act + s * I + c) = a8;
        *reinterpret_cast<u16x8*>(d_pre + s * 2 * I + c) = dg8;
        *reinterpret_cast<u16x8*>(d_pre + s * 2 * I + I + c) = du8;
    }
#pragma unroll
    for (int o = kWave / 2; o >= 1; o >>= 1) dp += __shfl_xor(dp, o);
    if (lane == 0) d_prob[s] = dp;
}

// One wave per token t.  Lane k < K holds route (t, k): dp_k = d_prob of its
// slot (0 if the route was dropped); g_k = p_k * (dp_k - sum_j p_j dp_j).
// The token's E-wide logit-gradient row is written whole: g_k at column
// ids[t, k], 0 elsewhere.
__global__ __launch_bounds__(256) void route_bwd_kernel(const int32_t* __restrict__ ids,
                                                        const float* __restrict__ probs,
                                                        const int32_t* __restrict__ token_routes,
                                                        const float* __restrict__ d_prob, int N,
                                                        int E, int K, int R,
                                                        float* __restrict__ d_logits) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t t = static_cast<int64_t>(blockIdx.x) * (blockDim.x / kWave) + threadIdx.x / kWave;
    if (t >= N) return;
    float pk = 0.0f, dpk = 0.0f;
    int idk = -1;
    if (lane < K) {
        pk = probs[t * K + lane];
        idk = ids[t * K + lane];
        const int r = token_routes[t * K + lane];
        dpk = r >= 0 && r < R ? d_prob[r] : 0.0f;
    }
    float inner = pk * dpk;
#pragma unroll
    for (int o = kWave / 2; o >= 1; o >>= 1) inner += __shfl_xor(inner, o);
    const float gk = pk * (dpk - inner);
    for (int c = lane; c < E; c += kWave) {
        float v = 0.0f;
        for (int k = 0; k < K; ++k) {
            const int id = __shfl(idk, k);
            const float g = __shfl(gk, k);
            v = id == c ? g : v;
        }
        d_logits[t * E + c] = v;
    }
}

}  // namespace
}  // namespace moe

extern "C" int moe_swiglu_bwd(const uint16_t* preact, const uint16_t* d_act,
                              const float* slot_probs, int64_t R, int32_t I, uint16_t* act,
                              uint16_t* d_preact, float* d_prob, hipStream_t stream) {
    using namespace moe;
    if (R < 0 || I < 1) return MOE_ERR_INVALID_ARG;
    if (I % 64 || I > kMaxDim || R > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    if (R == 0) return MOE_OK;
    for (const void* q : {static_cast<const void*>(preact), static_cast<const void*>(d_act),
                          static_cast<const void*>(slot_probs), static_cast<const void*>(act),
                          static_cast<const void*>(d_preact), static_cast<const void*>(d_prob)}) {
        if (!q) return MOE_ERR_INVALID_ARG;
        if (!aligned16(q)) return MOE_ERR_MISALIGNED;
    }
    const int64_t blocks = (R + 3) / 4;
    swiglu_bwd_kernel<<<static_cast<unsigned>(blocks), 256, 0, stream>>>(
        preact, d_act, slot_probs, static_cast<int>(R), I, act, d_preact, d_prob);
    return launch_status();
}

extern "C" int moe_route_bwd(const int32_t* topk_ids, const float* topk_probs,
                             const int32_t* token_routes, const float* d_prob, int64_t N,
                             int32_t E, int32_t K, int64_t R, float* d_logits,
                             hipStream_t stream) {
    using namespace moe;
    if (N < 0 || E < 1 || K < 1 || K > E || R < 0) return MOE_ERR_INVALID_ARG;
    if (N > kMaxN || E > kMaxE || K > kMaxK || R > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    if (N == 0) return MOE_OK;
    for (const void* q : {static_cast<const void*>(topk_ids), static_cast<const void*>(topk_probs),
                          static_cast<const void*>(token_routes), static_cast<const void*>(d_prob),
                          static_cast<const void*>(d_logits)}) {
        if (!q) return MOE_ERR_INVALID_ARG;
        if (!aligned16(q)) return MOE_ERR_MISALIGNED;
    }
    route_bwd_kernel<<<static_cast<unsigned>((N + 3) / 4), 256, 0, stream>>>(
        topk_ids, topk_probs, token_routes, d_prob, static_cast<int>(N), E, K,
        static_cast<int>(R), d_logits);
    return launch_status();
}
