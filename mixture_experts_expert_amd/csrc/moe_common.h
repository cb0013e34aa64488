// Internal helpers shared by the HIP sources of libmoe_native (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe_native.h"

namespace moe {

constexpr int kWave = 64;          // CDNA wavefront width
constexpr int kBlockM = 32;        // route-list layout block (BM)
constexpr int64_t kMaxN = 16384;   // tokens per call (capacity selection holds an expert's candidates in LDS)
constexpr int kMaxE = 1024;
constexpr int kMaxK = 32;
constexpr int kMaxDim = 16384;     // H and I

// ---------------------------------------------------------------- host-side checks

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int launch_status() {
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

// Shape checks shared by the entry points; C must equal moe_source_capacity's value.
int check_route_shape(int64_t N, int32_t E, int32_t K, int64_t C);
int check_dims(int32_t H, int32_t I);

// ---------------------------------------------------------------- device helpers

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float32 -> bf16, round to nearest even: gfx950's v_cvt_pk_bf16_f32 (one
// instruction per pair, where the integer rounding takes six).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    const f32x2_t f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Inclusive prefix sum across the 64 lanes of a wave, in DPP lane moves (no
// LDS round trip): shifts by 1, 2, 4 and 8 lanes inside each 16-lane row,
// then lane 15's row total broadcast into rows 1 and 3 and lane 31's into
// rows 2 and 3.  A lane whose source is outside its row adds 0.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);   // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);   // row_bcast:15
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);   // row_bcast:31
    return v;
}

// Exclusive prefix sum over a whole block (blockDim.x a multiple of 64, at
// most 1024 threads).  `scratch` must hold 16 ints in LDS; returns this
// thread's exclusive prefix and writes the block total to *total.
__device__ __forceinline__ int block_exclusive_scan(int v, int* scratch, int* total) {
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    const int nwaves = blockDim.x / kWave;
    int inc = wave_inclusive_scan(v);
    if (lane == kWave - 1) scratch[wave] = inc;
    __syncthreads();
    int base = 0, tot = 0;
    for (int w = 0; w < nwaves; ++w) {
        int c = scratch[w];
        if (w < wave) base += c;
        tot += c;
    }
    __syncthreads();   // scratch may be reused right after
    *total = tot;
    return base + inc - v;
}

// Dropless align launch (align.hip), shared with the routing entry point.
int launch_align_dropless(const int32_t* topk_ids, const float* topk_probs,
                          const int32_t* route_within, const int32_t* route_counts, int64_t N,
                          int32_t E, int32_t K, int32_t* sorted_slot_ids, float* slot_probs,
                          int32_t* expert_ids, int32_t* block_start, int32_t* token_routes,
                          int32_t* token_route_count, int32_t* num_tokens_post_padded,
                          hipStream_t stream, const int32_t* n_live = nullptr);

}  // namespace moe
