// Probes of a compute unit's matrix cores and LDS read path (measurement
// instruments, not steps of the layer): one 512-thread workgroup per compute
// unit (a static LDS allocation above half the 160 KB keeps a second one
// off), issuing nothing but bf16 32x32x16 MFMAs on four independent
// accumulators per wave, or nothing but 16-byte LDS reads, eight in flight
// per wave.  Each workgroup records its engine-clock ticks (s_memtime) and
// its 100 MHz constant-clock ticks (s_memrealtime) over the loop, so the rate
// comes with the clock the chip ran it at.
#include "../../include/moe_probe.h"
#include "gemm_common.h"

namespace moe {
namespace {

// One workgroup per compute unit: 96 KB of static LDS (more than half of
// the 160 KB) leaves no room for a second.
constexpr int kHoldFloats = 96 * 1024 / 4;

// The workgroup's clocks over its loop: engine-clock ticks, constant-clock
// ticks (one word each), written by one lane.
__device__ __forceinline__ void put_clocks(uint64_t* clocks, uint64_t c, uint64_t r) {
    if (threadIdx.x == 0) {
        clocks[2 * blockIdx.x] = c;
        clocks[2 * blockIdx.x + 1] = r;
    }
}

__global__ __launch_bounds__(8 * kWave) void probe_mfma_rate_kernel(int iters, uint64_t* clocks) {
    __shared__ float hold[kHoldFloats];
    if (threadIdx.x < 8) hold[threadIdx.x] = 0.0f;
    __syncthreads();
    const float z = hold[threadIdx.x & 7];   // 0; read back so the allocation stays
    bf16x8 x, y;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        x[j] = static_cast<__bf16>(z + 0.001f * static_cast<float>((threadIdx.x + j) & 15));
        y[j] = static_cast<__bf16>(z + 0.002f * static_cast<float>(j));
    }
    floatx16 a0 = {}, a1 = {}, a2 = {}, a3 = {};
    __syncthreads();
    const uint64_t c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
        a0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, a0, 0, 0, 0);
        a1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, a1, 0, 0, 0);
        a2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, a2, 0, 0, 0);
        a3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, a3, 0, 0, 0);
    }
    __syncthreads();
    const uint64_t c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
    put_clocks(clocks, c1 - c0, r1 - r0);
    const float f = a0[0] + a1[5] + a2[10] + a3[15];
    if (f == 1.2345e-30f) clocks[2 * blockIdx.x] = 0;   // keeps the MFMAs live
}

__global__ __launch_bounds__(8 * kWave) void probe_lds_read_kernel(int iters, uint64_t* clocks) {
    __shared__ __attribute__((aligned(16))) float hold[kHoldFloats];
    u32x4* blocks = reinterpret_cast<u32x4*>(hold);       // the first 64 KB: 64 blocks of 1 KB
    for (int i = threadIdx.x; i < 4096; i += 8 * kWave) blocks[i] = u32x4{uint32_t(i), 1u, 2u, 3u};
    __syncthreads();
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const uint64_t c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
        // eight 1 KB blocks per wave (lane-contiguous, no bank conflicts), all
        // in flight, then one use that keeps them and does no ALU work
        u32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = blocks[((wave * 8 + u + it) & 63) * kWave + lane];
        asm volatile("" :: "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]), "v"(v[6]), "v"(v[7]));
    }
    __syncthreads();
    const uint64_t c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
    put_clocks(clocks, c1 - c0, r1 - r0);
}

}  // namespace
}  // namespace moe

// groups workgroups of 512 threads (one per compute unit at most), each
// running `iters` loop trips; clocks[2*g], clocks[2*g+1] = workgroup g's
// engine-clock and constant-clock ticks.
extern "C" int moe_probe_mfma_rate(int32_t groups, int32_t iters, uint64_t* clocks, hipStream_t stream) {
    using namespace moe;
    if (!clocks || groups < 0 || iters < 1) return MOE_ERR_INVALID_ARG;
    if (groups == 0) return MOE_OK;
    probe_mfma_rate_kernel<<<groups, 8 * kWave, 0, stream>>>(iters, clocks);
    return launch_status();
}

extern "C" int moe_probe_lds_read(int32_t groups, int32_t iters, uint64_t* clocks, hipStream_t stream) {
    using namespace moe;
    if (!clocks || groups < 0 || iters < 1) return MOE_ERR_INVALID_ARG;
    if (groups == 0) return MOE_OK;
    probe_lds_read_kernel<<<groups, 8 * kWave, 0, stream>>>(iters, clocks);
    return launch_status();
}
