// Step 5 of the MoE FFN forward: the contention-free gather-combine.
//
// [PF] "Permute-Free Grouped GEMM for MoE (bf16, gfx950)", section 2 and
// section 5 (route_gather_combine): each output token pulls its own routes
// from the route-ordered FC2 output, so every output row has exactly one
// writer and no atomic scatter (or its scratch) exists.
//
// Work item = one 16-byte chunk (8 bf16 columns) of one token row.  A thread
// reads the token's K route indices (the same few cache lines for all of the
// row's threads), issues all K row loads before summing, adds them in float32
// in k order starting from +0.0, and stores 16 bytes of y.  HBM-bound: the
// route rows are read once, y is written once.
#include "moe_common.h"

namespace moe {
namespace {

template <int KMAX>
__global__ __launch_bounds__(256) void gather_combine_kernel(
    const uint16_t* __restrict__ route_out, const int* __restrict__ token_routes, int N, int K,
    int H, int R, uint16_t* __restrict__ y) {
    const int chunks = H / 8;
    const int64_t item = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (item >= static_cast<int64_t>(N) * chunks) return;
    const int t = static_cast<int>(item / chunks);
    const int c = static_cast<int>(item - static_cast<int64_t>(t) * chunks);
    int r[KMAX];
    uint4 v[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        r[k] = k < K ? token_routes[static_cast<int64_t>(t) * K + k] : -1;
        if (r[k] >= R) r[k] = -1;   // device data is range-checked, never trusted
        v[k] = make_uint4(0, 0, 0, 0);
        if (r[k] >= 0)
            v[k] = *reinterpret_cast<const uint4*>(route_out + static_cast<int64_t>(r[k]) * H + c * 8);
    }
    float acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        if (r[k] < 0) continue;
        const uint32_t w[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            acc[2 * j] += __uint_as_float(w[j] << 16);
            acc[2 * j + 1] += __uint_as_float(w[j] & 0xFFFF0000u);
        }
    }
    uint4 o;
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
    o.z = pack_bf16x2(acc[4], acc[5]);
    o.w = pack_bf16x2(acc[6], acc[7]);
    *reinterpret_cast<uint4*>(y + static_cast<int64_t>(t) * H + c * 8) = o;
}

// Dispatch side of an expert-parallel exchange: the send buffer holds each
// slot's token row in route order, rows[s] = x[sorted_slot_ids[s]], with a
// zero row for the sentinel (pads) -- the rows a uniform all-to-all moves,
// C per expert from every source.  Work item = one 16-byte chunk of one
// slot row; HBM-bound (the kept rows read, every slot row written once).
__global__ __launch_bounds__(256) void dispatch_rows_kernel(
    const uint16_t* __restrict__ x, const int* __restrict__ sorted_slot_ids, int N, int H, int R,
    uint16_t* __restrict__ rows) {
    const int chunks = H / 8;
    const int64_t item = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (item >= static_cast<int64_t>(R) * chunks) return;
    const int s = static_cast<int>(item / chunks);
    const int c = static_cast<int>(item - static_cast<int64_t>(s) * chunks);
    const int tok = sorted_slot_ids[s];
    uint4 v = make_uint4(0, 0, 0, 0);
    if (static_cast<unsigned>(tok) < static_cast<unsigned>(N))   // device data: range-checked
        v = *reinterpret_cast<const uint4*>(x + static_cast<int64_t>(tok) * H + c * 8);
    *reinterpret_cast<uint4*>(rows + static_cast<int64_t>(s) * H + c * 8) = v;
}

template <int KMAX>
void launch_combine(const uint16_t* ro, const int* tr, int N, int K, int H, int R, uint16_t* y,
                    hipStream_t s) {
    const int64_t items = static_cast<int64_t>(N) * (H / 8);
    const int blocks = static_cast<int>((items + 255) / 256);
    gather_combine_kernel<KMAX><<<blocks, 256, 0, s>>>(ro, tr, N, K, H, R, y);
}

}  // namespace
}  // namespace moe

extern "C" int moe_gather_combine(const uint16_t* route_out, const int32_t* token_routes, int64_t N,
                                  int32_t K, int32_t H, int64_t R, uint16_t* y, hipStream_t stream) {
    using namespace moe;
    if (N < 0 || K < 1 || H < 1 || R < 0) return MOE_ERR_INVALID_ARG;
    if (N > kMaxN || K > kMaxK || H % 64 || H > kMaxDim || R > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    if (N == 0) return MOE_OK;
    if (!route_out || !token_routes || !y) return MOE_ERR_INVALID_ARG;
    if (!aligned16(route_out) || !aligned16(token_routes) || !aligned16(y)) return MOE_ERR_MISALIGNED;
    const int n = static_cast<int>(N), r = static_cast<int>(R);
    if (K <= 2) launch_combine<2>(route_out, token_routes, n, K, H, r, y, stream);
    else if (K <= 4) launch_combine<4>(route_out, token_routes, n, K, H, r, y, stream);
    else if (K <= 8) launch_combine<8>(route_out, token_routes, n, K, H, r, y, stream);
    else if (K <= 16) launch_combine<16>(route_out, token_routes, n, K, H, r, y, stream);
    else launch_combine<32>(route_out, token_routes, n, K, H, r, y, stream);
    return launch_status();
}

extern "C" int moe_dispatch_rows(const uint16_t* x, const int32_t* sorted_slot_ids, int64_t N,
                                 int32_t H, int64_t R, uint16_t* rows, hipStream_t stream) {
    using namespace moe;
    if (N < 0 || H < 1 || R < 0) return MOE_ERR_INVALID_ARG;
    if (N > INT32_MAX || H % 64 || H > kMaxDim || R > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    if (R == 0) return MOE_OK;
    if (!x || !sorted_slot_ids || !rows) return MOE_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(sorted_slot_ids) || !aligned16(rows)) return MOE_ERR_MISALIGNED;
    const int64_t items = R * (H / 8);
    const int64_t blocks = (items + 255) / 256;
    if (blocks > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    dispatch_rows_kernel<<<static_cast<int>(blocks), 256, 0, stream>>>(
        x, sorted_slot_ids, static_cast<int>(N), H, static_cast<int>(R), rows);
    return launch_status();
}
