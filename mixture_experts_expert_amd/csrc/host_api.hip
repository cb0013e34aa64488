#include <algorithm>
// Host-only entry points of libmoe_native: capacity arithmetic, status strings
// and the shape checks shared by the device entry points.
#include <cmath>
#include <cstdint>

#include "moe_common.h"

namespace moe {

int check_route_shape(int64_t N, int32_t E, int32_t K, int64_t C) {
    if (N < 0 || E < 1 || K < 1 || K > E || C < 0) return MOE_ERR_INVALID_ARG;
    if (N > kMaxN || E > kMaxE || K > kMaxK) return MOE_ERR_UNSUPPORTED;
    const int64_t Cp = moe_padded_capacity(C);
    if (Cp < 0 || static_cast<int64_t>(E) * Cp > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

int check_dims(int32_t H, int32_t I) {
    if (H < 1 || I < 1) return MOE_ERR_INVALID_ARG;
    if (H % 64 || I % 64 || H > kMaxDim || I > kMaxDim) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

}  // namespace moe

extern "C" {

const char* moe_status_string(int status) {
    switch (status) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
        case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
        case MOE_ERR_MISALIGNED: return "MOE_ERR_MISALIGNED";
        case MOE_ERR_LAUNCH: return "MOE_ERR_LAUNCH";
        default: return "MOE_ERR_UNKNOWN";
    }
}

// C = ceil(N*K*F/E) with F = mant * 2^s exactly (mant a 53-bit integer):
// C = ceil(N*K*mant * 2^s / E), all in unsigned 128-bit integers.  For s < 0
// the nested-ceiling identity ceil(a/(b*c)) = ceil(ceil(a/b)/c) keeps every
// intermediate in range.
int64_t moe_source_capacity(int64_t N, int32_t K, int32_t E, double F) {
    if (N < 0 || K < 1 || E < 1 || K > E) return MOE_ERR_INVALID_ARG;
    if (!std::isfinite(F) || !(F > 0.0)) return MOE_ERR_INVALID_ARG;
    if (N == 0) return 0;
    if (N > (int64_t(1) << 40)) return MOE_ERR_UNSUPPORTED;
    int ex = 0;
    const double m = std::frexp(F, &ex);                 // F = m * 2^ex, m in [0.5, 1)
    const uint64_t mant = static_cast<uint64_t>(std::ldexp(m, 53));   // exact
    const int s = ex - 53;                               // F = mant * 2^s
    typedef unsigned __int128 u128;
    const u128 num = static_cast<u128>(static_cast<uint64_t>(N)) * static_cast<uint64_t>(K) * mant;  // < 2^124
    u128 a;
    if (s >= 0) {
        if (s >= 127 || (num >> (127 - s)) != 0) return MOE_ERR_UNSUPPORTED;
        a = num << s;
    } else {
        const int t = -s;
        a = (t >= 127) ? u128(1) : ((num + ((u128(1) << t) - 1)) >> t);   // ceil(num / 2^t), num > 0
    }
    const u128 c = (a + static_cast<u128>(E) - 1) / static_cast<u128>(E);
    if (c > static_cast<u128>(INT32_MAX)) return MOE_ERR_UNSUPPORTED;
    return static_cast<int64_t>(c);
}

int32_t moe_layout_block_m(void) { return moe::kBlockM; }

int64_t moe_padded_capacity(int64_t C) {
    if (C < 0) return MOE_ERR_INVALID_ARG;
    if (C > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    return (C + moe::kBlockM - 1) / moe::kBlockM * moe::kBlockM;
}

int64_t moe_dropless_bound(int64_t N, int32_t K, int32_t E) {
    if (N < 0 || E < 1 || K < 1 || K > E) return MOE_ERR_INVALID_ARG;
    if (N > moe::kMaxN || E > moe::kMaxE || K > moe::kMaxK) return MOE_ERR_UNSUPPORTED;
    const int64_t r = N * std::min(K, E) + static_cast<int64_t>(E) * (moe::kBlockM - 1);
    return (r + moe::kBlockM - 1) / moe::kBlockM * moe::kBlockM;
}

}  // extern "C"
