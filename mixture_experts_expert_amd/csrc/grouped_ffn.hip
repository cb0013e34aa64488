// Step 4 of the MoE FFN forward: permute-free grouped FC1 -> SwiGLU*prob -> FC2.
//
// [PF] "Permute-Free Grouped GEMM for MoE (bf16, gfx950)":
//   section 2  the activations stay in token order; the FC1 A-tile loads read
//              x[sorted_slot_ids[slot]] directly, so no permuted copy exists;
//   section 3  one align drives both FCs: FC1 gathers A through the route list,
//              FC2 reads its A (the activation) by route position;
//   section 6  the gated activation act(gate)*up*prob feeds FC2 directly.
// [FC] "feat(cuda-graphs): capture fixed-capacity MoE execution", Design
//   notes: every expert owns exactly Cp rows, so the GEMM geometry is fixed
//   by the shapes alone.
//
// gfx950 design (not the pages' FlyDSL kernel):
//   * one workgroup per (expert, M-tile, N-tile); the M-tile spans up to 256
//     slots so an expert's weight panel is streamed from HBM once;
//   * bf16 MFMA 32x32x16 with float32 accumulators;
//   * operands are K-contiguous on both sides (x rows, weight rows), staged
//     through LDS in 64-wide K slabs with an XOR swizzle of the 16-byte
//     chunks so the MFMA operand reads are bank-conflict free;
//   * buffer loads with a per-expert descriptor: the sentinel row N (and any
//     row past an expert's segment) lies outside the descriptor and reads as
//     zeros, which is how pad slots enter the GEMM;
//   * the FC1 tile holds matching gate and up columns, so the SwiGLU and the
//     routing probability are applied to the accumulators in registers and
//     only the I-wide bf16 activation is written;
//   * tiles are renumbered so that consecutive tiles (same expert, adjacent
//     N-tiles, sharing the gathered A rows) land on the same XCD and its L2.
#include <algorithm>
#include <initializer_list>

#include "moe_common.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBK = 64;          // K slab (bf16 elements) per LDS stage: 128 bytes per row
constexpr int kXcds = 8;         // MI355X: 8 XCDs, workgroups dealt round-robin
constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit data format (CDNA)

struct FfnArgs {
    const uint16_t* a;            // FC1: x [N, H];   FC2: act [E*Cp, I]
    const uint16_t* w;            // FC1: w1 [E, 2I, H]; FC2: w2 [E, H, I]
    const int* sorted_slot_ids;   // FC1 only
    const float* slot_probs;      // FC1 only
    uint16_t* out;                // FC1: act [E*Cp, I]; FC2: route_out [E*Cp, H]
    int N;                        // tokens (FC1 sentinel row)
    int Kdim;                     // contraction length: FC1 H, FC2 I
    int ncols;                    // output columns: FC1 I, FC2 H
    int wrows;                    // weight rows per expert: FC1 2I, FC2 H
    int Cp;                       // slots per expert
    int MT, NT;                   // M-tiles per expert, N-tiles per expert
};

__device__ __forceinline__ int xcd_remap(int bid, int G) {
    const int q = G / kXcds, r = G % kXcds;
    const int x = bid % kXcds, s = bid / kXcds;
    return x < r ? x * (q + 1) + s : r * (q + 1) + (x - r) * q + s;
}

// byte offset of 16-byte chunk c of LDS row r (128-byte rows)
__device__ __forceinline__ uint32_t lds_off(int r, int c) {
    return static_cast<uint32_t>(r * 128 + ((c ^ (r & 7)) << 4));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kRsrcWord3);
}

__device__ __forceinline__ float silu(float g) {
    // g * sigmoid(g) = g / (1 + e^-g), e^-g = 2^(-g * log2 e)
    const float e = __builtin_amdgcn_exp2f(-g * 1.4426950408889634f);
    return g * __builtin_amdgcn_rcpf(1.0f + e);
}

template <int BMT, int BNT, int WM, int WN, bool FC1>
__global__ __launch_bounds__(WM * WN * kWave) void ffn_gemm_kernel(FfnArgs p) {
    constexpr int NTHR = WM * WN * kWave;
    constexpr int WTM = BMT / WM;
    constexpr int WTN = BNT / WN;
    constexpr int MI = WTM / 32;
    constexpr int NI = WTN / 32;
    constexpr int NIH = NI / 2;
    constexpr int A_PER = BMT * 8 / NTHR;
    constexpr int B_PER = BNT * 8 / NTHR;
    static_assert(MI >= 1 && NI >= 1 && A_PER >= 1 && B_PER >= 1, "tile too small");
    static_assert(!FC1 || NI % 2 == 0, "FC1 waves need matching gate and up blocks");
    static_assert(BMT * 8 % NTHR == 0 && BNT * 8 % NTHR == 0, "uneven tile load");

    __shared__ __attribute__((aligned(16))) uint8_t sA[BMT * kBK * 2];
    __shared__ __attribute__((aligned(16))) uint8_t sB[BNT * kBK * 2];
    __shared__ float s_prob[FC1 ? BMT : 1];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int wm = wave / WN, wn = wave % WN;

    int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int nt = logical % p.NT;
    logical /= p.NT;
    const int mt = logical % p.MT;
    const int e = logical / p.MT;
    const int m0 = mt * BMT;
    const int64_t slot0 = static_cast<int64_t>(e) * p.Cp + m0;   // first slot of this tile

    // ---- operand descriptors and per-thread row offsets (fixed over the K loop)
    __amdgpu_buffer_rsrc_t ra_rsrc, rb_rsrc;
    if (FC1) {
        ra_rsrc = make_rsrc(p.a, static_cast<uint32_t>(p.N) * p.Kdim * 2u);
    } else {
        ra_rsrc = make_rsrc(p.a + static_cast<int64_t>(e) * p.Cp * p.Kdim,
                            static_cast<uint32_t>(p.Cp) * p.Kdim * 2u);
    }
    rb_rsrc = make_rsrc(p.w + static_cast<int64_t>(e) * p.wrows * p.Kdim,
                        static_cast<uint32_t>(p.wrows) * p.Kdim * 2u);

    uint32_t a_goff[A_PER], a_loff[A_PER], b_goff[B_PER], b_loff[B_PER];
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
        const int q = tid + i * NTHR, r = q >> 3, c = q & 7;
        int row;
        if (FC1) {
            row = p.N;   // sentinel: outside the descriptor, reads zeros
            if (m0 + r < p.Cp) {
                const int tok = p.sorted_slot_ids[slot0 + r];
                if (static_cast<unsigned>(tok) < static_cast<unsigned>(p.N)) row = tok;
            }
        } else {
            row = m0 + r;   // rows past Cp lie outside the expert's descriptor
        }
        a_goff[i] = static_cast<uint32_t>(row) * p.Kdim * 2u + c * 16u;
        a_loff[i] = lds_off(r, c);
    }
#pragma unroll
    for (int i = 0; i < B_PER; ++i) {
        const int q = tid + i * NTHR, r = q >> 3, c = q & 7;
        int wrow;
        if (FC1) {
            const int j0 = nt * (BNT / 2);
            wrow = r < BNT / 2 ? j0 + r : p.ncols + j0 + (r - BNT / 2);
        } else {
            wrow = nt * BNT + r;
        }
        b_goff[i] = static_cast<uint32_t>(wrow) * p.Kdim * 2u + c * 16u;
        b_loff[i] = lds_off(r, c);
    }
    if (FC1) {
        for (int i = tid; i < BMT; i += NTHR)
            s_prob[i] = m0 + i < p.Cp ? p.slot_probs[slot0 + i] : 0.0f;
    }

    floatx16 acc[MI][NI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[mi][ni][j] = 0.0f;

    u32x4 ra[A_PER], rb[B_PER];
    auto gload = [&](int kt) {
        const uint32_t koff = static_cast<uint32_t>(kt) * kBK * 2u;
#pragma unroll
        for (int i = 0; i < A_PER; ++i)
            ra[i] = __builtin_amdgcn_raw_buffer_load_b128(ra_rsrc, a_goff[i] + koff, 0, 0);
#pragma unroll
        for (int i = 0; i < B_PER; ++i)
            rb[i] = __builtin_amdgcn_raw_buffer_load_b128(rb_rsrc, b_goff[i] + koff, 0, 0);
    };

    // B-tile LDS row of block ni for this wave (FC1: gate blocks, then up blocks)
    auto b_row = [&](int ni) {
        if (FC1) {
            return ni < NIH ? wn * (WTN / 2) + ni * 32 : BNT / 2 + wn * (WTN / 2) + (ni - NIH) * 32;
        }
        return wn * WTN + ni * 32;
    };

    const int KT = p.Kdim / kBK;
    gload(0);
    for (int kt = 0; kt < KT; ++kt) {
        __syncthreads();
#pragma unroll
        for (int i = 0; i < A_PER; ++i) *reinterpret_cast<u32x4*>(sA + a_loff[i]) = ra[i];
#pragma unroll
        for (int i = 0; i < B_PER; ++i) *reinterpret_cast<u32x4*>(sB + b_loff[i]) = rb[i];
        __syncthreads();
        if (kt + 1 < KT) gload(kt + 1);
#pragma unroll
        for (int ks = 0; ks < kBK / 16; ++ks) {
            const int c = ks * 2 + (lane >> 5);
            bf16x8 af[MI], bfr[NI];
#pragma unroll
            for (int mi = 0; mi < MI; ++mi) {
                const int r = wm * WTM + mi * 32 + (lane & 31);
                af[mi] = *reinterpret_cast<const bf16x8*>(sA + lds_off(r, c));
            }
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) {
                const int r = b_row(ni) + (lane & 31);
                bfr[ni] = *reinterpret_cast<const bf16x8*>(sB + lds_off(r, c));
            }
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                for (int ni = 0; ni < NI; ++ni)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0);
        }
    }

    // ---- epilogue.  32x32 accumulator layout: lane holds column (lane & 31)
    // and rows 8*(j/4) + 4*(lane/32) + (j%4), j = 0..15.
    const int row_lane = 4 * (lane >> 5);
    const int col_lane = lane & 31;
    if (FC1) {
        const int I = p.ncols;
        const int j0 = nt * (BNT / 2);
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int nh = 0; nh < NIH; ++nh) {
                const int col = j0 + wn * (WTN / 2) + nh * 32 + col_lane;
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int row = wm * WTM + mi * 32 + 8 * (j >> 2) + row_lane + (j & 3);
                    if (m0 + row < p.Cp && col < I) {
                        const float g = acc[mi][nh][j], u = acc[mi][nh + NIH][j];
                        p.out[(slot0 + row) * I + col] = f32_to_bf16(silu(g) * u * s_prob[row]);
                    }
                }
            }
    } else {
        const int H = p.ncols;
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) {
                const int col = nt * BNT + wn * WTN + ni * 32 + col_lane;
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int row = wm * WTM + mi * 32 + 8 * (j >> 2) + row_lane + (j & 3);
                    if (m0 + row < p.Cp && col < H)
                        p.out[(slot0 + row) * H + col] = f32_to_bf16(acc[mi][ni][j]);
                }
            }
    }
}

template <int BMT, int BNT, int WM, int WN>
void launch_gemm(FfnArgs a, bool fc1, int E, hipStream_t s) {
    a.MT = (a.Cp + BMT - 1) / BMT;
    a.NT = fc1 ? (a.ncols + BNT / 2 - 1) / (BNT / 2) : (a.ncols + BNT - 1) / BNT;
    const int grid = E * a.MT * a.NT;
    if (fc1) ffn_gemm_kernel<BMT, BNT, WM, WN, true><<<grid, WM * WN * kWave, 0, s>>>(a);
    else ffn_gemm_kernel<BMT, BNT, WM, WN, false><<<grid, WM * WN * kWave, 0, s>>>(a);
}

// M-tile: the one (of 256, 128, 64, 32) that pads Cp the least; ties go to
// the larger tile (fewer re-reads of each weight panel).
int pick_tile_m(int Cp) {
    int best = 256, best_rows = (Cp + 255) / 256 * 256;
    for (int t : {128, 64, 32}) {
        const int rows = (Cp + t - 1) / t * t;
        if (rows < best_rows) { best = t; best_rows = rows; }
    }
    return best;
}

void launch(const FfnArgs& a, bool fc1, int E, hipStream_t s) {
    switch (pick_tile_m(a.Cp)) {
        case 256: launch_gemm<256, 256, 2, 4>(a, fc1, E, s); break;
        case 128: launch_gemm<128, 256, 2, 4>(a, fc1, E, s); break;
        case 64: launch_gemm<64, 128, 2, 2>(a, fc1, E, s); break;
        default: launch_gemm<32, 128, 1, 2>(a, fc1, E, s); break;
    }
}

// Host checks shared by the three FFN entry points.  Buffer offsets inside a
// kernel are 32-bit: x, one expert's weights and one expert's activation rows
// must each stay below 2 GiB.
int check_ffn(int64_t N, int32_t H, int32_t I, int32_t E, int64_t C, int* Cp) {
    if (N < 0 || E < 1 || C < 0) return MOE_ERR_INVALID_ARG;
    int st = check_dims(H, I);
    if (st != MOE_OK) return st;
    if (N > kMaxN || E > kMaxE) return MOE_ERR_UNSUPPORTED;
    const int64_t Cp64 = moe_padded_capacity(C);
    if (Cp64 < 0) return MOE_ERR_UNSUPPORTED;
    const int64_t big = static_cast<int64_t>(1) << 31;
    if (static_cast<int64_t>(E) * Cp64 > INT32_MAX || (N + 1) * H * 2 >= big ||
        Cp64 * std::max(H, I) * 2 >= big || static_cast<int64_t>(2) * I * H * 2 >= big)
        return MOE_ERR_UNSUPPORTED;
    *Cp = static_cast<int>(Cp64);
    return MOE_OK;
}

int check_ptrs(std::initializer_list<const void*> ptrs) {
    for (const void* q : ptrs) {
        if (!q) return MOE_ERR_INVALID_ARG;
        if (!aligned16(q)) return MOE_ERR_MISALIGNED;
    }
    return MOE_OK;
}

FfnArgs fc1_args(const uint16_t* x, const uint16_t* w1, const int32_t* ssi, const float* sp,
                 int64_t N, int32_t H, int32_t I, int Cp, uint16_t* act) {
    FfnArgs a{};
    a.a = x; a.w = w1; a.sorted_slot_ids = ssi; a.slot_probs = sp; a.out = act;
    a.N = static_cast<int>(N); a.Kdim = H; a.ncols = I; a.wrows = 2 * I; a.Cp = Cp;
    return a;
}

FfnArgs fc2_args(const uint16_t* act, const uint16_t* w2, int64_t N, int32_t H, int32_t I, int Cp,
                 uint16_t* route_out) {
    FfnArgs a{};
    a.a = act; a.w = w2; a.out = route_out;
    a.N = static_cast<int>(N); a.Kdim = I; a.ncols = H; a.wrows = H; a.Cp = Cp;
    return a;
}

}  // namespace
}  // namespace moe

extern "C" int moe_grouped_fc1_swiglu(const uint16_t* x, const uint16_t* w1,
                                      const int32_t* sorted_slot_ids, const float* slot_probs,
                                      int64_t N, int32_t H, int32_t I, int32_t E, int64_t C,
                                      uint16_t* act, hipStream_t stream) {
    using namespace moe;
    int Cp = 0;
    int st = check_ffn(N, H, I, E, C, &Cp);
    if (st != MOE_OK) return st;
    if (N == 0 || C == 0) return MOE_OK;
    st = check_ptrs({x, w1, sorted_slot_ids, slot_probs, act});
    if (st != MOE_OK) return st;
    launch(fc1_args(x, w1, sorted_slot_ids, slot_probs, N, H, I, Cp, act), true, E, stream);
    return launch_status();
}

extern "C" int moe_grouped_fc2(const uint16_t* act, const uint16_t* w2, int64_t N, int32_t H,
                               int32_t I, int32_t E, int64_t C, uint16_t* route_out,
                               hipStream_t stream) {
    using namespace moe;
    int Cp = 0;
    int st = check_ffn(N, H, I, E, C, &Cp);
    if (st != MOE_OK) return st;
    if (N == 0 || C == 0) return MOE_OK;
    st = check_ptrs({act, w2, route_out});
    if (st != MOE_OK) return st;
    launch(fc2_args(act, w2, N, H, I, Cp, route_out), false, E, stream);
    return launch_status();
}

extern "C" int moe_grouped_ffn_fwd(const uint16_t* x, const uint16_t* w1, const uint16_t* w2,
                                   const int32_t* sorted_slot_ids, const float* slot_probs,
                                   int64_t N, int32_t H, int32_t I, int32_t E, int64_t C,
                                   uint16_t* act, uint16_t* route_out, hipStream_t stream) {
    using namespace moe;
    int Cp = 0;
    int st = check_ffn(N, H, I, E, C, &Cp);
    if (st != MOE_OK) return st;
    if (N == 0 || C == 0) return MOE_OK;
    st = check_ptrs({x, w1, w2, sorted_slot_ids, slot_probs, act, route_out});
    if (st != MOE_OK) return st;
    launch(fc1_args(x, w1, sorted_slot_ids, slot_probs, N, H, I, Cp, act), true, E, stream);
    launch(fc2_args(act, w2, N, H, I, Cp, route_out), false, E, stream);
    return launch_status();
}
