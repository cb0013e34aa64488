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

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer descriptor: base, stride 0, num_records = bytes, 32-bit data format.
// A load whose offset (everything is passed in the per-lane voffset, which the
// range check covers) lies at or beyond `bytes` returns zeros and touches no
// memory: this is how the sentinel row N and rows past an expert's segment
// read as zeros.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    i32x4 r;
    // the descriptor lives in scalar registers: every lane holds the same value
    r.x = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(a)));
    r.y = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(a >> 32) & 0xFFFFu));
    r.z = __builtin_amdgcn_readfirstlane(static_cast<int>(bytes));
    r.w = kRsrcWord3;
    return r;
}

// LDS byte address of a __shared__ object (what M0 and ds_* instructions use).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
        (const __attribute__((address_space(3))) void*)p));
}

// 16 bytes per lane from global memory straight into LDS: lane L's data lands
// at M0 + 16*L, so one wave fills one contiguous kilobyte.  Issued as inline
// assembly so the compiler neither tracks it (it would otherwise wait for every
// pending LDS-bound load before any LDS read) nor reorders it across the
// explicit waits below ("memory" clobber).
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t voff, uint32_t lds) {
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
                 :: "v"(voff), "s"(rsrc), "{m0}"(__builtin_amdgcn_readfirstlane(lds))
                 : "memory");
}

// Wait until at most N of this wave's vector-memory operations are pending.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

__device__ __forceinline__ float silu(float g) {
    // g * sigmoid(g) = g / (1 + e^-g), e^-g = 2^(-g * log2 e)
    const float e = __builtin_amdgcn_exp2f(-g * 1.4426950408889634f);
    return g * __builtin_amdgcn_rcpf(1.0f + e);
}

// LDS layout of one stage: tile row r (ROWB = 2*BK bytes, CPR = ROWB/16
// chunks of 8 K values) at r*ROWB; logical chunk c sits at physical chunk
// c ^ ((r / RP) % CPR) with RP = 256/ROWB rows per 256 bytes.  An MFMA operand
// read has 16 consecutive lanes fetch one chunk of 16 consecutive rows; with
// 64 four-byte banks the swizzle spreads them over all 256 bytes.
template <int BK>
__device__ __forceinline__ uint32_t lds_off(int r, int c) {
    constexpr int ROWB = BK * 2, CPR = ROWB / 16, RP = 256 / ROWB;
    return static_cast<uint32_t>(r * ROWB + ((c ^ ((r / RP) % CPR)) << 4));
}

template <int BMT, int BNT, int WM, int WN, int BK, int NA, int NB, bool FC1>
__global__ __launch_bounds__(WM * WN * kWave) void ffn_gemm_kernel(FfnArgs p) {
    constexpr int NW = WM * WN;
    constexpr int NTHR = NW * kWave;
    constexpr int WTM = BMT / WM;
    constexpr int WTN = BNT / WN;
    constexpr int MI = WTM / 32;
    constexpr int NI = WTN / 32;
    constexpr int ROWB = BK * 2;                           // bytes of a tile row per stage
    constexpr int CPR = ROWB / 16;                         // 16-byte chunks per tile row
    constexpr int RPI = 1024 / ROWB;                       // tile rows per 1 KB DMA load
    constexpr int A_STAGE = BMT * ROWB;
    constexpr int B_STAGE = BNT * ROWB;
    constexpr int B_RING = NA * A_STAGE;                   // the B ring follows the A ring
    constexpr int A_INST = BMT / RPI / NW;                 // DMA loads per wave per stage
    constexpr int B_INST = BNT / RPI / NW;
    constexpr int LOADS = A_INST + B_INST;                 // per wave per K slab
    constexpr int OUT_COLS = FC1 ? BNT / 2 : BNT;          // output columns of this tile
    constexpr int OUT_PITCH = OUT_COLS * 2 + 16;           // padded bf16 row of the staged output
    constexpr int RINGS = NA * A_STAGE + NB * B_STAGE;
    constexpr int LDS_BYTES = RINGS > BMT * OUT_PITCH ? RINGS : BMT * OUT_PITCH;
    // Step j issues A(j+NA-1) then B(j+NB-1); loads complete in issue order.
    // Before computing slab kt, the newer of A(kt) and B(kt) must have landed:
    // A(kt) if NA < NB (then B(kt+NB-NA) of the same step and NA-2 whole steps
    // follow it), else B(kt) (NB-2 whole steps follow it).
    constexpr int WAIT = NA < NB ? B_INST + (NA - 2) * LOADS : (NB - 2) * LOADS;
    static_assert(MI >= 1 && NI >= 1, "tile too small");
    static_assert(BK == 32 || BK == 64, "K slab");
    static_assert(A_INST >= 1 && B_INST >= 1 && BMT % (RPI * NW) == 0 && BNT % (RPI * NW) == 0,
                  "whole DMA blocks per wave");
    static_assert(NA >= 2 && NB >= 2 && WAIT < 64, "stage rings");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");

    __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS_BYTES];

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

    // ---- DMA addressing.  Wave w's load i covers the RPI tile rows of block
    // q = w + i*NW; lane L brings row RPI*q + L/CPR, physical chunk L%CPR,
    // i.e. the logical chunk that the swizzle of that row puts there.
    const int lrow = lane / CPR;
    auto lchunk = [&](int q) -> uint32_t {
        const int r = RPI * q + lrow;
        return static_cast<uint32_t>((lane % CPR) ^ ((r / (256 / ROWB)) % CPR));
    };
    const uint32_t row_bytes = static_cast<uint32_t>(p.Kdim) * 2u;
    i32x4 ra_rsrc, rb_rsrc;
    if (FC1) {
        ra_rsrc = make_rsrc(p.a, static_cast<uint32_t>(p.N) * row_bytes);
    } else {
        ra_rsrc = make_rsrc(p.a + static_cast<int64_t>(e) * p.Cp * p.Kdim,
                            static_cast<uint32_t>(p.Cp) * row_bytes);
    }
    rb_rsrc = make_rsrc(p.w + static_cast<int64_t>(e) * p.wrows * p.Kdim,
                        static_cast<uint32_t>(p.wrows) * row_bytes);

    uint32_t a_voff[A_INST], b_voff[B_INST];
#pragma unroll
    for (int i = 0; i < A_INST; ++i) {
        const int q = wave + i * NW;
        const int r = RPI * q + lrow;
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
        a_voff[i] = static_cast<uint32_t>(row) * row_bytes + lchunk(q) * 16u;
    }
#pragma unroll
    for (int i = 0; i < B_INST; ++i) {
        const int q = wave + i * NW;
        const int R = RPI * q + lrow;                    // tile row
        int wrow;
        if (FC1) {
            // FC1's B tile interleaves 16 gate rows and the 16 matching up rows
            // in each 32-row MFMA block, so one accumulator block carries both.
            const int w = R & 31;
            wrow = (w < 16 ? 0 : p.ncols) + nt * (BNT / 2) + (R >> 5) * 16 + (w & 15);
        } else {
            wrow = nt * BNT + R;
        }
        b_voff[i] = static_cast<uint32_t>(wrow) * row_bytes + lchunk(q) * 16u;
    }
    const uint32_t lds0 = lds_addr(smem);

    auto issue_a = [&](int buf, int kt) {
        const uint32_t koff = static_cast<uint32_t>(kt) * ROWB;
        const uint32_t st = lds0 + buf * A_STAGE;
#pragma unroll
        for (int i = 0; i < A_INST; ++i) dma16(ra_rsrc, a_voff[i] + koff, st + (wave + i * NW) * 1024);
    };
    auto issue_b = [&](int buf, int kt) {
        const uint32_t koff = static_cast<uint32_t>(kt) * ROWB;
        const uint32_t st = lds0 + B_RING + buf * B_STAGE;
#pragma unroll
        for (int i = 0; i < B_INST; ++i) dma16(rb_rsrc, b_voff[i] + koff, st + (wave + i * NW) * 1024);
    };

    floatx16 acc[MI][NI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[mi][ni][j] = 0.0f;

    auto compute = [&](int abuf, int bbuf) {
        const uint8_t* sA = smem + abuf * A_STAGE;
        const uint8_t* sB = smem + B_RING + bbuf * B_STAGE;
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const int c = ks * 2 + (lane >> 5);
            bf16x8 af[MI], bfr[NI];
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
                af[mi] = *reinterpret_cast<const bf16x8*>(sA + lds_off<BK>(wm * WTM + mi * 32 + (lane & 31), c));
#pragma unroll
            for (int ni = 0; ni < NI; ++ni)
                bfr[ni] = *reinterpret_cast<const bf16x8*>(sB + lds_off<BK>(wn * WTN + ni * 32 + (lane & 31), c));
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                for (int ni = 0; ni < NI; ++ni)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0);
        }
    };

    // ---- K loop over two LDS rings: the gathered A slabs (L2/MALL hits, short
    // latency) NA deep, the weight slabs (the HBM stream) NB deep, so NB-1
    // weight slabs are in flight while one is consumed.  Step j issues
    // A(j+NA-1) then B(j+NB-1); the prologue replays the steps before 0.
    // Loads past the end of K are issued anyway (they read the next row or,
    // past the descriptor, zeros, into stages never computed) so every step
    // waits for the same count.  The barrier after the wait publishes slab kt
    // and retires slab kt-1, whose stages the new loads overwrite.
    const int KT = p.Kdim / BK;
    __syncthreads();   // the token rows are read; the rings are free
    constexpr int LEAD = NA > NB ? NA : NB;
#pragma unroll
    for (int j = -(LEAD - 1); j < 0; ++j) {
        if (j + NA - 1 >= 0) issue_a(j + NA - 1, j + NA - 1);
        if (j + NB - 1 >= 0) issue_b(j + NB - 1, j + NB - 1);
    }
    int abuf = 0, bbuf = 0;
    for (int kt = 0; kt < KT; ++kt) {
        wait_vmcnt<WAIT>();
        __syncthreads();
        issue_a(abuf == 0 ? NA - 1 : abuf - 1, kt + NA - 1);   // stage (kt + NA - 1) % NA
        issue_b(bbuf == 0 ? NB - 1 : bbuf - 1, kt + NB - 1);
        compute(abuf, bbuf);
        abuf = abuf + 1 == NA ? 0 : abuf + 1;
        bbuf = bbuf + 1 == NB ? 0 : bbuf + 1;
    }
    wait_vmcnt<0>();   // no DMA may land in the LDS the epilogue reuses
    __syncthreads();

    // ---- epilogue.  32x32 accumulator layout: lane holds column (lane & 31)
    // and rows 8*(j/4) + 4*(lane/32) + (j%4), j = 0..15.  The bf16 tile is
    // staged in LDS (rows padded by 16 bytes) and written out in 16-byte
    // chunks along rows.
    const int row_lane = 4 * (lane >> 5);
    const int col_lane = lane & 31;
    if (FC1) {
        // Lane l (column l&31 of a block) holds gate if (l & 16) == 0, else the
        // up value of column l^16.  Partners swap every value and both form the
        // activation.  (Selecting values, never vector elements, keeps the
        // compiler from building a dynamic element index.)
        const bool gate_lane = (lane & 16) == 0;
        float prob[MI][16];   // routing probability of each accumulator row (0 past Cp)
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int row = wm * WTM + mi * 32 + 8 * (j >> 2) + row_lane + (j & 3);
                prob[mi][j] = m0 + row < p.Cp ? p.slot_probs[slot0 + row] : 0.0f;
            }
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) {
                const int col = (wn * WTN + ni * 32) / 2 + (lane & 15);
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const float mine = acc[mi][ni][j];
                    const float other = __shfl_xor(mine, 16, kWave);
                    const float g = gate_lane ? mine : other;
                    const float u = gate_lane ? other : mine;
                    const int row = wm * WTM + mi * 32 + 8 * (j >> 2) + row_lane + (j & 3);
                    // both partners form the same value and store it to the same place
                    *reinterpret_cast<uint16_t*>(smem + row * OUT_PITCH + col * 2) =
                        f32_to_bf16(silu(g) * u * prob[mi][j]);
                }
            }
    } else {
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) {
                const int col = wn * WTN + ni * 32 + col_lane;
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int row = wm * WTM + mi * 32 + 8 * (j >> 2) + row_lane + (j & 3);
                    *reinterpret_cast<uint16_t*>(smem + row * OUT_PITCH + col * 2) = f32_to_bf16(acc[mi][ni][j]);
                }
            }
    }
    __syncthreads();
    constexpr int OCPR = OUT_COLS / 8;           // 16-byte chunks per output row
    const int col0 = nt * OUT_COLS;
    for (int q = tid; q < BMT * OCPR; q += NTHR) {
        const int r = q / OCPR, c = q - r * OCPR;
        if (m0 + r < p.Cp && col0 + c * 8 < p.ncols)
            *reinterpret_cast<u32x4*>(p.out + (slot0 + r) * p.ncols + col0 + c * 8) =
                *reinterpret_cast<const u32x4*>(smem + r * OUT_PITCH + c * 16);
    }
}

template <int BMT, int BNT, int WM, int WN, int BK, int NA, int NB>
void launch_gemm(FfnArgs a, bool fc1, int E, hipStream_t s) {
    a.MT = (a.Cp + BMT - 1) / BMT;
    a.NT = fc1 ? (a.ncols + BNT / 2 - 1) / (BNT / 2) : (a.ncols + BNT - 1) / BNT;
    const int grid = E * a.MT * a.NT;
    if (fc1) ffn_gemm_kernel<BMT, BNT, WM, WN, BK, NA, NB, true><<<grid, WM * WN * kWave, 0, s>>>(a);
    else ffn_gemm_kernel<BMT, BNT, WM, WN, BK, NA, NB, false><<<grid, WM * WN * kWave, 0, s>>>(a);
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
        // 64-wide K slabs (128 contiguous bytes per weight row per step keep the
        // HBM stream efficient); rings sized to the 160 KB LDS.
        case 256: launch_gemm<256, 256, 2, 4, 64, 2, 3>(a, fc1, E, s); break;
        case 128: launch_gemm<128, 256, 2, 4, 64, 2, 3>(a, fc1, E, s); break;
        case 64: launch_gemm<64, 128, 2, 2, 64, 2, 3>(a, fc1, E, s); break;
        default: launch_gemm<32, 128, 1, 2, 64, 2, 3>(a, fc1, E, s); break;
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
