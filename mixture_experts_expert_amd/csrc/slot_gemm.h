// Grouped GEMM whose output rows are an expert's slots (internal):
//
//   out[seg + s, n] = sum_k A[seg + s, k] * B_e[k, n]     s < Cp, n < Nn, k < Kd
//
// with A route-ordered (row s of expert e's segment seg = e*Cp) and B_e expert
// e's weight matrix, stored N-major ([Nn][Kd], FC2's W2 in the forward) or
// K-major ([Kd][Nn], the transposed-weight view of a dgrad).  With a row map
// the output row of slot seg + s is out_rows[seg + s] instead (any row of
// the E*Cp-row output; entries outside it drop the row).
//
// [PF] "Permute-Free Grouped GEMM for MoE (bf16, gfx950)", sections 3 and 5:
// FC2 of the forward (A = act by route position) and the FC1 data gradient
// (A = d_preact by route position, B = W1 read K-major).
//
// gfx950 design: bf16 MFMA 32x32x16 with float32 accumulators, 256x256 output
// tiles, 64-deep K slabs staged through LDS by DMA rings (A two stages deep,
// B three).  One persistent workgroup per CU walks its tiles (t, t+G, ...)
// with the rings running across tile boundaries, and its waves specialise:
// four producer waves issue the slab loads and wait for them, eight consumer
// waves run the MFMAs and store the output.  Vector-memory wait counters are
// per wave and count stores as well as loads, so consumers that never wait
// let a tile's stores drain while the next tile loads and computes; the two
// kinds meet at one barrier per K step.
#pragma once

#include "gemm_common.h"

namespace moe {
namespace {

struct SlotArgs {
    const uint16_t* a;            // A rows (row-major, K contiguous)
    const uint16_t* b;            // expert weights, b_estride elements apart
    uint16_t* out;                // [E*Cp, ldo]
    const int* out_rows;          // row map (ROWMAP only): slot -> output row
    int lda, ldb, ldo;            // row pitches in elements
    int Nn, Kd;                   // output columns, contraction length
    int Cp;                       // slots per expert
    int MT, NT, tiles;            // tiles per expert (M, N), all tiles
    int64_t b_estride;
    int krot;                     // expert e starts its K walk at slab (e*krot) % KT
};

template <bool BKM, bool ROWMAP = false>
__global__ __launch_bounds__(768) void slot_gemm_kernel(SlotArgs p) {
    constexpr int BMT = 256, BNT = 256, BK = 64, WM = 2, WN = 4, NA = 2, NB = 3;
    constexpr int NC = WM * WN;                    // consumer waves
    constexpr int NP = 4;                          // producer waves
    constexpr int WTM = BMT / WM, WTN = BNT / WN;
    constexpr int MI = WTM / 32, NI = WTN / 32;
    constexpr int AROWB = BK * 2;                  // A stage: BMT rows of BK values
    constexpr int BROWB = BKM ? BNT * 2 : BK * 2;  // B stage: BK rows of BNT, or BNT rows of BK
    constexpr int A_STAGE = BMT * AROWB;
    constexpr int B_STAGE = BKM ? BK * BROWB : BNT * BROWB;
    constexpr int A_RPI = 1024 / AROWB, B_RPI = 1024 / BROWB;   // rows per 1 KB DMA load
    constexpr int A_CPR = AROWB / 16, B_CPR = BROWB / 16;       // 16-byte chunks per row
    constexpr int A_INST = A_STAGE / 1024 / NP, B_INST = B_STAGE / 1024 / NP;
    constexpr int B_RING = NA * A_STAGE;
    constexpr int LDS_BYTES = NA * A_STAGE + NB * B_STAGE;
    constexpr int SLICES = BK / 16;
    static_assert(A_INST >= 1 && B_INST >= 1 && A_STAGE % (1024 * NP) == 0 && B_STAGE % (1024 * NP) == 0,
                  "whole DMA blocks per producer");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");
    static_assert(B_INST < 64, "wait counts");

    __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS_BYTES];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
    const int half = lane >> 5;
    const int G = gridDim.x;
    const int KT = (p.Kd + BK - 1) / BK;
    const int len = p.Cp;
    const int t0 = xcd_remap(blockIdx.x, G);
    if (t0 >= p.tiles) return;                     // the whole workgroup
    const int S = (p.tiles - t0 + G - 1) / G * KT; // K steps of this workgroup

    if (wave >= NC) {
        // ---------------- producer: 1 KB blocks q = pw + i*NP of each stage
        const int pw = wave - NC;
        const uint32_t a_rowb = static_cast<uint32_t>(p.lda) * 2u;
        const uint32_t b_rowb = static_cast<uint32_t>(p.ldb) * 2u;
        // A pointer (the tile and K step whose A slab is issued next) and
        // B pointer; each keeps what follows from its tile
        struct Ptr {
            int t, kt, rot;
            i32x4 r;
            uint32_t base[A_INST > B_INST ? A_INST : B_INST];   // per-lane row offsets
        };
        auto place_a = [&](Ptr& d) {
            const int rest = d.t / p.NT;
            const int e = rest / p.MT, m0 = (rest % p.MT) * BMT;
            const int seg = min(e, p.tiles / (p.MT * p.NT) - 1) * p.Cp;   // pointers past the end read nothing
            const bool live = d.t < p.tiles;
            d.rot = (e * p.krot) % KT;
            d.r = make_rsrc(p.a + static_cast<int64_t>(seg) * p.lda, static_cast<uint32_t>(len) * a_rowb);
#pragma unroll
            for (int i = 0; i < A_INST; ++i) {
                const int r = A_RPI * (pw + i * NP) + lane / A_CPR;   // tile row
                const int row = live && m0 + r < len ? m0 + r : -1;
                const int chunk = (lane % A_CPR) ^ ((r / (256 / AROWB)) % A_CPR);
                d.base[i] = row < 0 ? kOob : static_cast<uint32_t>(row) * a_rowb + chunk * 16u;
            }
        };
        auto place_b = [&](Ptr& d) {
            const int nt = d.t % p.NT, rest = d.t / p.NT;
            const int e = min(rest / p.MT, p.tiles / (p.MT * p.NT) - 1);
            const bool live = d.t < p.tiles;
            d.rot = (e * p.krot) % KT;
            d.r = make_rsrc(p.b + static_cast<int64_t>(e) * p.b_estride,
                            static_cast<uint32_t>(BKM ? p.Kd : p.Nn) * b_rowb);
#pragma unroll
            for (int i = 0; i < B_INST; ++i) {
                const int r = B_RPI * (pw + i * NP) + lane / B_CPR;
                if (BKM) {
                    // K-major: stage row r is K row (slab*BK + r), columns n0.. ; chunk ^ 4*(r%4)
                    const int chunk = (lane % B_CPR) ^ (4 * (r & 3));
                    d.base[i] = live ? static_cast<uint32_t>(r) * b_rowb + (nt * BNT + chunk * 8) * 2u : kOob;
                } else {
                    // N-major: stage row r is weight row n0 + r (past Nn: zeros)
                    const int chunk = (lane % B_CPR) ^ ((r / (256 / BROWB)) % B_CPR);
                    d.base[i] = live ? static_cast<uint32_t>(nt * BNT + r) * b_rowb + chunk * 16u : kOob;
                }
            }
        };
        auto slab = [&](const Ptr& d) {
            const int k = d.kt + d.rot;
            return k < KT ? k : k - KT;
        };
        auto advance = [&](Ptr& d, bool is_a) {
            if (++d.kt == KT) {
                d.kt = 0;
                d.t += G;
                if (is_a) place_a(d); else place_b(d);
            }
        };
        const uint32_t lds0 = lds_addr(smem);
        auto issue_a = [&](Ptr& d, int stage_off) {
            const uint32_t koff = static_cast<uint32_t>(slab(d)) * AROWB;
#pragma unroll
            for (int i = 0; i < A_INST; ++i)
                dma16(d.r, d.base[i] == kOob ? kOob : d.base[i] + koff, lds0 + stage_off + (pw + i * NP) * 1024);
            advance(d, true);
        };
        auto issue_b = [&](Ptr& d, int stage_off) {
            const uint32_t koff = static_cast<uint32_t>(slab(d)) * (BKM ? BK * b_rowb : BK * 2u);
#pragma unroll
            for (int i = 0; i < B_INST; ++i)
                dma16<true>(d.r, d.base[i] == kOob ? kOob : d.base[i] + koff,
                            lds0 + B_RING + stage_off + (pw + i * NP) * 1024);
            advance(d, false);
        };
        Ptr pa, pb;
        pa.t = pb.t = t0;
        pa.kt = pb.kt = 0;
        place_a(pa);
        place_b(pb);
        // prologue: B(0), then A(0) and B(1) (a step's order: A, then B)
        issue_b(pb, 0);
        issue_a(pa, 0);
        issue_b(pb, B_STAGE);
        wait_vmcnt<B_INST>();                      // A(0), B(0) are in; B(1) may not be
        __syncthreads();
        int a_fill = A_STAGE, b_fill = 2 * B_STAGE;
        for (int g = 0; g < S; ++g) {
            // refill the stages computed at step g-1: A(g+1), B(g+2)
            issue_a(pa, a_fill);
            issue_b(pb, b_fill);
            a_fill = a_fill == 0 ? A_STAGE : 0;
            b_fill = b_fill + B_STAGE == NB * B_STAGE ? 0 : b_fill + B_STAGE;
            wait_vmcnt<B_INST>();                  // slab g+1 is in: A(g+1) and the older B(g+1)
            __syncthreads();
            // a tile ends at step g: the consumers stage its output in the
            // two stages step g read, which stay unfilled until they are done
            if ((g + 1) % KT == 0) __syncthreads();
        }
        wait_vmcnt<0>();   // no DMA may still be writing LDS when the workgroup ends
        return;
    }

    // ---------------- consumer
    const int wm = wave / WN, wn = wave % WN;
    floatx16 acc[MI][NI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[mi][ni][j] = 0.0f;
    __syncthreads();
    int tc = t0, ktc = 0, a_rd = 0, b_rd = 0;
    // ROWMAP: the output rows of the slots whose staged rows the lane writes
    // (rows h*64 + j*8 + lane/8 of the wave's piece), fetched at the tile's
    // first step and used at its end
    int orow[ROWMAP ? MI / 2 * 8 : 1];
    for (int g = 0; g < S; ++g) {
        if (ROWMAP && ktc == 0) {
            const int rest = tc / p.NT;
            const int e = rest / p.MT, m0 = (rest % p.MT) * BMT;
#pragma unroll
            for (int h = 0; h < MI / 2; ++h)
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int slot = m0 + wm * WTM + h * 64 + j * 8 + lane / 8;
                    orow[h * 8 + j] = slot < len ? p.out_rows[static_cast<int64_t>(e) * p.Cp + slot] : -1;
                }
        }
        const uint8_t* sA = smem + a_rd;
        const lds_u8* sB = (const lds_u8*)smem + B_RING + b_rd;
#pragma unroll
        for (int ks = 0; ks < SLICES; ++ks) {
            bf16x8 af[MI], bfr[NI];
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
                af[mi] = *reinterpret_cast<const bf16x8*>(sA + lds_off<BK>(wm * WTM + mi * 32 + (lane & 31), ks * 2 + half));
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) {
                if (BKM)
                    bfr[ni] = tr_frag(sB, tr_off<BROWB>(lane, wn * WTN + ni * 32, ks * 16, 0),
                                           tr_off<BROWB>(lane, wn * WTN + ni * 32, ks * 16, 1));
                else
                    bfr[ni] = *reinterpret_cast<const bf16x8*>(
                        (const uint8_t*)smem + B_RING + b_rd + lds_off<BK>(wn * WTN + ni * 32 + (lane & 31), ks * 2 + half));
            }
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                for (int ni = 0; ni < NI; ++ni)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[ni], af[mi], acc[mi][ni], 0, 0, 0);
        }
        const int a_done = a_rd, b_done = b_rd;   // the stages this step read
        a_rd = a_rd == 0 ? A_STAGE : 0;
        b_rd = b_rd + B_STAGE == NB * B_STAGE ? 0 : b_rd + B_STAGE;
        if (++ktc == KT) {
            // the tile is done: lane (row l&31, half h) holds columns
            // 8g + 4h + (0..3) of each 32-column block in acc[4g..4g+3];
            // packed to bf16, a swap of lane halves gives each lane 8
            // consecutive columns.  After a barrier (every consumer is past
            // this step's LDS reads) each consumer stages its 128 x 64 piece,
            // 64 rows at a time, in its own 8 KB of the two stages this step
            // read (16-byte chunks swizzled by row) and writes each row's 128
            // bytes with 8 lanes; the producers refill those stages only
            // after the next barrier.  Rows past Cp and columns past Nn get an
            // offset beyond the descriptor: the store is dropped.
            const int nt = tc % p.NT, rest = tc / p.NT;
            const int e = rest / p.MT, m0 = (rest % p.MT) * BMT;
            // the output rows: the expert's segment, or (ROWMAP) the whole
            // E*Cp-row output, whose size the host keeps below 2^31 bytes
            const int rows_out = p.tiles / (p.MT * p.NT) * p.Cp;
            const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
                ROWMAP ? p.out : p.out + static_cast<int64_t>(e) * p.Cp * p.ldo, static_cast<short>(0),
                (ROWMAP ? rows_out : len) * p.ldo * 2, kRsrcWord3);
            typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
            static_assert(NC == 8 && WTN == 64 && MI % 2 == 0 && A_STAGE >= 4 * 8192 && B_STAGE >= 4 * 8192,
                          "staging: 8 KB per consumer in the stages a step reads");
            __syncthreads();
            lds_u8* st = (lds_u8*)smem + (wave < NC / 2 ? a_done + wave * 8192 : B_RING + b_done + (wave - NC / 2) * 8192);
            auto so = [](int r, int c) { return static_cast<uint32_t>(r * 128 + ((c ^ (r & 7)) << 4)); };
#pragma unroll
            for (int h = 0; h < MI / 2; ++h) {
                asm volatile("" ::: "memory");
#pragma unroll
                for (int m2 = 0; m2 < 2; ++m2) {
                    const int mi = 2 * h + m2;
#pragma unroll
                    for (int ni = 0; ni < NI; ++ni) {
                        uint32_t gq[4][2];
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            gq[q][0] = pack_bf16x2(acc[mi][ni][4 * q], acc[mi][ni][4 * q + 1]);
                            gq[q][1] = pack_bf16x2(acc[mi][ni][4 * q + 2], acc[mi][ni][4 * q + 3]);
                        }
#pragma unroll
                        for (int q = 0; q < 2; ++q) {
                            const auto s0 = __builtin_amdgcn_permlane32_swap(gq[2 * q][0], gq[2 * q + 1][0], false, false);
                            const auto s1 = __builtin_amdgcn_permlane32_swap(gq[2 * q][1], gq[2 * q + 1][1], false, false);
                            u32x4 d;
                            d[0] = s0[0]; d[1] = s1[0]; d[2] = s0[1]; d[3] = s1[1];
                            *(lds_u32x4*)(st + so(m2 * 32 + (lane & 31), ni * 4 + 2 * q + half)) = d;
                        }
#pragma unroll
                        for (int j = 0; j < 16; ++j) acc[mi][ni][j] = 0.0f;
                    }
                }
                // the wave reads back what its other lanes wrote: LDS
                // operations of one wave complete in order, and the clobbers
                // keep the compiler from moving them across
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int r = j * 8 + lane / 8, c = lane % 8;
                    const u32x4 v = *(const lds_u32x4*)(st + so(r, c));
                    const int srow = h * 64 + r;                      // row of the wave's piece
                    int row;
                    bool row_live;
                    if (ROWMAP) {
                        row = orow[ROWMAP ? h * 8 + j : 0];       // slot m0 + wm*WTM + srow's
                        row_live = static_cast<unsigned>(row) < static_cast<unsigned>(rows_out);
                    } else {
                        row = m0 + wm * WTM + srow;
                        row_live = row < len;
                    }
                    const int col = nt * BNT + wn * WTN + c * 8;
                    const uint32_t off = row_live && col < p.Nn
                        ? (static_cast<uint32_t>(row) * p.ldo + col) * 2u : kOob;
                    __builtin_amdgcn_raw_buffer_store_b128(v, orsrc, off, 0, 0);
                }
                asm volatile("" ::: "memory");
            }
            ktc = 0;
            tc += G;
        }
        __syncthreads();
    }
}

}  // namespace
}  // namespace moe
