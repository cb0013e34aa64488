// Backward of the permute-free grouped FFN: data-gradient and weight-gradient
// GEMMs.
//
// [PF] "Permute-Free Grouped GEMM for MoE (bf16, gfx950)":
//   section 3  FC2 dgrad gathers the token-space gradient dy into the route
//              buffer (here inside the A-tile loads, as the forward gathers x);
//              FC1 dgrad's per-route input gradients are reduced to token rows
//              by the contention-free gather-combine (combine.hip);
//   section 5  dgrad contracts against the transposed-weight view; wgrad is
//              expert-centric, contracts over the slot axis with an LDS fill
//              and transpose reads, and each dW tile has exactly one owner,
//              which writes it as bf16 or adds it into a float32 main
//              gradient inside the kernel.
//
// Per expert e (slots [e*Cp, (e+1)*Cp)):
//
//   FC2 dgrad  d_act[s, i]  = sum_h dy[row(s), h] * W2[e][h, i]
//   FC1 dgrad  d_a[s, h]    = sum_j d_pre[s, j]   * W1[e][j, h]
//   FC2 wgrad  dW2[e][h, i] = sum_s dy[row(s), h] * act[s, i]
//   FC1 wgrad  dW1[e][j, h] = sum_s d_pre[s, j]   * x[row(s), h]
//
// with row(s) = sorted_slot_ids[s] (the sentinel N reads as a zero row).
//
// gfx950 design:
//   * bf16 MFMA 32x32x16, float32 accumulators, 256x256 output tiles, 64-deep
//     K slabs staged through LDS by DMA (global -> LDS) rings;
//   * K-major operands (the weights [K][N] of dgrad; both slot-indexed
//     operands of wgrad) hold one K row per LDS row, and the MFMA fragments
//     (8 consecutive K per lane) come from two ds_read_b64_tr_b16 transpose
//     reads.  gfx950's transpose read hands lane i of a 16-lane group element
//     i%4 of the 8-byte pieces addressed by lanes 4j + i/4 (j = 0..3); so when
//     lane c addresses row k0 + c/4, columns n0 + 4(c%4) .. +3, lane i
//     receives column n0 + i of rows k0 .. k0+3;
//   * dgrad's A operand is row-major by slot (read with ds_read_b128, like
//     the forward);
//   * K-major stages swizzle their 16-byte chunks by row (chunk ^ 4*(row%4)):
//     the four rows of one transpose read then fall on disjoint banks;
//   * gathered rows come straight from token order through the route list;
//   * FC2 dgrad: one workgroup of 8 waves per output tile (long K: the loads
//     overlap the MFMAs within the tile); consecutive tiles (same expert,
//     neighbouring N-tiles) are renumbered onto the same XCD;
//   * FC1 dgrad: the persistent producer/consumer slot GEMM (slot_gemm.h),
//     whose consumer waves store without waiting on the loads;
//   * wgrad: short K and a large output per tile, so one persistent
//     workgroup per CU with producer and consumer waves (below).
#include <algorithm>
#include <initializer_list>

#include "gemm_common.h"
#include "slot_gemm.h"

namespace moe {
namespace {

enum RowSrc : int {
    kRowWeight = 0,   // row k of expert e's weight matrix
    kRowRoute = 1,    // row s of a route-ordered buffer (the expert's segment)
    kRowGather = 2,   // token row sorted_slot_ids[s] of a token-ordered buffer
};

struct BwdArgs {
    const uint16_t* a;            // A source: dy (FC2) or d_pre (FC1)
    const uint16_t* b;            // B source: W2 / W1 (dgrad), act / x (wgrad)
    const int* sorted_slot_ids;
    uint16_t* out;
    int lda, ldb, ldo;            // row pitches in elements
    int N;                        // token rows of gathered sources
    int M, Nn, Kd;                // per-expert product: out[M, Nn] over Kd
    int Cp;                       // slots per expert
    int MT, NT, tiles;
    int64_t b_estride;            // weights: elements between experts (dgrad)
    int64_t o_estride;            // dW: elements between experts (wgrad)
    float* out32;                 // float32 main gradient the wgrad adds into (or null)
};

typedef const __attribute__((address_space(4))) int* const_int_ptr;

// Data gradient: out rows are the expert's slots, A is row-major by slot
// (the expert's segment of a route-ordered buffer, or gathered token rows),
// B is the expert's weight matrix, K-major.
template <int BMT, int BNT, int WM, int WN, int BK, int NA, int NB, int ASRC>
__global__ __launch_bounds__(WM * WN * kWave) void dgrad_kernel(BwdArgs p) {
    constexpr int NW = WM * WN;
    constexpr int WTM = BMT / WM, WTN = BNT / WN;
    constexpr int MI = WTM / 32, NI = WTN / 32;
    constexpr int AROWB = BK * 2;                  // A: BMT rows of BK columns
    constexpr int BROWB = BNT * 2;                 // B: BK rows of BNT columns
    constexpr int A_STAGE = BMT * AROWB;
    constexpr int B_STAGE = BK * BROWB;
    constexpr int A_RPI = 1024 / AROWB;            // rows per DMA load
    constexpr int A_CPR = AROWB / 16, B_CPR = BROWB / 16;       // 16-byte chunks per row
    constexpr int B_RPI = 1024 / BROWB;
    constexpr int A_INST = A_STAGE / 1024 / NW, B_INST = B_STAGE / 1024 / NW;
    constexpr int LOADS = A_INST + B_INST;
    constexpr int B_RING = NA * A_STAGE;
    constexpr int LDS_BYTES = NA * A_STAGE + NB * B_STAGE;
    constexpr int WAIT = NA < NB ? B_INST + (NA - 2) * LOADS : (NB - 2) * LOADS;
    static_assert(MI >= 1 && NI >= 1 && BK == 64, "tile shape");
    static_assert(A_INST >= 1 && B_INST >= 1 && A_STAGE % (1024 * NW) == 0 &&
                  B_STAGE % (1024 * NW) == 0, "whole DMA blocks per wave");
    static_assert(NA >= 2 && NB >= 2 && WAIT < 64, "stage rings");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");
    static_assert(ASRC != kRowWeight, "dgrad: slots x weights");

    __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS_BYTES];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
    const int wm = wave / WN, wn = wave % WN;
    const int half = lane >> 5;

    // ---- the tile: expert, then M-tile, then N-tile (innermost)
    int t = xcd_remap(blockIdx.x, gridDim.x);
    const int nt = t % p.NT;
    t /= p.NT;
    const int mt = t % p.MT;
    const int e = t / p.MT;
    const int m0 = mt * BMT, n0 = nt * BNT;
    const int seg = e * p.Cp, len = p.Cp;
    const int KT = (p.Kd + BK - 1) / BK;

    // ---- descriptors (everything outside them reads zeros)
    const uint32_t a_rowb = static_cast<uint32_t>(p.lda) * 2u;
    const uint32_t b_rowb = static_cast<uint32_t>(p.ldb) * 2u;
    const i32x4 ra = ASRC == kRowGather
        ? make_rsrc(p.a, static_cast<uint32_t>(p.N) * a_rowb)
        : make_rsrc(p.a + static_cast<int64_t>(seg) * p.lda, static_cast<uint32_t>(len) * a_rowb);
    const i32x4 rb = make_rsrc(p.b + static_cast<int64_t>(e) * p.b_estride, static_cast<uint32_t>(p.Kd) * b_rowb);

    // ---- DMA addressing.  Wave w's load i fills 1 KB block q = w + i*NW of
    // the stage: RPI rows, lane L at row RPI*q + L/CPR, physical chunk L%CPR,
    // i.e. the logical chunk the row's swizzle puts there.
    auto dma_row = [&](int rpi, int cpr, int i) { return rpi * (wave + i * NW) + lane / cpr; };

    // A rows (gathered or route) are fixed for the tile; row-major stages use
    // the forward's swizzle (chunk ^ (row/2) % 8)
    uint32_t a_fix[A_INST];
#pragma unroll
    for (int i = 0; i < A_INST; ++i) {
        const int r = dma_row(A_RPI, A_CPR, i);
        int row;
        if (ASRC == kRowGather) {
            const int tok = m0 + r < len ? p.sorted_slot_ids[seg + m0 + r] : p.N;
            row = static_cast<unsigned>(tok) < static_cast<unsigned>(p.N) ? tok : p.N;
        } else {
            row = m0 + r;
        }
        const int chunk = (lane % A_CPR) ^ ((r / (256 / AROWB)) % A_CPR);
        a_fix[i] = static_cast<uint32_t>(row) * a_rowb + chunk * 16u;
    }

    const uint32_t lds0 = lds_addr(smem);
    auto a_voff = [&](int i, int kt) -> uint32_t {
        return kt < KT ? a_fix[i] + static_cast<uint32_t>(kt) * AROWB : kOob;
    };
    // B (weights, K-major): chunk ^ 4*(row%4)
    auto b_voff = [&](int i, int kt) -> uint32_t {
        const int rr = dma_row(B_RPI, B_CPR, i);
        const int chunk = (lane % B_CPR) ^ (4 * (rr & 3));
        return kt < KT ? static_cast<uint32_t>(kt * BK + rr) * b_rowb + (n0 + chunk * 8) * 2u : kOob;
    };
    auto issue_a = [&](int i, int kt, int stage_off) {
        dma16(ra, a_voff(i, kt), lds0 + stage_off + (wave + i * NW) * 1024);
    };
    auto issue_b = [&](int i, int kt, int stage_off) {
        dma16<true>(rb, b_voff(i, kt), lds0 + B_RING + stage_off + (wave + i * NW) * 1024);
    };

    floatx16 acc[MI][NI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[mi][ni][j] = 0.0f;

    int a_read = 0, b_read = 0;
    int a_fill = (NA - 1) * A_STAGE, b_fill = (NB - 1) * B_STAGE;

    constexpr int LEAD = NA > NB ? NA : NB;
#pragma unroll
    for (int j = -(LEAD - 1); j < 0; ++j) {
        if (j + NA - 1 >= 0)
#pragma unroll
            for (int i = 0; i < A_INST; ++i) issue_a(i, j + NA - 1, (j + NA - 1) * A_STAGE);
        if (j + NB - 1 >= 0)
#pragma unroll
            for (int i = 0; i < B_INST; ++i) issue_b(i, j + NB - 1, (j + NB - 1) * B_STAGE);
    }

    constexpr int SLICES = BK / 16;
    for (int kt = 0; kt < KT; ++kt) {
        wait_vmcnt<WAIT>();
        __syncthreads();
        const lds_u8* sB = (const lds_u8*)smem + B_RING + b_read;
#pragma unroll
        for (int ks = 0; ks < SLICES; ++ks) {
            bf16x8 af[MI], bfr[NI];
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
                af[mi] = *reinterpret_cast<const bf16x8*>(
                    smem + a_read + lds_off<BK>(wm * WTM + mi * 32 + (lane & 31), ks * 2 + half));
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) {
                const int tn = wn * WTN + ni * 32;
                bfr[ni] = tr_frag(sB, tr_off<BROWB>(lane, tn, ks * 16, 0),
                                  tr_off<BROWB>(lane, tn, ks * 16, 1));
            }
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                for (int ni = 0; ni < NI; ++ni)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[ni], af[mi], acc[mi][ni], 0, 0, 0);
            // this slice's share of the refill: slabs kt+NA-1 and kt+NB-1
            // into the stages computed at step kt-1
#pragma unroll
            for (int q = ks * LOADS / SLICES; q < (ks + 1) * LOADS / SLICES; ++q) {
                if (q < A_INST) issue_a(q, kt + NA - 1, a_fill);
                else issue_b(q - A_INST, kt + NB - 1, b_fill);
            }
        }
        const int a = a_read, b = b_read;
        a_read = a + A_STAGE == NA * A_STAGE ? 0 : a + A_STAGE;
        b_read = b + B_STAGE == NB * B_STAGE ? 0 : b + B_STAGE;
        a_fill = a;
        b_fill = b;
    }

    // ---- epilogue: lane (row l&31, half h) holds columns 8g + 4h + (0..3)
    // of each 32-column block in acc[4g .. 4g+3]; bf16 and a swap of lane
    // halves give each lane 8 consecutive columns.  The workgroup's last
    // loads (past K: zeros into stages nobody reads) land first; then each
    // wave stages its WTM x WTN piece in its own part of the idle rings
    // (16-byte chunks swizzled by row) and writes it out in whole rows of
    // WTN*2 bytes (straight from the accumulators, one store would write
    // 32-byte pieces of 32 rows).  Rows and columns past the output get an
    // offset beyond the descriptor: the store is dropped.
    static_assert(NW * WTM * WTN * 2 <= LDS_BYTES, "staging fits the rings");
    constexpr int CPRO = WTN / 8;                  // 16-byte chunks per staged row
    wait_vmcnt<0>();
    __syncthreads();
    const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
        p.out + static_cast<int64_t>(seg) * p.ldo, static_cast<short>(0), len * p.ldo * 2, kRsrcWord3);
    typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
    lds_u8* st = (lds_u8*)smem + wave * (WTM * WTN * 2);
    auto so = [](int r, int c) { return static_cast<uint32_t>(r * (WTN * 2) + ((c ^ (r % CPRO)) << 4)); };
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
            uint32_t g[4][2];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                g[q][0] = pack_bf16x2(acc[mi][ni][4 * q], acc[mi][ni][4 * q + 1]);
                g[q][1] = pack_bf16x2(acc[mi][ni][4 * q + 2], acc[mi][ni][4 * q + 3]);
            }
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const auto s0 = __builtin_amdgcn_permlane32_swap(g[2 * q][0], g[2 * q + 1][0], false, false);
                const auto s1 = __builtin_amdgcn_permlane32_swap(g[2 * q][1], g[2 * q + 1][1], false, false);
                u32x4 d;
                d[0] = s0[0]; d[1] = s1[0]; d[2] = s0[1]; d[3] = s1[1];
                // columns ni*32 + 16q + 8*half of the wave's WTN
                *(lds_u32x4*)(st + so(mi * 32 + (lane & 31), ni * 4 + 2 * q + half)) = d;
            }
        }
    }
    // the wave reads back what its other lanes wrote: LDS operations of one
    // wave complete in order, and the clobbers keep the compiler from moving
    // them across
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int j = 0; j < WTM * CPRO / kWave; ++j) {
        const int r = j * (kWave / CPRO) + lane / CPRO, c = lane % CPRO;
        const u32x4 v = *(const lds_u32x4*)(st + so(r, c));
        const int row = m0 + wm * WTM + r, col = n0 + wn * WTN + c * 8;
        const uint32_t off = row < len && col < p.Nn ? (static_cast<uint32_t>(row) * p.ldo + col) * 2u : kOob;
        __builtin_amdgcn_raw_buffer_store_b128(v, orsrc, off, 0, 0);
    }
}

// ---- weight gradient.  dW[e][m, n] = sum over the expert's slots s of
// A[s, m] * B[s, n], both operands K-major (slot-indexed rows: the expert's
// segment of a route-ordered buffer, or the token rows the route list
// names).  The contraction is short (Cp slots: a few K slabs per tile) and
// every tile writes a large output (as many bytes as it reads), so:
//   * one persistent workgroup per CU walks its tiles (t, t + G, ...) with
//     the load rings running across tile boundaries;
//   * four producer waves issue the K-slab loads and eight consumer waves
//     run the MFMAs and the stores.  Vector-memory wait counters are per wave
//     and count stores too: the producers wait only on their loads and the
//     consumers never wait, so the dW stores drain while later slabs load
//     and compute.  Both kinds meet at one barrier per K step: after it the
//     step's slab is in LDS (the producers waited for it) and the stage
//     computed at the previous step is free;
//   * the bf16 output goes out in whole 128-byte lines, marked non-temporal:
//     a consumer stages each 32-row block of its piece in LDS and 8 lanes
//     then write one row's 128 bytes (stored straight from the accumulator
//     layout, one instruction would write 32-byte quarters of 32 lines;
//     streamed partial lines are far slower than whole ones);
//   * ACC32: the tile is added into the float32 main gradient out32 instead
//     ([PF] section 5, in-kernel main-gradient accumulation): each lane reads
//     its 4 consecutive columns of a row (16 bytes), adds its float32 sums
//     and writes them back, default cache policy, so the four quarters of a
//     128-byte line that neighbouring instructions touch meet in L2.  The
//     tile's one owner reads and writes every element once: no atomics, and
//     the result does not depend on the schedule.
template <int ASRC, int BSRC, bool ACC32 = false>
__global__ __launch_bounds__(768) void wgrad_kernel(BwdArgs p) {
    constexpr int BMT = 256, BNT = 256, WM = 2, WN = 4, BK = 64, D = 2;
    constexpr int NC = WM * WN;                    // consumer waves
    constexpr int NP = 4;                          // producer waves
    constexpr int WTM = BMT / WM, WTN = BNT / WN;
    constexpr int MI = WTM / 32, NI = WTN / 32;
    constexpr int ROWB = BMT * 2;                  // bytes of a staged slot row (both operands)
    constexpr int STAGE = BK * ROWB;
    constexpr int RPI = 1024 / ROWB;               // slot rows per 1 KB DMA load
    constexpr int CPR = ROWB / 16;                 // 16-byte chunks per staged row
    constexpr int INST = STAGE / 1024 / NP;        // DMA loads per producer per operand and slab
    constexpr int B_RING = D * STAGE;
    constexpr int RINGS = 2 * D * STAGE;
    constexpr int SBLK = 32 * WTN * 2;             // a consumer's staged 32-row block
    constexpr int LDS_BYTES = RINGS + NC * SBLK;
    constexpr int SLICES = BK / 16;
    // a producer's loads issued after slab g+1's, when it waits for that slab
    constexpr int WAIT = (D - 2) * 2 * INST;
    static_assert(BMT == BNT && RPI == 2 && INST >= 1 && D >= 2, "tile shape");
    static_assert(WAIT < 64, "wait counts");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");
    static_assert(ASRC != kRowWeight && BSRC != kRowWeight, "wgrad rows are slots");

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
        // ---------------- producer: loads 1 KB blocks q = pw + i*NP of each stage
        const int pw = wave - NC;
        const int E = p.tiles / (p.MT * p.NT);
        const uint32_t a_rowb = static_cast<uint32_t>(p.lda) * 2u;
        const uint32_t b_rowb = static_cast<uint32_t>(p.ldb) * 2u;
        struct Ptr {
            int t, kt, e, c0;
            i32x4 r;
            int tok[INST][2];
        };
        auto place = [&](Ptr& d, bool is_a) {
            const int nt = d.t % p.NT, rest = d.t / p.NT;
            d.e = rest / p.MT;
            d.c0 = is_a ? (rest % p.MT) * BMT : nt * BNT;
            const int src = is_a ? ASRC : BSRC;
            const uint16_t* base = is_a ? p.a : p.b;
            const uint32_t rowb = is_a ? a_rowb : b_rowb;
            d.r = src == kRowGather
                ? make_rsrc(base, static_cast<uint32_t>(p.N) * rowb)
                : make_rsrc(base + static_cast<int64_t>(min(d.e, E - 1)) * p.Cp * (rowb / 2),
                            static_cast<uint32_t>(len) * rowb);
        };
        auto fetch_tokens = [&](Ptr& d, int src) {
            if (src != kRowGather) return;
            const bool live = d.t < p.tiles;
#pragma unroll
            for (int i = 0; i < INST; ++i) {
                const int base = d.kt * BK + RPI * (pw + i * NP);
                if (live && base < len) {
                    const const_int_ptr q = (const_int_ptr)(p.sorted_slot_ids) + static_cast<int64_t>(d.e) * p.Cp + base;
                    d.tok[i][0] = q[0];
                    d.tok[i][1] = q[1];
                } else {
                    d.tok[i][0] = d.tok[i][1] = -1;
                }
            }
        };
        auto advance = [&](Ptr& d, bool is_a, int src) {
            if (++d.kt == KT) {
                d.kt = 0;
                d.t += G;
                place(d, is_a);
            }
            fetch_tokens(d, src);
        };
        auto voff = [&](const Ptr& d, int src, uint32_t rowb, int i) -> uint32_t {
            const int rr = RPI * (pw + i * NP) + lane / CPR;          // row within the stage
            const int slot = d.kt * BK + rr;
            int row;
            if (src == kRowGather) {
                const int tok = half ? d.tok[i][1] : d.tok[i][0];
                row = static_cast<unsigned>(tok) < static_cast<unsigned>(p.N) ? tok : -1;
            } else {
                row = d.t < p.tiles && slot < len ? slot : -1;
            }
            const int chunk = (lane % CPR) ^ (4 * (rr & 3));
            return row < 0 ? kOob : static_cast<uint32_t>(row) * rowb + (d.c0 + chunk * 8) * 2u;
        };
        const uint32_t lds0 = lds_addr(smem);
        auto issue_slab = [&](Ptr& pa, Ptr& pb, int stage_off) {
#pragma unroll
            for (int i = 0; i < INST; ++i)
                dma16(pa.r, voff(pa, ASRC, a_rowb, i), lds0 + stage_off + (pw + i * NP) * 1024);
#pragma unroll
            for (int i = 0; i < INST; ++i)
                dma16(pb.r, voff(pb, BSRC, b_rowb, i), lds0 + B_RING + stage_off + (pw + i * NP) * 1024);
            advance(pa, true, ASRC);
            advance(pb, false, BSRC);
        };
        Ptr pa, pb;
        pa.t = pb.t = t0;
        pa.kt = pb.kt = 0;
        place(pa, true);
        place(pb, false);
        fetch_tokens(pa, ASRC);
        fetch_tokens(pb, BSRC);
#pragma unroll
        for (int j = 0; j < D - 1; ++j) issue_slab(pa, pb, j * STAGE);   // slabs 0 .. D-2
        wait_vmcnt<WAIT>();                                             // slab 0 is in
        __syncthreads();
        int fill = (D - 1) * STAGE;
        for (int g = 0; g < S; ++g) {
            issue_slab(pa, pb, fill);                                   // slab g+D-1
            fill = fill + STAGE == D * STAGE ? 0 : fill + STAGE;        // slab g's stage, free next step
            wait_vmcnt<WAIT>();                                         // slab g+1 is in
            __syncthreads();
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
    int tc = t0, ktc = 0, rd = 0;
    for (int g = 0; g < S; ++g) {
        const lds_u8* sA = (const lds_u8*)smem + rd;
        const lds_u8* sB = (const lds_u8*)smem + B_RING + rd;
#pragma unroll
        for (int ks = 0; ks < SLICES; ++ks) {
            bf16x8 af[MI], bfr[NI];
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
                af[mi] = tr_frag(sA, tr_off<ROWB>(lane, wm * WTM + mi * 32, ks * 16, 0),
                                 tr_off<ROWB>(lane, wm * WTM + mi * 32, ks * 16, 1));
#pragma unroll
            for (int ni = 0; ni < NI; ++ni)
                bfr[ni] = tr_frag(sB, tr_off<ROWB>(lane, wn * WTN + ni * 32, ks * 16, 0),
                                  tr_off<ROWB>(lane, wn * WTN + ni * 32, ks * 16, 1));
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                for (int ni = 0; ni < NI; ++ni)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[ni], af[mi], acc[mi][ni], 0, 0, 0);
        }
        rd = rd + STAGE == D * STAGE ? 0 : rd + STAGE;
        if (++ktc == KT) {
            // the tile is done: lane (row l&31, half h) holds columns
            // 8g + 4h + (0..3) of each 32-column block in acc[4g..4g+3]; a
            // swap of lane halves gives each lane 8 consecutive columns
            const int nt = tc % p.NT, rest = tc / p.NT;
            const int e = rest / p.MT;
            const int row0 = (rest % p.MT) * BMT + wm * WTM, col0 = nt * BNT + wn * WTN;
            if constexpr (ACC32) {
                const __amdgpu_buffer_rsrc_t mrsrc = __builtin_amdgcn_make_buffer_rsrc(
                    p.out32 + static_cast<int64_t>(e) * p.o_estride, static_cast<short>(0), p.M * p.ldo * 4,
                    kRsrcWord3);
                const int orow = row0 + (lane & 31);
#pragma unroll
                for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                    for (int ni = 0; ni < NI; ++ni) {
                        uint32_t off[4];
                        u32x4 old[4];
#pragma unroll
                        for (int g = 0; g < 4; ++g) {
                            const int r = orow + mi * 32, col = col0 + ni * 32 + 8 * g + 4 * half;
                            off[g] = r < p.M && col < p.Nn ? (static_cast<uint32_t>(r) * p.ldo + col) * 4u : kOob;
                            old[g] = __builtin_amdgcn_raw_buffer_load_b128(mrsrc, off[g], 0, 0);
                        }
#pragma unroll
                        for (int g = 0; g < 4; ++g) {
                            u32x4 v;
#pragma unroll
                            for (int j = 0; j < 4; ++j)
                                v[j] = __float_as_uint(__uint_as_float(old[g][j]) + acc[mi][ni][4 * g + j]);
                            __builtin_amdgcn_raw_buffer_store_b128(v, mrsrc, off[g], 0, 0);
                        }
#pragma unroll
                        for (int j = 0; j < 16; ++j) acc[mi][ni][j] = 0.0f;
                    }
            } else {
            const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
                p.out + static_cast<int64_t>(e) * p.o_estride, static_cast<short>(0), p.M * p.ldo * 2, kRsrcWord3);
            // Each 32-row block goes through this wave's LDS block (16-byte
            // chunks swizzled by row, so 8 consecutive rows hit distinct
            // banks), then out at 8 lanes per 128-byte row piece.  The wave
            // reads back what its other lanes wrote: LDS operations of one
            // wave complete in order, and the clobbers keep the compiler from
            // moving them across.
            lds_u8* st = (lds_u8*)smem + RINGS + wave * SBLK;
            auto so = [](int r, int c) { return static_cast<uint32_t>(r * (WTN * 2) + ((c ^ (r & 7)) << 4)); };
#pragma unroll
            for (int mi = 0; mi < MI; ++mi) {
                asm volatile("" ::: "memory");
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
                        *(__attribute__((address_space(3))) u32x4*)(st + so(lane & 31, ni * 4 + 2 * q + half)) = d;
                    }
#pragma unroll
                    for (int j = 0; j < 16; ++j) acc[mi][ni][j] = 0.0f;
                }
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                constexpr int CPRO = WTN / 8;              // 16-byte chunks per output row piece
#pragma unroll
                for (int j = 0; j < 32 * CPRO / kWave; ++j) {
                    const int r = j * (kWave / CPRO) + lane / CPRO, c = lane % CPRO;
                    const u32x4 v = *(const __attribute__((address_space(3))) u32x4*)(st + so(r, c));
                    const int orow = row0 + mi * 32 + r, col = col0 + c * 8;
                    const uint32_t off = orow < p.M && col < p.Nn
                        ? (static_cast<uint32_t>(orow) * p.ldo + col) * 2u : kOob;
                    __builtin_amdgcn_raw_buffer_store_b128(v, orsrc, off, 0, kStoreNT);
                }
                asm volatile("" ::: "memory");
            }
            }
            ktc = 0;
            tc += G;
        }
        __syncthreads();
    }
}

template <int ASRC>
int launch_dgrad(BwdArgs a, int E, hipStream_t s) {
    constexpr int BMT = 256, BNT = 256, WM = 2, WN = 4, BK = 64, NA = 2, NB = 3;
    a.MT = (a.Cp + BMT - 1) / BMT;
    a.NT = (a.Nn + BNT - 1) / BNT;
    const int64_t tiles = static_cast<int64_t>(E) * a.MT * a.NT;
    if (tiles > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    a.tiles = static_cast<int>(tiles);
    dgrad_kernel<BMT, BNT, WM, WN, BK, NA, NB, ASRC><<<a.tiles, WM * WN * kWave, 0, s>>>(a);
    return MOE_OK;
}

// FC1 dgrad (A = the route-ordered d_preact) runs on the producer/consumer
// slot GEMM: the same tiles and K order as dgrad_kernel, the same results bit
// for bit, about 10% faster at the Qwen3-30B-A3B shape (the FC2 dgrad, whose
// gathered dy rows would need per-tile token loads in the producers, stays on
// dgrad_kernel).
int launch_fc1_dgrad(const BwdArgs& a, int E, hipStream_t s) {
    SlotArgs sa{};
    sa.a = a.a; sa.b = a.b; sa.out = a.out;
    sa.lda = a.lda; sa.ldb = a.ldb; sa.ldo = a.ldo;
    sa.Nn = a.Nn; sa.Kd = a.Kd; sa.Cp = a.Cp;
    sa.MT = (a.Cp + 255) / 256;
    sa.NT = (a.Nn + 255) / 256;
    const int64_t tiles = static_cast<int64_t>(E) * sa.MT * sa.NT;
    if (tiles > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    sa.tiles = static_cast<int>(tiles);
    sa.b_estride = a.b_estride;
    sa.krot = 0;
    slot_gemm_kernel<true><<<std::min(sa.tiles, device_cus()), 12 * kWave, 0, s>>>(sa);
    return MOE_OK;
}

template <int ASRC, int BSRC, bool ACC32 = false>
int launch_wgrad(BwdArgs a, int E, hipStream_t s) {
    constexpr int BT = 256;                        // square output tiles
    a.MT = (a.M + BT - 1) / BT;
    a.NT = (a.Nn + BT - 1) / BT;
    const int64_t tiles = static_cast<int64_t>(E) * a.MT * a.NT;
    if (tiles > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    a.tiles = static_cast<int>(tiles);
    // one workgroup (8 consumer + 4 producer waves, all of LDS) per CU
    wgrad_kernel<ASRC, BSRC, ACC32><<<std::min(a.tiles, device_cus()), 12 * kWave, 0, s>>>(a);
    return MOE_OK;
}

// Host checks shared by the backward GEMM entry points (the forward's
// envelope; 32-bit buffer offsets inside the kernels).
int check_bwd(int64_t N, int32_t H, int32_t I, int32_t E, int64_t C, int* Cp) {
    if (N < 0 || E < 1 || C < 0) return MOE_ERR_INVALID_ARG;
    int st = check_dims(H, I);
    if (st != MOE_OK) return st;
    if (N > kMaxN || E > kMaxE) return MOE_ERR_UNSUPPORTED;
    const int64_t Cp64 = moe_padded_capacity(C);
    if (Cp64 < 0) return MOE_ERR_UNSUPPORTED;
    const int64_t big = static_cast<int64_t>(1) << 31;
    if (static_cast<int64_t>(E) * Cp64 > INT32_MAX || (N + 1) * H * 2 >= big ||
        Cp64 * std::max(H, 2 * I) * 2 >= big || static_cast<int64_t>(2) * I * H * 2 >= big)
        return MOE_ERR_UNSUPPORTED;
    *Cp = static_cast<int>(Cp64);
    return MOE_OK;
}

int check_ptrs16(std::initializer_list<const void*> ptrs) {
    for (const void* q : ptrs) {
        if (!q) return MOE_ERR_INVALID_ARG;
        if (!aligned16(q)) return MOE_ERR_MISALIGNED;
    }
    return MOE_OK;
}

}  // namespace
}  // namespace moe

extern "C" int moe_grouped_fc2_dgrad(const uint16_t* dy, const uint16_t* w2,
                                     const int32_t* sorted_slot_ids, int64_t N, int32_t H,
                                     int32_t I, int32_t E, int64_t C, uint16_t* d_act,
                                     hipStream_t stream) {
    using namespace moe;
    int Cp = 0;
    int st = check_bwd(N, H, I, E, C, &Cp);
    if (st != MOE_OK) return st;
    if (N == 0 || C == 0) return MOE_OK;
    st = check_ptrs16({dy, w2, sorted_slot_ids, d_act});
    if (st != MOE_OK) return st;
    BwdArgs a{};
    a.a = dy; a.b = w2; a.sorted_slot_ids = sorted_slot_ids; a.out = d_act;
    a.lda = H; a.ldb = I; a.ldo = I; a.N = static_cast<int>(N);
    a.M = Cp; a.Nn = I; a.Kd = H; a.Cp = Cp;
    a.b_estride = static_cast<int64_t>(H) * I;
    st = launch_dgrad<kRowGather>(a, E, stream);
    return st != MOE_OK ? st : launch_status();
}

extern "C" int moe_grouped_fc1_dgrad(const uint16_t* d_preact, const uint16_t* w1, int64_t N,
                                     int32_t H, int32_t I, int32_t E, int64_t C, uint16_t* d_a,
                                     hipStream_t stream) {
    using namespace moe;
    int Cp = 0;
    int st = check_bwd(N, H, I, E, C, &Cp);
    if (st != MOE_OK) return st;
    if (N == 0 || C == 0) return MOE_OK;
    st = check_ptrs16({d_preact, w1, d_a});
    if (st != MOE_OK) return st;
    BwdArgs a{};
    a.a = d_preact; a.b = w1; a.out = d_a;
    a.lda = 2 * I; a.ldb = H; a.ldo = H; a.N = static_cast<int>(N);
    a.M = Cp; a.Nn = H; a.Kd = 2 * I; a.Cp = Cp;
    a.b_estride = static_cast<int64_t>(2) * I * H;
    st = launch_fc1_dgrad(a, E, stream);
    return st != MOE_OK ? st : launch_status();
}

extern "C" int moe_grouped_fc2_wgrad(const uint16_t* dy, const uint16_t* act,
                                     const int32_t* sorted_slot_ids, int64_t N, int32_t H,
                                     int32_t I, int32_t E, int64_t C, uint16_t* dw2,
                                     hipStream_t stream) {
    using namespace moe;
    int Cp = 0;
    int st = check_bwd(N, H, I, E, C, &Cp);
    if (st != MOE_OK) return st;
    if (N == 0 || C == 0) return MOE_OK;   // nothing routed: dW2 is left as it was
    st = check_ptrs16({dy, act, sorted_slot_ids, dw2});
    if (st != MOE_OK) return st;
    BwdArgs a{};
    a.a = dy; a.b = act; a.sorted_slot_ids = sorted_slot_ids; a.out = dw2;
    a.lda = H; a.ldb = I; a.ldo = I; a.N = static_cast<int>(N);
    a.M = H; a.Nn = I; a.Kd = Cp; a.Cp = Cp;
    a.o_estride = static_cast<int64_t>(H) * I;
    st = launch_wgrad<kRowGather, kRowRoute>(a, E, stream);
    return st != MOE_OK ? st : launch_status();
}

extern "C" int moe_grouped_fc1_wgrad(const uint16_t* d_preact, const uint16_t* x,
                                     const int32_t* sorted_slot_ids, int64_t N, int32_t H,
                                     int32_t I, int32_t E, int64_t C, uint16_t* dw1,
                                     hipStream_t stream) {
    using namespace moe;
    int Cp = 0;
    int st = check_bwd(N, H, I, E, C, &Cp);
    if (st != MOE_OK) return st;
    if (N == 0 || C == 0) return MOE_OK;
    st = check_ptrs16({d_preact, x, sorted_slot_ids, dw1});
    if (st != MOE_OK) return st;
    BwdArgs a{};
    a.a = d_preact; a.b = x; a.sorted_slot_ids = sorted_slot_ids; a.out = dw1;
    a.lda = 2 * I; a.ldb = H; a.ldo = H; a.N = static_cast<int>(N);
    a.M = 2 * I; a.Nn = H; a.Kd = Cp; a.Cp = Cp;
    a.o_estride = static_cast<int64_t>(2) * I * H;
    st = launch_wgrad<kRowRoute, kRowGather>(a, E, stream);
    return st != MOE_OK ? st : launch_status();
}

// Float32 main-gradient forms: the same tiles, K order and float32 sums as
// the bf16 entry points above, added into main_dw (see ACC32).
namespace moe {
namespace {

int check_main(int32_t H, int32_t I) {
    // one expert's float32 dW must lie within a buffer descriptor's 2 GiB
    const int64_t big = static_cast<int64_t>(1) << 31;
    return static_cast<int64_t>(2) * I * H * 4 >= big ? MOE_ERR_UNSUPPORTED : MOE_OK;
}

}  // namespace
}  // namespace moe

extern "C" int moe_grouped_fc2_wgrad_accum(const uint16_t* dy, const uint16_t* act,
                                           const int32_t* sorted_slot_ids, int64_t N, int32_t H,
                                           int32_t I, int32_t E, int64_t C, float* main_dw2,
                                           hipStream_t stream) {
    using namespace moe;
    int Cp = 0;
    int st = check_bwd(N, H, I, E, C, &Cp);
    if (st == MOE_OK) st = check_main(H, I);
    if (st != MOE_OK) return st;
    if (N == 0 || C == 0) return MOE_OK;   // nothing routed: the sums are zero
    st = check_ptrs16({dy, act, sorted_slot_ids, main_dw2});
    if (st != MOE_OK) return st;
    BwdArgs a{};
    a.a = dy; a.b = act; a.sorted_slot_ids = sorted_slot_ids; a.out32 = main_dw2;
    a.lda = H; a.ldb = I; a.ldo = I; a.N = static_cast<int>(N);
    a.M = H; a.Nn = I; a.Kd = Cp; a.Cp = Cp;
    a.o_estride = static_cast<int64_t>(H) * I;
    st = launch_wgrad<kRowGather, kRowRoute, true>(a, E, stream);
    return st != MOE_OK ? st : launch_status();
}

extern "C" int moe_grouped_fc1_wgrad_accum(const uint16_t* d_preact, const uint16_t* x,
                                           const int32_t* sorted_slot_ids, int64_t N, int32_t H,
                                           int32_t I, int32_t E, int64_t C, float* main_dw1,
                                           hipStream_t stream) {
    using namespace moe;
    int Cp = 0;
    int st = check_bwd(N, H, I, E, C, &Cp);
    if (st == MOE_OK) st = check_main(H, I);
    if (st != MOE_OK) return st;
    if (N == 0 || C == 0) return MOE_OK;
    st = check_ptrs16({d_preact, x, sorted_slot_ids, main_dw1});
    if (st != MOE_OK) return st;
    BwdArgs a{};
    a.a = d_preact; a.b = x; a.sorted_slot_ids = sorted_slot_ids; a.out32 = main_dw1;
    a.lda = 2 * I; a.ldb = H; a.ldo = H; a.N = static_cast<int>(N);
    a.M = 2 * I; a.Nn = H; a.Kd = Cp; a.Cp = Cp;
    a.o_estride = static_cast<int64_t>(2) * I * H;
    st = launch_wgrad<kRowRoute, kRowGather, true>(a, E, stream);
    return st != MOE_OK ? st : launch_status();
}
