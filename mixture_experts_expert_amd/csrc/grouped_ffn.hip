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
//   * 256x256 tiles over (expert, M-tile, N-tile); the M-tile spans an
//     expert's whole capacity (up to 256 slots, 320 in the dropless form) so
//     its weight panel is streamed from HBM once;
//   * persistent workgroups (one per resident slot) walk the tiles, and the
//     LDS load rings run across tile boundaries: the last K steps of a tile
//     already fetch the first slabs of the workgroup's next tile;
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
//     N-tiles, sharing the gathered A rows) land on the same XCD and its L2;
//   * 256x256 tiles leave through a staged epilogue: the tile is written
//     into the two LDS stages its last K step freed and goes out in whole
//     128-byte lines, which disturbs the load stream far less than 32-byte
//     pieces straight from the accumulator layout;
//   * FC2 with an output row map (an expert-parallel rank's return layout)
//     runs on the producer/consumer slot GEMM (slot_gemm.h).
#include <algorithm>
#include <atomic>
#include <cmath>
#include <initializer_list>

#include "gemm_common.h"
#include "slot_gemm.h"

namespace moe {
namespace {

constexpr int kKRotate = 5;      // K slabs between the starting slabs of consecutive experts

struct FfnArgs {
    const uint16_t* a;            // FC1: x [N, H];   FC2: act [E*Cp, I]
    const uint16_t* w;            // FC1: w1 [E, 2I, H]; FC2: w2 [E, H, I]
    const int* sorted_slot_ids;   // FC1 only
    const float* slot_probs;      // FC1 only
    uint16_t* out;                // FC1: act [E*Cp, I]; FC2: route_out [E*Cp, H]
    uint16_t* preact;             // FC1 only, may be null: raw [gate | up] [E*Cp, 2I]
    int N;                        // tokens (FC1 sentinel row)
    int Kdim;                     // contraction length: FC1 H, FC2 I
    int ncols;                    // output columns: FC1 I, FC2 H
    int wrows;                    // weight rows per expert: FC1 2I, FC2 H
    int Cp;                       // slots per expert
    int MT, NT;                   // M-tiles per expert, N-tiles per expert
    int tiles;                    // E * MT * NT (fixed segments)
    // Variable segments (the dropless route list): expert e owns the slots
    // [block_start[e]*BM, block_start[e+1]*BM) (the last one ends at the
    // extent); the tile count follows from these device values.
    const int* block_start;
    const int* extent;
    int E;
    int R;                        // slots of the route list (its static bound)
};

// One persistent workgroup per resident slot walks the tiles r*G + slot
// (G workgroups, slot = the XCD-aware renumbering of its id), with one
// continuous pair of LDS rings: the last steps of a tile already stream the
// first K slabs of the block's next tile, so HBM keeps streaming across tile
// boundaries and the epilogue (registers -> global, no LDS) overlaps them.
//
// Accumulators hold C transposed (the MFMA takes the weight fragment as its
// first operand): a lane owns one output row (slot) and 16 output columns in
// runs of 4, so SwiGLU pairs and the routing probability live in the lane and
// a swap of lane halves leaves 8 consecutive bf16 columns per lane for one
// 16-byte store.
template <int BMT, int BNT, int WM, int WN, int BK, int NA, int NB, bool FC1, bool DYN,
          bool SAVE = false, int EPI = 0>
__global__ __launch_bounds__(WM * WN * kWave) void ffn_gemm_kernel(FfnArgs p) {
    constexpr int NW = WM * WN;
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
    constexpr int OUT_COLS = FC1 ? BNT / 2 : BNT;          // output columns of a tile
    // 16-byte stores per lane per tile (FC1 with SAVE also stores the raw
    // gate and up columns, the pre-activation the backward keeps)
    constexpr int STORES = FC1 ? (SAVE ? 3 : 1) * MI * NI : 2 * MI * NI;
    static_assert(FC1 || !SAVE, "only FC1 has a pre-activation");
    constexpr int LDS_BYTES = NA * A_STAGE + NB * B_STAGE;
    // Step j issues A(j+NA-1) then B(j+NB-1); vector-memory operations retire
    // in issue order.  Before computing slab kt, the newer of A(kt) and B(kt)
    // must have landed: A(kt) if NA < NB (then B(kt+NB-NA) of the same step and
    // NA-2 whole steps follow it), else B(kt) (NB-2 whole steps follow it).  At
    // the first step of every tile but the block's first, the previous tile's
    // STORES epilogue stores were issued after the current slab's loads too.
    constexpr int WAIT = NA < NB ? B_INST + (NA - 2) * LOADS : (NB - 2) * LOADS;
    static_assert(MI >= 1 && NI >= 1, "tile too small");
    static_assert(BK == 32 || BK == 64, "K slab");
    static_assert(A_INST >= 1 && B_INST >= 1 && BMT % (RPI * NW) == 0 && BNT % (RPI * NW) == 0,
                  "whole DMA blocks per wave");
    static_assert(NA >= 2 && NB >= 2 && WAIT + STORES < 64, "stage rings");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");
    // Staged epilogue (EPI 1: default store policy, 2: non-temporal): the
    // tile leaves through the A and B stages its last K step freed.  FC1
    // stages its 128-column tile as many rows at a time as they hold (all
    // 256 rows of a 256-row tile; 288 then 32 of a 320-row one, though the
    // launcher keeps that shape on direct stores); FC2 gives each wave 8 KB
    // of them for its piece, 64 rows at a time.
    static_assert(EPI == 0 || ((BMT == 256 || BMT == 320) && BNT == 256 && BK == 64 && WM == 2 && WN == 4),
                  "staged epilogue shape");
    static_assert(!DYN || LDS_BYTES >= (3 * kMaxE + 1) * 4, "room for the tile list");

    __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS_BYTES];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
    const int wm = wave / WN, wn = wave % WN;
    const int half = lane >> 5;                             // 0: lanes 0-31, 1: lanes 32-63
    const int KT = p.Kdim / BK;                             // >= max(NA, NB - 1) (host)
    const uint32_t row_bytes = static_cast<uint32_t>(p.Kdim) * 2u;
    const int G = gridDim.x;

    // ---- DMA addressing.  Wave w's load i covers the RPI tile rows of block
    // q = w + i*NW; lane L brings row RPI*q + L/CPR, physical chunk L%CPR,
    // i.e. the logical chunk that the swizzle of that row puts there.
    const int lrow = lane / CPR;
    auto dma_row = [&](int i) { return RPI * (wave + i * NW) + lrow; };
    auto dma_chunk = [&](int i) -> uint32_t {
        return static_cast<uint32_t>(((lane % CPR) ^ ((dma_row(i) / (256 / ROWB)) % CPR)) * 16);
    };

    struct Tile {
        int e, m0, nt;
        int seg, len;                 // the expert's first slot and its slot count
        int rot;                      // first K slab: tiles walk K cyclically from here
        i32x4 ra, rb;                 // per-expert descriptors (FC2's A and the weights)
        uint32_t av[A_INST], bv[B_INST];
    };
    // FC1's A descriptor covers all of x, whatever the tile
    const i32x4 x_rsrc = make_rsrc(p.a, FC1 ? static_cast<uint32_t>(p.N) * row_bytes : 0u);
    // Every expert walks its K slabs from its own starting slab.  Weight rows
    // are often a power of two bytes apart; if every workgroup fetched the same
    // K offset at once, all requests would share their low address bits and
    // crowd onto few HBM channels.  The tiles of one expert keep one start so
    // that they still share the gathered A slabs in L2.
    auto decode = [&](int t, Tile& d) {
        d.nt = t % p.NT;
        t /= p.NT;
        d.m0 = (t % p.MT) * BMT;
        d.e = t / p.MT;
        d.rot = (d.e * kKRotate) % KT;
        d.seg = d.e * p.Cp;
        d.len = p.Cp;
    };
    // ---- variable segments.  Tiles are numbered expert by expert and, within
    // an expert, column tile by column tile with the row tiles innermost, so
    // the row tiles of one weight panel run side by side (consecutive tiles
    // share an XCD) and read it from L2 together.  The block starts are device
    // data: segments are clamped to the route list, never trusted.
    typedef const __attribute__((address_space(4))) int* const_int_ptr;
    const const_int_ptr bs = (const_int_ptr)(p.block_start);
    int extent_slots = 0;
    auto seg_lo = [&](int v) { return min(max(v, 0), p.R / kBlockM) * kBlockM; };
    auto tiles_of = [&](int len) { return (len + BMT - 1) / BMT * p.NT; };
    auto set_tile = [&](Tile& d, int e, int nt, int mi, int seg, int len) {
        d.e = e;
        d.nt = nt;
        d.m0 = mi * BMT;
        d.rot = (e * kKRotate) % KT;
        d.seg = seg;
        d.len = len;
    };
    // Lane k of every wave holds the workgroup's k-th tile (t0 + k*G), built
    // once before the loads start: expert (-1 past the last tile), column
    // tile | row tile << 16, segment start, segment length.
    int lt_e = -1, lt_ntm = 0, lt_seg = 0, lt_len = 0;
    // Past 64 tiles a cursor walks the experts in the same numbering,
    // reading the block starts through the scalar cache.
    int cur_e = -1, t_before = 0, cur_start = 0, cur_len = 0;
    auto find = [&](int k, int t, Tile& d) -> bool {   // the k-th tile t, or false past the last
        if (k < kWave) {
            const int e = __builtin_amdgcn_readlane(lt_e, k);
            if (e < 0) return false;
            const int ntm = __builtin_amdgcn_readlane(lt_ntm, k);
            set_tile(d, e, ntm & 0xffff, ntm >> 16, __builtin_amdgcn_readlane(lt_seg, k),
                     __builtin_amdgcn_readlane(lt_len, k));
            return true;
        }
        while (cur_e < p.E && (cur_e < 0 || t >= t_before + tiles_of(cur_len))) {
            if (cur_e >= 0) t_before += tiles_of(cur_len);
            ++cur_e;
            if (cur_e < p.E) {
                cur_start = seg_lo(bs[cur_e]);
                const int hi = cur_e + 1 < p.E ? seg_lo(bs[cur_e + 1]) : extent_slots;
                cur_len = max(hi - cur_start, 0);
            }
        }
        if (cur_e >= p.E) return false;
        const int r = t - t_before, mt = (cur_len + BMT - 1) / BMT;
        set_tile(d, cur_e, r / mt, r % mt, cur_start, cur_len);
        return true;
    };
    auto kslab = [&](const Tile& d, int kt) {   // the K slab a tile fetches at its step kt
        const int k = kt + d.rot;
        return k < KT ? k : k - KT;
    };
    // Weight rows (and FC2's activation rows) follow from the tile alone.
    auto address_fixed = [&](Tile& d) {
        d.rb = make_rsrc(p.w + static_cast<int64_t>(d.e) * p.wrows * p.Kdim,
                         static_cast<uint32_t>(p.wrows) * row_bytes);
#pragma unroll
        for (int i = 0; i < B_INST; ++i) {
            const int R = dma_row(i);                       // tile row
            int wrow;
            if (FC1) {
                // FC1's B tile interleaves 16 gate rows and the 16 matching up
                // rows in each 32-row MFMA block, so one accumulator block
                // carries both.
                const int w = R & 31;
                wrow = (w < 16 ? 0 : p.ncols) + d.nt * (BNT / 2) + (R >> 5) * 16 + (w & 15);
            } else {
                wrow = d.nt * BNT + R;
            }
            d.bv[i] = static_cast<uint32_t>(wrow) * row_bytes + dma_chunk(i);
        }
        if (!FC1) {
            // rows past Cp lie outside the expert's descriptor and read zeros
            d.ra = make_rsrc(p.a + static_cast<int64_t>(d.seg) * p.Kdim,
                             static_cast<uint32_t>(d.len) * row_bytes);
#pragma unroll
            for (int i = 0; i < A_INST; ++i)
                d.av[i] = static_cast<uint32_t>(d.m0 + dma_row(i)) * row_bytes + dma_chunk(i);
        }
    };
    // FC1's A rows are the tokens the route list names for the tile's slots.
    auto load_tokens = [&](const Tile& d, int (&tok)[A_INST]) {
        const int64_t slot0 = static_cast<int64_t>(d.seg) + d.m0;
#pragma unroll
        for (int i = 0; i < A_INST; ++i)
            tok[i] = d.m0 + dma_row(i) < d.len ? p.sorted_slot_ids[slot0 + dma_row(i)] : p.N;
    };
    auto address_a = [&](Tile& d, const int (&tok)[A_INST]) {
#pragma unroll
        for (int i = 0; i < A_INST; ++i) {
            // the sentinel row N lies outside the descriptor and reads zeros
            const int row = static_cast<unsigned>(tok[i]) < static_cast<unsigned>(p.N) ? tok[i] : p.N;
            d.av[i] = static_cast<uint32_t>(row) * row_bytes + dma_chunk(i);
        }
    };
    // A block with no next tile still issues its look-ahead loads (so every
    // wait counts the same operations), at an offset beyond every descriptor:
    // they read zeros into stages that are never computed.
    auto address_none = [&](Tile& d) {
        d.ra = make_rsrc(p.a, 0);
        d.rb = make_rsrc(p.w, 0);
#pragma unroll
        for (int i = 0; i < A_INST; ++i) d.av[i] = kOob;
#pragma unroll
        for (int i = 0; i < B_INST; ++i) d.bv[i] = kOob;
    };

    const uint32_t lds0 = lds_addr(smem);
    auto issue_a = [&](const Tile& d, int stage_off, int kt) {
        const uint32_t koff = static_cast<uint32_t>(kslab(d, kt)) * ROWB;
        const uint32_t st = lds0 + stage_off;
#pragma unroll
        for (int i = 0; i < A_INST; ++i) dma16(FC1 ? x_rsrc : d.ra, d.av[i] + koff, st + (wave + i * NW) * 1024);
    };
    auto issue_b = [&](const Tile& d, int stage_off, int kt) {
        const uint32_t koff = static_cast<uint32_t>(kslab(d, kt)) * ROWB;
        const uint32_t st = lds0 + B_RING + stage_off;
#pragma unroll
        for (int i = 0; i < B_INST; ++i) dma16<true>(d.rb, d.bv[i] + koff, st + (wave + i * NW) * 1024);
    };

    floatx16 acc[MI][NI];
    auto zero_acc = [&]() {
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < NI; ++ni)
#pragma unroll
                for (int j = 0; j < 16; ++j) acc[mi][ni][j] = 0.0f;
    };
    // Byte offsets (within each ring) of the stage the current step computes
    // and of the stage it refills -- the one the previous step computed.
    int a_read = 0, b_read = 0;
    int a_fill = (NA - 1) * A_STAGE, b_fill = (NB - 1) * B_STAGE;
    auto frags = [&](int ks, bf16x8 (&af)[MI], bf16x8 (&bfr)[NI]) {
        const uint8_t* sA = smem + a_read;
        const uint8_t* sB = smem + B_RING + b_read;
        const int c = ks * 2 + half;
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
            af[mi] = *reinterpret_cast<const bf16x8*>(sA + lds_off<BK>(wm * WTM + mi * 32 + (lane & 31), c));
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
            bfr[ni] = *reinterpret_cast<const bf16x8*>(sB + lds_off<BK>(wn * WTN + ni * 32 + (lane & 31), c));
    };
    auto mfmas = [&](const bf16x8 (&af)[MI], const bf16x8 (&bfr)[NI]) {
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < NI; ++ni)
                acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[ni], af[mi], acc[mi][ni], 0, 0, 0);
    };

    // ---- the block's first tile and the prologue (the steps before step 0)
    int t = xcd_remap(blockIdx.x, G);   // fixed segments: < tiles (the host caps G)
    if (DYN) {
        // The tile list, built in LDS before any load lands there: per expert
        // its segment and the tiles before it (a scan), then per lane k a
        // binary search for tile t + k*G.
        int* s_tp = reinterpret_cast<int*>(smem);            // [E + 1] tiles before expert e
        int* s_lo = s_tp + kMaxE + 1;                         // [E] segment start
        int* s_len = s_lo + kMaxE;                            // [E] segment length
        extent_slots = min(max(((const_int_ptr)(p.extent))[0], 0), p.R);
        for (int e = threadIdx.x; e < p.E; e += NW * kWave) {
            const int lo = seg_lo(p.block_start[e]);
            const int hi = e + 1 < p.E ? seg_lo(p.block_start[e + 1]) : extent_slots;
            const int len = max(hi - lo, 0);
            s_lo[e] = lo;
            s_len[e] = len;
            s_tp[e + 1] = tiles_of(len);
        }
        __syncthreads();
        if (wave == 0) {
            int carry = 0;
            for (int b = 0; b < p.E; b += kWave) {
                const int e = b + lane;
                int v = e < p.E ? s_tp[e + 1] : 0;
#pragma unroll
                for (int d = 1; d < kWave; d <<= 1) {
                    const int u = __shfl_up(v, d);
                    if (lane >= d) v += u;
                }
                if (e < p.E) s_tp[e + 1] = v + carry;
                carry += __shfl(v, kWave - 1);
            }
            if (lane == 0) s_tp[0] = 0;
        }
        __syncthreads();
        const int tk = t + lane * G;
        if (tk < s_tp[p.E]) {
            int lo = 0, hi = p.E;                             // s_tp[lo] <= tk < s_tp[hi]
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (s_tp[mid] <= tk) lo = mid; else hi = mid;
            }
            const int r = tk - s_tp[lo], mt = (s_len[lo] + BMT - 1) / BMT;
            lt_e = lo;
            lt_ntm = (r / mt) | ((r % mt) << 16);
            lt_seg = s_lo[lo];
            lt_len = s_len[lo];
        }
        __syncthreads();   // the list is read: the LDS belongs to the load rings from here on
    }
    Tile cur, nxt;
    int k = 0;                           // cur is the workgroup's k-th tile
    if (DYN) {
        if (!find(0, t, cur)) return;    // more workgroups than tiles: nothing to do
    } else {
        decode(t, cur);
    }
    address_fixed(cur);
    if (FC1) {
        int tok[A_INST];
        load_tokens(cur, tok);
        address_a(cur, tok);
    }
    zero_acc();
    constexpr int LEAD = NA > NB ? NA : NB;
#pragma unroll
    for (int j = -(LEAD - 1); j < 0; ++j) {                 // steps -(LEAD-1)..-1
        if (j + NA - 1 >= 0) issue_a(cur, (j + NA - 1) * A_STAGE, j + NA - 1);   // A(0) .. A(NA-2)
        if (j + NB - 1 >= 0) issue_b(cur, (j + NB - 1) * B_STAGE, j + NB - 1);   // B(0) .. B(NB-2)
    }

    // One K step (after its wait and barrier, which publish slab kt and retire
    // slab kt-1): for each 16-deep slice, fetch the MFMA operands, queue the
    // MFMAs, then issue a share of the loads that refill the retired stages
    // with the slabs NA-1 and NB-1 ahead (from the next tile once this one
    // runs out).  Spreading the loads over the slices lets the memory pipe
    // work while the matrix cores do; the issue order (all of A's loads, then
    // all of B's) is the one the waits count on.
    constexpr int SLICES = BK / 16;
    auto issue_share = [&](int kt, int lo, int hi) {
        const int ta = kt + NA - 1, tb = kt + NB - 1;
        const bool a_cur = ta < KT, b_cur = tb < KT;
        const uint32_t ka = static_cast<uint32_t>(a_cur ? kslab(cur, ta) : kslab(nxt, ta - KT)) * ROWB;
        const uint32_t kb = static_cast<uint32_t>(b_cur ? kslab(cur, tb) : kslab(nxt, tb - KT)) * ROWB;
#pragma unroll
        for (int q = 0; q < LOADS; ++q) {
            if (q < lo || q >= hi) continue;
            if (q < A_INST) {
                const i32x4 r = FC1 ? x_rsrc : (a_cur ? cur.ra : nxt.ra);
                const uint32_t v = (a_cur ? cur.av[q] : nxt.av[q]) + ka;
                dma16(r, v, lds0 + a_fill + (wave + q * NW) * 1024);
            } else {
                const int i = q - A_INST;
                const i32x4 r = b_cur ? cur.rb : nxt.rb;
                const uint32_t v = (b_cur ? cur.bv[i] : nxt.bv[i]) + kb;
                dma16<true>(r, v, lds0 + B_RING + b_fill + (wave + i * NW) * 1024);
            }
        }
    };
    auto step = [&](int kt) {
        bf16x8 af[MI], bfr[NI];
#pragma unroll
        for (int ks = 0; ks < SLICES; ++ks) {
            frags(ks, af, bfr);
            mfmas(af, bfr);
            issue_share(kt, ks * LOADS / SLICES, (ks + 1) * LOADS / SLICES);
        }
        const int a = a_read, b = b_read;
        a_read = a + A_STAGE == NA * A_STAGE ? 0 : a + A_STAGE;
        b_read = b + B_STAGE == NB * B_STAGE ? 0 : b + B_STAGE;
        a_fill = a;
        b_fill = b;
    };

    bool first = true;
    for (;;) {
        const int tn = t + G;
        bool has_next;
        if (DYN) {
            has_next = find(k + 1, tn, nxt);
        } else {
            has_next = tn < p.tiles;
            if (has_next) decode(tn, nxt);
        }
        if (has_next) {
            address_fixed(nxt);
        } else {
            nxt.e = nxt.m0 = nxt.nt = nxt.rot = nxt.seg = nxt.len = 0;
            address_none(nxt);
        }
        float prob[MI];                                     // FC1: probability of the lane's rows
        int ntok[A_INST];

        // step 0 (peeled: FC1 then fetches the next tile's token rows and this
        // tile's probabilities, and waits for them in step 1, so no
        // compiler-inserted wait lands on the K loop or the epilogue)
        if (first) wait_vmcnt<WAIT>(); else wait_vmcnt<WAIT + STORES>();
        __syncthreads();
        step(0);
        if (FC1) {
            const int64_t slot0 = static_cast<int64_t>(cur.seg) + cur.m0;
#pragma unroll
            for (int mi = 0; mi < MI; ++mi) {
                const int row = wm * WTM + mi * 32 + (lane & 31);
                prob[mi] = cur.m0 + row < cur.len ? p.slot_probs[slot0 + row] : 0.0f;
            }
            if (has_next) load_tokens(nxt, ntok);
        }

        // step 1
        wait_vmcnt<WAIT>();
        __syncthreads();
        if (FC1) {
            if (has_next) address_a(nxt, ntok);
#pragma unroll
            for (int mi = 0; mi < MI; ++mi) asm volatile("" : "+v"(prob[mi]));
        }
        step(1);

        for (int kt = 2; kt < KT; ++kt) {
            wait_vmcnt<WAIT>();
            __syncthreads();
            step(kt);
        }

        // ---- epilogue: registers -> global.  Lane (row l&31, half h) holds
        // columns 8g + 4h + (0..3) in acc[4g..4g+3].  Packed to bf16, a swap
        // of lane halves gives lane l < 32 the columns 8g..8g+7 for even g and
        // lane l+32 those for odd g.  Rows past Cp and columns past the output
        // width get an offset beyond the descriptor: the store is dropped.
        const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
            p.out + static_cast<int64_t>(cur.seg) * p.ncols, static_cast<short>(0),
            cur.len * p.ncols * 2, kRsrcWord3);
        const __amdgpu_buffer_rsrc_t prsrc = __builtin_amdgcn_make_buffer_rsrc(
            SAVE ? p.preact + static_cast<int64_t>(cur.seg) * 2 * p.ncols : p.out, static_cast<short>(0),
            SAVE ? cur.len * p.ncols * 4 : 0, kRsrcWord3);
        // FC1: the lane's 8 activations of block (mi, ni), tile columns
        // (wn*WTN + ni*32)/2 + 8*half ..
        auto fc1_act = [&](int mi, int ni) {
            const floatx16& v = acc[mi][ni];
            uint32_t x[2], y[2];
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                x[q] = pack_bf16x2(silu(v[2 * q]) * v[2 * q + 8] * prob[mi],
                                   silu(v[2 * q + 1]) * v[2 * q + 9] * prob[mi]);
                y[q] = pack_bf16x2(silu(v[2 * q + 4]) * v[2 * q + 12] * prob[mi],
                                   silu(v[2 * q + 5]) * v[2 * q + 13] * prob[mi]);
            }
            const auto s0 = __builtin_amdgcn_permlane32_swap(x[0], y[0], false, false);
            const auto s1 = __builtin_amdgcn_permlane32_swap(x[1], y[1], false, false);
            u32x4 d;
            d[0] = s0[0]; d[1] = s1[0]; d[2] = s0[1]; d[3] = s1[1];
            return d;
        };
        // FC2: the lane's 8 outputs of block (mi, ni), half q: the wave's
        // columns ni*32 + 16q + 8*half ..
        auto fc2_out = [&](int mi, int ni, int q) {
            uint32_t g[2][2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                g[h][0] = pack_bf16x2(acc[mi][ni][8 * q + 4 * h], acc[mi][ni][8 * q + 4 * h + 1]);
                g[h][1] = pack_bf16x2(acc[mi][ni][8 * q + 4 * h + 2], acc[mi][ni][8 * q + 4 * h + 3]);
            }
            const auto s0 = __builtin_amdgcn_permlane32_swap(g[0][0], g[1][0], false, false);
            const auto s1 = __builtin_amdgcn_permlane32_swap(g[0][1], g[1][1], false, false);
            u32x4 d;
            d[0] = s0[0]; d[1] = s1[0]; d[2] = s0[1]; d[3] = s1[1];
            return d;
        };
        if constexpr (EPI != 0) {
            constexpr int POLICY = EPI == 2 ? kStoreNT : kStoreSys;
            typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
            __syncthreads();                                // every wave is past the last K step
            const uint32_t rA = static_cast<uint32_t>(a_fill), rB = static_cast<uint32_t>(B_RING + b_fill);
            if constexpr (FC1) {
                // The freed A and B stages hold CAP rows of 256 bytes (16
                // chunks, swizzled by row) of a 128-column tile: rows
                // [base, base + CAP) of the tile go there per round, then 16
                // lanes write each row whole.  Parts: the activation, then
                // (SAVE) the raw gate and up columns of the same rows, at col
                // and I + col of preact.
                constexpr int ROWS_A = A_STAGE / 256, CAP = ROWS_A + B_STAGE / 256;
                static_assert(OUT_COLS == 128 && CAP % 32 == 0, "staged FC1 rows");
                auto so = [&](int sr, int c) {
                    const int rr = sr < ROWS_A ? sr : sr - ROWS_A;
                    return (sr < ROWS_A ? rA : rB) + static_cast<uint32_t>(rr * 256 + ((c ^ (rr & 15)) << 4));
                };
                // raw gate (part 0: acc[0..7]) or up (part 1: acc[8..15])
                // columns of block (mi, ni) as 8 bf16, like fc1_act's
                auto fc1_raw = [&](int mi, int ni, int part) {
                    const floatx16& v = acc[mi][ni];
                    uint32_t x[2], y[2];
#pragma unroll
                    for (int q = 0; q < 2; ++q) {
                        x[q] = pack_bf16x2(v[8 * part + 2 * q], v[8 * part + 2 * q + 1]);
                        y[q] = pack_bf16x2(v[8 * part + 2 * q + 4], v[8 * part + 2 * q + 5]);
                    }
                    const auto s0 = __builtin_amdgcn_permlane32_swap(x[0], y[0], false, false);
                    const auto s1 = __builtin_amdgcn_permlane32_swap(x[1], y[1], false, false);
                    u32x4 d;
                    d[0] = s0[0]; d[1] = s1[0]; d[2] = s0[1]; d[3] = s1[1];
                    return d;
                };
                bool started = false;
#pragma unroll
                for (int part = 0; part < (SAVE ? 3 : 1); ++part) {
#pragma unroll
                    for (int base = 0; base < BMT; base += CAP) {
                        if (started) __syncthreads();      // the previous round is read back
                        started = true;
#pragma unroll
                        for (int mi = 0; mi < MI; ++mi) {
                            const int r0 = wm * WTM + mi * 32;   // the block's first tile row
                            if (r0 < base || r0 >= base + CAP) continue;
#pragma unroll
                            for (int ni = 0; ni < NI; ++ni)
                                *(lds_u32x4*)((lds_u8*)smem + so(r0 - base + (lane & 31),
                                                                 ((wn * WTN + ni * 32) / 2 + 8 * half) / 8)) =
                                    part == 0 ? fc1_act(mi, ni) : fc1_raw(mi, ni, part - 1);
                        }
                        __syncthreads();
                        const int cnt = BMT - base < CAP ? BMT - base : CAP;   // rows this round
#pragma unroll
                        for (int j = 0; j < (CAP + NW * 4 - 1) / (NW * 4); ++j) {
                            const int sr = j * NW * 4 + wave * 4 + lane / 16, c = lane % 16;
                            if (j * NW * 4 >= cnt) break;            // uniform: whole instructions
                            const u32x4 v = *(const lds_u32x4*)((lds_u8*)smem + so(sr, c));
                            const int row = cur.m0 + base + sr, col = cur.nt * OUT_COLS + c * 8;
                            const bool live = sr < cnt && row < cur.len && col < p.ncols;
                            if (part == 0) {
                                __builtin_amdgcn_raw_buffer_store_b128(
                                    v, orsrc, live ? (static_cast<uint32_t>(row) * p.ncols + col) * 2u : kOob, 0, POLICY);
                            } else {
                                const uint32_t poff = (static_cast<uint32_t>(row) * 2u * p.ncols + col +
                                                       (part - 1) * static_cast<uint32_t>(p.ncols)) * 2u;
                                __builtin_amdgcn_raw_buffer_store_b128(v, prsrc, live ? poff : kOob, 0, POLICY);
                            }
                        }
                    }
                }
            } else {
                // each wave gets 8 KB of the freed stages (slots that do not
                // straddle them) for its WTM x 64 piece, 64 rows (two row
                // blocks) of 128 bytes (8 chunks swizzled by row) per round;
                // the wave reads back what its other lanes wrote (LDS
                // operations of one wave complete in order; the clobbers keep
                // the compiler from moving them across), 8 lanes per line
                constexpr int SLOTS_A = A_STAGE / 8192;
                static_assert(WTN == 64 && SLOTS_A + B_STAGE / 8192 >= NW, "staged FC2 slots");
                const uint32_t base = wave < SLOTS_A ? rA + wave * 8192u : rB + (wave - SLOTS_A) * 8192u;
                auto so = [&](int r, int c) { return base + static_cast<uint32_t>(r * 128 + ((c ^ (r & 7)) << 4)); };
#pragma unroll
                for (int h = 0; h < (MI + 1) / 2; ++h) {
                    asm volatile("" ::: "memory");
#pragma unroll
                    for (int m2 = 0; m2 < 2; ++m2) {
                        if (2 * h + m2 >= MI) continue;
#pragma unroll
                        for (int ni = 0; ni < NI; ++ni)
#pragma unroll
                            for (int q = 0; q < 2; ++q)
                                *(lds_u32x4*)((lds_u8*)smem + so(m2 * 32 + (lane & 31), ni * 4 + 2 * q + half)) =
                                    fc2_out(2 * h + m2, ni, q);
                    }
                    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                    const int nrows = 2 * h + 1 < MI ? 64 : 32;
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        if (j * 8 >= nrows) break;
                        const int r = j * 8 + lane / 8, c = lane % 8;
                        const u32x4 v = *(const lds_u32x4*)((lds_u8*)smem + so(r, c));
                        const int row = cur.m0 + wm * WTM + h * 64 + r, col = cur.nt * OUT_COLS + wn * WTN + c * 8;
                        const uint32_t off = row < cur.len && col < p.ncols
                            ? (static_cast<uint32_t>(row) * p.ncols + col) * 2u : kOob;
                        __builtin_amdgcn_raw_buffer_store_b128(v, orsrc, off, 0, POLICY);
                    }
                    asm volatile("" ::: "memory");
                }
            }
        } else {
#pragma unroll
            for (int mi = 0; mi < MI; ++mi) {
                const int row = cur.m0 + wm * WTM + mi * 32 + (lane & 31);   // slot within the expert
#pragma unroll
                for (int ni = 0; ni < NI; ++ni) {
                    if (FC1) {
                        const int col = cur.nt * OUT_COLS + (wn * WTN + ni * 32) / 2 + 8 * half;
                        const bool live = row < cur.len && col < p.ncols;
                        const uint32_t off = live ? (static_cast<uint32_t>(row) * p.ncols + col) * 2u : kOob;
                        __builtin_amdgcn_raw_buffer_store_b128(fc1_act(mi, ni), orsrc, off, 0, 0);
                        if (SAVE) {
                            // the same columns of the raw gate (acc[0..7]) and up
                            // (acc[8..15]) rows, at col and I + col of the row
                            const floatx16& v = acc[mi][ni];
                            uint32_t gx[2], gy[2], ux[2], uy[2];
#pragma unroll
                            for (int q = 0; q < 2; ++q) {
                                gx[q] = pack_bf16x2(v[2 * q], v[2 * q + 1]);
                                gy[q] = pack_bf16x2(v[2 * q + 4], v[2 * q + 5]);
                                ux[q] = pack_bf16x2(v[2 * q + 8], v[2 * q + 9]);
                                uy[q] = pack_bf16x2(v[2 * q + 12], v[2 * q + 13]);
                            }
                            const auto g0 = __builtin_amdgcn_permlane32_swap(gx[0], gy[0], false, false);
                            const auto g1 = __builtin_amdgcn_permlane32_swap(gx[1], gy[1], false, false);
                            const auto u0 = __builtin_amdgcn_permlane32_swap(ux[0], uy[0], false, false);
                            const auto u1 = __builtin_amdgcn_permlane32_swap(ux[1], uy[1], false, false);
                            u32x4 dg, du;
                            dg[0] = g0[0]; dg[1] = g1[0]; dg[2] = g0[1]; dg[3] = g1[1];
                            du[0] = u0[0]; du[1] = u1[0]; du[2] = u0[1]; du[3] = u1[1];
                            const uint32_t poff = live
                                ? (static_cast<uint32_t>(row) * 2u * p.ncols + col) * 2u : kOob;
                            __builtin_amdgcn_raw_buffer_store_b128(dg, prsrc, poff, 0, 0);
                            __builtin_amdgcn_raw_buffer_store_b128(
                                du, prsrc, live ? poff + static_cast<uint32_t>(p.ncols) * 2u : kOob, 0, 0);
                        }
                    } else {
#pragma unroll
                        for (int q = 0; q < 2; ++q) {
                            const int col = cur.nt * OUT_COLS + wn * WTN + ni * 32 + 16 * q + 8 * half;
                            const uint32_t off = row < cur.len && col < p.ncols
                                ? (static_cast<uint32_t>(row) * p.ncols + col) * 2u : kOob;
                            __builtin_amdgcn_raw_buffer_store_b128(fc2_out(mi, ni, q), orsrc, off, 0, 0);
                        }
                    }
                }
            }
        }
        zero_acc();
        first = false;
        if (!has_next) break;
        t = tn;
        ++k;
        cur.e = nxt.e;
        cur.m0 = nxt.m0;
        cur.nt = nxt.nt;
        cur.rot = nxt.rot;
        cur.seg = nxt.seg;
        cur.len = nxt.len;
        cur.ra = nxt.ra;
        cur.rb = nxt.rb;
#pragma unroll
        for (int i = 0; i < A_INST; ++i) cur.av[i] = nxt.av[i];
#pragma unroll
        for (int i = 0; i < B_INST; ++i) cur.bv[i] = nxt.bv[i];
    }
    wait_vmcnt<0>();   // no DMA may still be writing LDS when the workgroup ends
}

template <int BMT, int BNT, int WM, int WN, int BK, int NA, int NB, bool FC1, bool DYN,
          bool SAVE = false, int EPI = 0>
void launch_persistent(const FfnArgs& a, hipStream_t s) {
    constexpr int threads = WM * WN * kWave;
    auto* k = ffn_gemm_kernel<BMT, BNT, WM, WN, BK, NA, NB, FC1, DYN, SAVE, EPI>;
    static std::atomic<int> occupancy{0};   // workgroups per CU (LDS and registers decide it)
    int occ = occupancy.load(std::memory_order_relaxed);
    if (occ == 0) {
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, reinterpret_cast<const void*>(k), threads, 0) !=
                hipSuccess || occ < 1)
            occ = 1;
        occupancy.store(occ, std::memory_order_relaxed);
    }
    // variable segments: the tile count is known only on the device, so every
    // resident slot starts and the surplus workgroups return at once
    const int grid = DYN ? device_cus() * occ : std::min(a.tiles, device_cus() * occ);
    k<<<grid, threads, 0, s>>>(a);
}

template <int BMT, int BNT, int WM, int WN, int BK, int NA, int NB>
int launch_gemm(FfnArgs a, bool fc1, int E, hipStream_t s, bool dyn = false) {
    // the cross-tile look-ahead reaches at most one tile ahead
    if (a.Kdim % BK != 0 || a.Kdim / BK < std::max(NA, NB - 1)) return MOE_ERR_UNSUPPORTED;
    a.MT = (a.Cp + BMT - 1) / BMT;
    a.NT = fc1 ? (a.ncols + BNT / 2 - 1) / (BNT / 2) : (a.ncols + BNT - 1) / BNT;
    a.tiles = E * a.MT * a.NT;
    a.E = E;
    // Tiles of 256 x 256 (FC1 and FC2) and 320 x 256 (FC2) leave through the
    // staged epilogue: FC1's activation non-temporal (FC2 reads it from HBM
    // at no measured cost), FC2's route_out with system scope (written
    // through the L2, so it does not evict the activation rows the expert's
    // other column tiles still read; the combine that reads route_out next
    // runs as fast as after default-policy stores, while non-temporal ones
    // slow it).  A 320-row FC1 tile keeps direct stores: staged, its
    // registers spill (280 vs 233 us).
    constexpr bool SHAPE = BNT == 256 && BK == 64 && WM == 2 && WN == 4;
    constexpr bool STAGED = SHAPE && BMT == 256;
    constexpr bool STAGED2 = SHAPE && (BMT == 256 || BMT == 320);
    if (dyn) {
        if (fc1) launch_persistent<BMT, BNT, WM, WN, BK, NA, NB, true, true, false, STAGED ? 2 : 0>(a, s);
        else launch_persistent<BMT, BNT, WM, WN, BK, NA, NB, false, true, false, STAGED2 ? 1 : 0>(a, s);
    } else {
        if (fc1 && a.preact) launch_persistent<BMT, BNT, WM, WN, BK, NA, NB, true, false, true, STAGED ? 2 : 0>(a, s);
        else if (fc1) launch_persistent<BMT, BNT, WM, WN, BK, NA, NB, true, false, false, STAGED ? 2 : 0>(a, s);
        else launch_persistent<BMT, BNT, WM, WN, BK, NA, NB, false, false, false, STAGED2 ? 1 : 0>(a, s);
    }
    return MOE_OK;
}

// M-tile: the one (of 256, 128, 64, 32) that pads Cp the least; ties go to
// the larger tile (fewer re-reads of each weight panel).  A 320-slot segment
// is the exception.
int pick_tile_m(int Cp) {
    // a segment of exactly 320 slots takes one 320-row tile: one weight pass
    if (Cp == 320) return 320;
    int best = 256, best_rows = (Cp + 255) / 256 * 256;
    for (int t : {128, 64, 32}) {
        const int rows = (Cp + t - 1) / t * t;
        if (rows < best_rows) { best = t; best_rows = rows; }
    }
    return best;
}

// Variable segments: every row tile of an expert streams its weight panel
// (from HBM or, beside a sibling tile, from L2), so the tile should hold a
// typical segment whole.  With routes spread evenly a segment holds about
// mean +- sqrt(mean) slots; the tile covers mean + 2 sqrt(mean).  Just past
// 256 rows a 320-row tile keeps one weight pass per expert (its LDS leaves
// room for two weight stages only, which costs less than a second, mostly
// empty row tile that streams the panel again); well past it the segments
// take several 256-row tiles either way.
int pick_tile_dyn(double mean) {
    const double est = mean + 2.0 * std::sqrt(mean);
    if (est > 256.0 && est <= 320.0) return 320;
    if (est > 128.0) return 256;
    if (est > 64.0) return 128;
    if (est > 32.0) return 64;
    return 32;
}

// FC2 with an output row map runs on the producer/consumer slot GEMM (same
// tiles, same K order: the same products bit for bit as the one-role kernel).
int launch_fc2_slots(const FfnArgs& a, int E, hipStream_t s, const int* out_rows = nullptr) {
    SlotArgs sa{};
    sa.a = a.a; sa.b = a.w; sa.out = a.out;
    sa.lda = a.Kdim; sa.ldb = a.Kdim; sa.ldo = a.ncols;
    sa.Nn = a.ncols; sa.Kd = a.Kdim; sa.Cp = a.Cp;
    sa.MT = (a.Cp + 255) / 256;
    sa.NT = (a.ncols + 255) / 256;
    const int64_t tiles = static_cast<int64_t>(E) * sa.MT * sa.NT;
    if (tiles > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    sa.tiles = static_cast<int>(tiles);
    sa.b_estride = static_cast<int64_t>(a.wrows) * a.Kdim;
    sa.krot = kKRotate;
    if (out_rows) {
        sa.out_rows = out_rows;
        slot_gemm_kernel<false, true><<<std::min(sa.tiles, device_cus()), 12 * kWave, 0, s>>>(sa);
    } else {
        slot_gemm_kernel<false><<<std::min(sa.tiles, device_cus()), 12 * kWave, 0, s>>>(sa);
    }
    return MOE_OK;
}

// Fixed segments tile Cp; variable ones (dyn) take their shape from the mean
// number of routes per expert, which only steers performance.
int launch(const FfnArgs& a, bool fc1, int E, hipStream_t s, bool dyn = false, double mean = 0.0) {

    if (a.Kdim < 128) {
        // a 64-long contraction: 32-wide K slabs, so a tile has the two
        // steps the cross-tile look-ahead needs
        return launch_gemm<32, 128, 1, 2, 32, 2, 3>(a, fc1, E, s, dyn);
    }
    switch (dyn ? pick_tile_dyn(mean) : pick_tile_m(a.Cp)) {
        // 64-wide K slabs (128 contiguous bytes per weight row per step keep the
        // HBM stream efficient); rings sized to the 160 KB LDS.
        case 320: return launch_gemm<320, 256, 2, 4, 64, 2, 2>(a, fc1, E, s, dyn);
        case 256: return launch_gemm<256, 256, 2, 4, 64, 2, 3>(a, fc1, E, s, dyn);
        case 128: return launch_gemm<128, 256, 2, 4, 64, 2, 3>(a, fc1, E, s, dyn);
        case 64: return launch_gemm<64, 128, 2, 2, 64, 2, 3>(a, fc1, E, s, dyn);
        default: return launch_gemm<32, 128, 1, 2, 64, 2, 3>(a, fc1, E, s, dyn);
    }
}

// Host checks shared by the three FFN entry points.  Buffer offsets inside a
// kernel are 32-bit: x, one expert's weights and one expert's activation rows
// must each stay below 2 GiB.
int check_ffn(int64_t N, int32_t H, int32_t I, int32_t E, int64_t C, int* Cp) {
    if (N < 0 || E < 1 || C < 0) return MOE_ERR_INVALID_ARG;
    int st = check_dims(H, I);
    if (st != MOE_OK) return st;
    // N is bounded only by the 32-bit offsets below: the GEMMs take any row
    // count (an expert-parallel rank's received rows exceed the routing
    // envelope), unlike the routing calls
    if (N > INT32_MAX || E > kMaxE) return MOE_ERR_UNSUPPORTED;
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
    st = launch(fc1_args(x, w1, sorted_slot_ids, slot_probs, N, H, I, Cp, act), true, E, stream);
    return st != MOE_OK ? st : launch_status();
}

extern "C" int moe_grouped_fc1_swiglu_save(const uint16_t* x, const uint16_t* w1,
                                           const int32_t* sorted_slot_ids, const float* slot_probs,
                                           int64_t N, int32_t H, int32_t I, int32_t E, int64_t C,
                                           uint16_t* act, uint16_t* preact, hipStream_t stream) {
    using namespace moe;
    int Cp = 0;
    int st = check_ffn(N, H, I, E, C, &Cp);
    if (st != MOE_OK) return st;
    if (static_cast<int64_t>(Cp) * I * 4 >= (static_cast<int64_t>(1) << 31)) return MOE_ERR_UNSUPPORTED;
    if (N == 0 || C == 0) return MOE_OK;
    st = check_ptrs({x, w1, sorted_slot_ids, slot_probs, act, preact});
    if (st != MOE_OK) return st;
    FfnArgs a = fc1_args(x, w1, sorted_slot_ids, slot_probs, N, H, I, Cp, act);
    a.preact = preact;
    st = launch(a, true, E, stream);
    return st != MOE_OK ? st : launch_status();
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
    st = launch(fc2_args(act, w2, N, H, I, Cp, route_out), false, E, stream);
    return st != MOE_OK ? st : launch_status();
}

extern "C" int moe_grouped_fc2_rows(const uint16_t* act, const uint16_t* w2, const int32_t* out_rows,
                                    int64_t N, int32_t H, int32_t I, int32_t E, int64_t C,
                                    uint16_t* route_out, hipStream_t stream) {
    using namespace moe;
    int Cp = 0;
    int st = check_ffn(N, H, I, E, C, &Cp);
    if (st != MOE_OK) return st;
    if (N == 0 || C == 0) return MOE_OK;
    // the mapped rows address the whole output through one 32-bit descriptor
    if (static_cast<int64_t>(E) * Cp * H * 2 >= (static_cast<int64_t>(1) << 31)) return MOE_ERR_UNSUPPORTED;
    st = check_ptrs({act, w2, out_rows, route_out});
    if (st != MOE_OK) return st;
    st = launch_fc2_slots(fc2_args(act, w2, N, H, I, Cp, route_out), E, stream, out_rows);
    return st != MOE_OK ? st : launch_status();
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
    st = launch(fc1_args(x, w1, sorted_slot_ids, slot_probs, N, H, I, Cp, act), true, E, stream);
    if (st != MOE_OK) return st;
    st = launch(fc2_args(act, w2, N, H, I, Cp, route_out), false, E, stream);
    return st != MOE_OK ? st : launch_status();
}

namespace moe {
namespace {

// Host checks and arguments of the dropless FFN calls; which = 1 (FC1),
// 2 (FC2) or 3 (both).
int ffn_dropless(int which, const uint16_t* x, const uint16_t* w1, const uint16_t* w2,
                 const int32_t* sorted_slot_ids, const float* slot_probs,
                 const int32_t* block_start, const int32_t* num_tokens_post_padded, int64_t N,
                 int32_t H, int32_t I, int32_t E, int32_t K, uint16_t* act, uint16_t* route_out,
                 hipStream_t stream) {
    if (N < 0 || E < 1 || K < 1 || K > E) return MOE_ERR_INVALID_ARG;
    int st = check_dims(H, I);
    if (st != MOE_OK) return st;
    const int64_t R = moe_dropless_bound(N, K, E);
    if (R < 0) return static_cast<int>(R);
    // an expert's segment holds at most N + BM - 1 slots; offsets are 32-bit
    const int64_t big = static_cast<int64_t>(1) << 31;
    if (R > INT32_MAX || (N + 1) * H * 2 >= big || (N + kBlockM) * std::max(H, I) * 2 >= big ||
        static_cast<int64_t>(2) * I * H * 2 >= big)
        return MOE_ERR_UNSUPPORTED;
    if (N == 0) return MOE_OK;
    if (which & 1) {
        st = check_ptrs({x, w1, sorted_slot_ids, slot_probs, block_start, num_tokens_post_padded, act});
        if (st != MOE_OK) return st;
    }
    if (which & 2) {
        st = check_ptrs({act, w2, block_start, num_tokens_post_padded, route_out});
        if (st != MOE_OK) return st;
    }
    // the tile shape follows the mean load per expert
    const double mean = static_cast<double>(N) * K / E;
    if (which & 1) {
        FfnArgs a1 = fc1_args(x, w1, sorted_slot_ids, slot_probs, N, H, I, 0, act);
        a1.block_start = block_start;
        a1.extent = num_tokens_post_padded;
        a1.R = static_cast<int>(R);
        st = launch(a1, true, E, stream, true, mean);
        if (st != MOE_OK) return st;
    }
    if (which & 2) {
        FfnArgs a2 = fc2_args(act, w2, N, H, I, 0, route_out);
        a2.block_start = block_start;
        a2.extent = num_tokens_post_padded;
        a2.R = static_cast<int>(R);
        st = launch(a2, false, E, stream, true, mean);
        if (st != MOE_OK) return st;
    }
    return launch_status();
}

}  // namespace
}  // namespace moe

extern "C" int moe_grouped_ffn_fwd_dropless(const uint16_t* x, const uint16_t* w1, const uint16_t* w2,
                                            const int32_t* sorted_slot_ids, const float* slot_probs,
                                            const int32_t* block_start,
                                            const int32_t* num_tokens_post_padded, int64_t N,
                                            int32_t H, int32_t I, int32_t E, int32_t K,
                                            uint16_t* act, uint16_t* route_out, hipStream_t stream) {
    return moe::ffn_dropless(3, x, w1, w2, sorted_slot_ids, slot_probs, block_start,
                             num_tokens_post_padded, N, H, I, E, K, act, route_out, stream);
}

extern "C" int moe_grouped_fc1_swiglu_dropless(const uint16_t* x, const uint16_t* w1,
                                               const int32_t* sorted_slot_ids,
                                               const float* slot_probs, const int32_t* block_start,
                                               const int32_t* num_tokens_post_padded, int64_t N,
                                               int32_t H, int32_t I, int32_t E, int32_t K,
                                               uint16_t* act, hipStream_t stream) {
    return moe::ffn_dropless(1, x, w1, nullptr, sorted_slot_ids, slot_probs, block_start,
                             num_tokens_post_padded, N, H, I, E, K, act, nullptr, stream);
}

extern "C" int moe_grouped_fc2_dropless(const uint16_t* act, const uint16_t* w2,
                                        const int32_t* block_start,
                                        const int32_t* num_tokens_post_padded, int64_t N,
                                        int32_t H, int32_t I, int32_t E, int32_t K,
                                        uint16_t* route_out, hipStream_t stream) {
    return moe::ffn_dropless(2, nullptr, nullptr, w2, nullptr, nullptr, block_start,
                             num_tokens_post_padded, N, H, I, E, K, const_cast<uint16_t*>(act),
                             route_out, stream);
}
