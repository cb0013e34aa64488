// Building blocks shared by the grouped GEMMs of libmoe_native (internal).
//
// Raw buffer descriptors whose range check turns out-of-range rows into
// zeros, LDS DMA loads (global memory straight into LDS) with explicit
// vector-memory waits, and the XCD-aware workgroup renumbering.
#pragma once

#include <atomic>

#include "moe_common.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kXcds = 8;         // MI355X: 8 XCDs, workgroups dealt round-robin
constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit data format (CDNA)
// An offset past every descriptor used here (each covers < 2 GiB): a load
// from it returns zeros without touching memory, a store to it is dropped.
constexpr uint32_t kOob = 0x80000000u;
// cache-policy operand of a buffer store: non-temporal (streamed)
constexpr int kStoreNT = 2;
// cache-policy operand of a buffer store: scope bits sc0 sc1 (system
// scope), so the L2 writes the line through instead of keeping it dirty
constexpr int kStoreSys = 17;

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

// The four descriptor words as scalars (a no-op when they already are).
__device__ __forceinline__ i32x4 uniform(i32x4 r) {
    r.x = __builtin_amdgcn_readfirstlane(r.x);
    r.y = __builtin_amdgcn_readfirstlane(r.y);
    r.z = __builtin_amdgcn_readfirstlane(r.z);
    r.w = __builtin_amdgcn_readfirstlane(r.w);
    return r;
}

// 16 bytes per lane from global memory straight into LDS: lane L's data lands
// at M0 + 16*L, so one wave fills one contiguous kilobyte.  Issued as inline
// assembly so the compiler neither tracks it (it would otherwise wait for every
// pending LDS-bound load before any LDS read) nor reorders it across the
// explicit waits below ("memory" clobber).  The compiler's hazard checks do
// not see into inline assembly, so the statement opens with the wait states
// gfx9-family parts need before a vector-memory instruction: 5 after a VALU
// write of an SGPR it reads (the descriptor may come from v_readfirstlane)
// and 1 after a write of M0 that an LDS DMA reads.  STREAM marks the data
// non-temporal (read once; the caches need not keep it).
template <bool STREAM = false>
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t voff, uint32_t lds) {
    if (STREAM)
        asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds"
                     :: "v"(voff), "s"(uniform(rsrc)), "{m0}"(__builtin_amdgcn_readfirstlane(lds))
                     : "memory");
    else
        asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                     :: "v"(voff), "s"(uniform(rsrc)), "{m0}"(__builtin_amdgcn_readfirstlane(lds))
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

typedef short i16x4 __attribute__((__vector_size__(4 * sizeof(short))));
typedef __attribute__((address_space(3))) uint8_t lds_u8;

// K-major LDS stages (one K row per LDS row, 16-byte chunks swizzled
// chunk ^ 4*(row%4)) feed the MFMA through gfx950's ds_read_b64_tr_b16,
// which hands lane i of a 16-lane group element i%4 of the 8-byte pieces
// addressed by lanes 4j + i/4 (j = 0..3): with lane c addressing row
// k0 + c/4, columns n0 + 4(c%4) .. +3, lane i receives column n0 + i of rows
// k0 .. k0+3.  Two such reads give a lane its 8 consecutive K values.
//
// Byte offset, within a K-major stage (rows of ROWB bytes), of the 8-byte
// piece that lane `lane` addresses in a transpose read of the 32-wide column
// block at column t, K rows kb .. kb+7 (read r = 0 or 1 covers kb+4r ..).
template <int ROWB>
__device__ __forceinline__ uint32_t tr_off(int lane, int t, int kb, int r) {
    const int g = lane >> 4, i = lane & 15;
    const int col = t + 16 * (g & 1) + 4 * (i & 3);
    const int k = kb + 8 * (g >> 1) + 4 * r + (i >> 2);
    const int lc = col >> 3, half = (col >> 2) & 1;
    return static_cast<uint32_t>(k * ROWB + ((lc ^ (4 * (k & 3))) << 4) + half * 8);
}

__device__ __forceinline__ bf16x8 tr_frag(const lds_u8* stage, uint32_t off0, uint32_t off1) {
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(stage + off0));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(stage + off1));
    typedef short i16x8 __attribute__((__vector_size__(8 * sizeof(short))));
    const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, v);
}

// Compute units of the current device, queried once per device.
int device_cus() {
    static std::atomic<int> cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    int n = dev < 64 ? cus[dev].load(std::memory_order_relaxed) : 0;
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) n = 1;
        if (dev < 64) cus[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

}  // namespace
}  // namespace moe
