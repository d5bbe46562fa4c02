// Device-side building blocks shared by the prefill and decode kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int v2i32 __attribute__((ext_vector_type(2)));

#define ATTN_LDS __attribute__((address_space(3)))
#define ATTN_GLOBAL __attribute__((address_space(1)))

constexpr int kHeadDim = 512;
constexpr int kPage = 64;           // keys per page = keys per K/V tile
constexpr int kRowBytes = 1024;     // one bf16 row of 512
constexpr int kTileBytes = kPage * kRowBytes;  // 64 KB

// LDS rows of a K or V tile are 1 KB apart, so every row starts in the same
// bank.  Storing 16-byte chunk c of row r at chunk c ^ swz(r) spreads the two
// read patterns over all banks: 16 consecutive rows at one chunk (the K
// operand reads) and 4 consecutive rows x 4 consecutive chunks (the
// transposed V operand reads).  swz is a bijection on r mod 16; its bits
// 1..2 separate the 4 rows of an aligned quad and so do its bits 2..3.
__host__ __device__ constexpr int swz(int r) {
    return ((r >> 2) & 1) | (((r >> 1) & 1) << 1) | ((r & 1) << 2) |
           ((((r >> 1) ^ (r >> 3)) & 1) << 3);
}

// Wait until at most N vector-memory operations of this wave are in flight
// (gfx9 s_waitcnt: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt left at max).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Wait until this wave's LDS (and scalar-memory) operations have completed,
// vector memory left in flight.
__device__ __forceinline__ void wait_lgkmcnt0() {
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
}

// Timing perturbation of the delay-injected test build (-DATTN_RACE_DELAY):
// 0 to 3 naps of about 128 cycles, the count set by the wave, the workgroup
// and the call site, after every LDS refill load and before every workgroup
// barrier.  The waves of a workgroup then reach each hand-off in other
// orders and at other distances than in the normal build, so a missing wait
// or barrier changes the results; the kernels are deterministic, so the
// delayed build must reproduce the normal build's bits.  Nothing is emitted
// in the normal build.
template <int SITE>
__device__ __forceinline__ void race_delay() {
#ifdef ATTN_RACE_DELAY
    const int k = (__builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6) + (int)blockIdx.x +
                   SITE) & 3;
    for (int i = 0; i < k; ++i) __builtin_amdgcn_s_sleep(2);
#endif
}

// Words of a raw buffer resource over `bytes` bytes at `base` (gfx9: stride 0,
// 32-bit data format).  Loads at offsets >= bytes return zeros.
__device__ __forceinline__ u32x4 buffer_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = (uint64_t)base;
    // the words are wave-uniform; readfirstlane keeps them in SGPRs
    return u32x4{(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
                 (uint32_t)__builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xffffu)),
                 (uint32_t)__builtin_amdgcn_readfirstlane((int)bytes), 0x00020000u};
}

// One wave moves one 1 KB tile row straight into LDS (16 bytes per lane, no
// VGPR staging).  The row lies REL bytes past byte `soff` of the resource and
// past LDS byte `lds_base`.  Lane i's 16 bytes land at LDS row start + 16 i,
// so lane i fetches the logical chunk the swizzle stores at chunk i: lane
// offset lane_off ^ SWZ, with lane_off = 16 i (possibly pre-XORed with a
// wave-dependent part of the row's swizzle; below 1 KB either way) and SWZ
// the row's remaining swizzle bits, shifted to bytes.  Bytes past the
// resource's extent arrive as zeros, which is how keys past the cache length
// are zero-filled.
//
// Issued from asm so that the compiler does not track it: its LDS-DMA
// bookkeeping would otherwise wait for every outstanding tile load before
// any LDS read.  Callers order it with wait_vmcnt and lds_barrier.  M0 carries
// the LDS address; it is written first so that the VALU op forming the lane
// offset fills the wait state the load needs after the SALU write; none of
// the kernels built with these helpers use M0 for anything else.  The SALU
// add also writes SCC, which the clobber list declares.
template <int SWZ, int REL, bool NT = false>
__device__ __forceinline__ void dma_row(u32x4 rsrc, uint32_t lds_base, uint32_t soff,
                                        int lane_off) {
    // lane_off and SWZ lie below 1 KB and REL is whole rows, so
    // (lane_off ^ SWZ) + REL is one XOR with the constant SWZ | REL
    static_assert(SWZ >= 0 && SWZ < kRowBytes && REL % kRowBytes == 0, "row offset layout");
    int voff;
    // NT: non-temporal (streaming) cache policy, for data read exactly once
    if constexpr (NT) {
        asm volatile(
            "s_add_u32 m0, %4, %3\n\t"
            "v_xor_b32 %0, %1, %2\n\t"
            "buffer_load_dwordx4 %0, %5, %6 offen nt lds"
            : "=&v"(voff)
            : "i"(SWZ | REL), "v"(lane_off), "i"(REL), "s"(lds_base), "s"(rsrc), "s"(soff)
            : "memory", "m0", "scc");
    } else {
        asm volatile(
            "s_add_u32 m0, %4, %3\n\t"
            "v_xor_b32 %0, %1, %2\n\t"
            "buffer_load_dwordx4 %0, %5, %6 offen lds"
            : "=&v"(voff)
            : "i"(SWZ | REL), "v"(lane_off), "i"(REL), "s"(lds_base), "s"(rsrc), "s"(soff)
            : "memory", "m0", "scc");
    }
    race_delay<0>();
}

// Compile-time loop: f(std::integral_constant<int, i>{}) for i = 0 .. N-1, so
// that the index can feed template arguments and asm immediates.
template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
    (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// A wave's 16 rows of one tile, rows 16 wave .. 16 wave + 15 (row 16 wave + i
// has swizzle swz(i)).
template <bool NT>
__device__ __forceinline__ void rows16_to_lds(u32x4 rsrc, const ATTN_LDS char* buf, int wave,
                                              int lane16) {
    const uint32_t off = (uint32_t)wave * 16 * kRowBytes;
    const uint32_t base = (uint32_t)(uintptr_t)buf + off;
    static_for<16>([&](auto I) {
        constexpr int i = decltype(I)::value;
        dma_row<(swz(i) << 4), i * kRowBytes, NT>(rsrc, base, off, lane16);
    });
}

// Workgroup barrier for LDS hand-offs: this wave's LDS operations complete,
// then s_barrier.  No memory-model fence, hence no implicit wait for the
// vector-memory loads still in flight (those are waited for explicitly).
__device__ __forceinline__ void lds_barrier() {
    race_delay<1>();
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// acc += a b on the VGPR form of v_mfma_f32_32x32x16_bf16.  The compiler
// places every builtin MFMA accumulator of a 512-register kernel in AGPRs;
// this form keeps a score tile in VGPRs, where the softmax reads it.  The
// caller must run mfma_vgpr_drain on the accumulators before any other
// instruction reads them (the asm is opaque to the hazard recognizer).
__device__ __forceinline__ void mfma32x32x16_vgpr(f32x16& acc, bf16x8 a, bf16x8 b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}

// acc = a b (inline zero accumulator), VGPR form: starts a chain without any
// VALU write feeding the MFMA.
__device__ __forceinline__ void mfma32x32x16_vgpr_first(f32x16& acc, bf16x8 a, bf16x8 b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}

// The same two forms for an A operand that VALU instructions have just
// written (e.g. widened FP8): the asm is opaque to the hazard recognizer, so
// the VALU-write -> MFMA-read wait states are issued here (5, more than the
// gfx950 requirement).
__device__ __forceinline__ void mfma32x32x16_vgpr_va(f32x16& acc, bf16x8 a, bf16x8 b) {
    asm volatile("s_nop 4\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                 : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma32x32x16_vgpr_first_va(f32x16& acc, bf16x8 a, bf16x8 b) {
    asm volatile("s_nop 4\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0"
                 : "=&v"(acc) : "v"(a), "v"(b));
}

// Wait states covering an XDL MFMA write -> VALU/VMEM/DS read of its result
// (at most 16 passes + a few on gfx950; 3 x 8 = 24 here), tied to the
// accumulator so that no reader can be scheduled above it.
__device__ __forceinline__ void mfma_vgpr_drain(f32x16& a0) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(a0));
}

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Transposed 8-byte LDS read: within each 16-lane group, lane i receives
// element (i % 4) of the 4-element chunk addressed by group lane 4j + i/4 as
// its element j.  With group lane 4j+q pointing at row (k0 + j), columns
// (c0 + 4q .. c0 + 4q + 3), lane i gets column c0 + i of rows k0 .. k0 + 3.
__device__ __forceinline__ bf16x4 lds_read_tr16(const ATTN_LDS char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((ATTN_LDS bf16x4*)p);
}

// p[idx] for a wave-uniform index, through the scalar data cache (a scalar
// load counts in lgkmcnt, so it never waits behind in-flight tile loads).
// The table must not change while the kernel runs.
__device__ __forceinline__ int load_uniform(const int* p, int idx) {
    const __attribute__((address_space(4))) int* c = (const __attribute__((address_space(4))) int*)p;
    return __builtin_amdgcn_readfirstlane(c[idx]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace attn
