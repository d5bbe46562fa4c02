// Device-side building blocks shared by the prefill and decode kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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
__device__ __forceinline__ int swz(int r) {
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

// Words of a raw buffer resource over `bytes` bytes at `base` (gfx9: stride 0,
// 32-bit data format).  Loads at offsets >= bytes return zeros.
__device__ __forceinline__ u32x4 buffer_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = (uint64_t)base;
    return u32x4{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, bytes, 0x00020000u};
}

// One wave moves one 1 KB row of a tile straight into LDS (16 bytes per lane,
// no VGPR staging): lane i's 16 bytes, read at byte row_off + lane_off of the
// resource, land at lds_row + 16 i.  With lane_off = (16 i) ^ (swz(row) << 4)
// the row is stored swizzled.  Bytes past the resource's extent arrive as
// zeros, which is how keys past the cache length are zero-filled.
//
// Issued from asm so that the compiler does not track it: its LDS-DMA
// bookkeeping would otherwise wait for every outstanding tile load before
// any LDS read.  The caller orders it with wait_vmcnt and lds_barrier.
__device__ __forceinline__ void row_to_lds(u32x4 rsrc, const ATTN_LDS char* lds_row,
                                           int lane_off, int row_off) {
    const uint32_t lds = (uint32_t)(uintptr_t)lds_row;
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(lds), "v"(lane_off), "s"(rsrc), "s"(row_off)
                 : "memory", "m0");
}

// Workgroup barrier for LDS hand-offs: this wave's LDS operations complete,
// then s_barrier.  No memory-model fence, hence no implicit wait for the
// vector-memory loads still in flight (those are waited for explicitly).
__device__ __forceinline__ void lds_barrier() {
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

// Wait states covering an XDL MFMA write -> VALU/VMEM/DS read of its result
// (at most 16 passes + a few on gfx950; 3 x 8 = 24 here), tied to the two
// accumulators so that no reader can be scheduled above it.
__device__ __forceinline__ void mfma_vgpr_drain(f32x16& a0, f32x16& a1) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(a0), "+v"(a1));
}

// acc *= alpha for an accumulator tile that lives in AGPRs, in place (VALU
// instructions cannot address AGPRs; each element goes through one VGPR).
__device__ __forceinline__ void agpr_scale(f32x16& acc, float alpha) {
    float e0 = acc[0], e1 = acc[1], e2 = acc[2], e3 = acc[3], e4 = acc[4], e5 = acc[5],
          e6 = acc[6], e7 = acc[7], e8 = acc[8], e9 = acc[9], e10 = acc[10], e11 = acc[11],
          e12 = acc[12], e13 = acc[13], e14 = acc[14], e15 = acc[15];
    float t0, t1;
#define ATTN_SC2(A, B)                                  \
    "v_accvgpr_read_b32 %16, " A "\n\t"                 \
    "v_accvgpr_read_b32 %17, " B "\n\t"                 \
    "v_mul_f32 %16, %16, %18\n\t"                       \
    "v_mul_f32 %17, %17, %18\n\t"                       \
    "v_accvgpr_write_b32 " A ", %16\n\t"                \
    "v_accvgpr_write_b32 " B ", %17\n\t"
    asm volatile(ATTN_SC2("%0", "%1") ATTN_SC2("%2", "%3") ATTN_SC2("%4", "%5")
                 ATTN_SC2("%6", "%7") ATTN_SC2("%8", "%9") ATTN_SC2("%10", "%11")
                 ATTN_SC2("%12", "%13") ATTN_SC2("%14", "%15") "s_nop 1"
                 : "+a"(e0), "+a"(e1), "+a"(e2), "+a"(e3), "+a"(e4), "+a"(e5), "+a"(e6),
                   "+a"(e7), "+a"(e8), "+a"(e9), "+a"(e10), "+a"(e11), "+a"(e12), "+a"(e13),
                   "+a"(e14), "+a"(e15), "=&v"(t0), "=&v"(t1)
                 : "v"(alpha));
#undef ATTN_SC2
    acc = f32x16{e0, e1, e2, e3, e4, e5, e6, e7, e8, e9, e10, e11, e12, e13, e14, e15};
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
