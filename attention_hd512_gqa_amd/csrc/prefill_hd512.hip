// Chunked causal GQA/MQA prefill at head_dim 512 over a paged bf16 KV cache,
// for gfx950 (MI355X).  One FlashAttention-style pass per workgroup: scores
// live in registers only, with an online softmax in fp32 (Writing a
// FlashAttention Prefill Kernel for Gemma 4, "Head dim 512 breaks the
// textbook" and "The bug that passed every test").
//
// Work unit (one workgroup, 4 waves): 128 packed query rows of one KV head of
// one sequence.  Packed row r is token r / g and query head r % g of the
// group, so every K/V tile brought into LDS serves all g heads of the group
// (A custom attention kernel for Gemma 4 on the RTX PRO 6000, "The kernel in
// three steps", step 1).  Wave w owns packed rows 32w .. 32w+31 with the full
// Q row in VGPRs and the full O row in accumulators (head dim 512: a
// gfx950 wave has up to 512 registers, so the register ceiling that pushed
// the Ada and Blackwell kernels to split head_dim across warps does not bind
// here, and no score partials need exchanging between waves).
//
// Per 64-key tile (= one page of one KV head):
//   K and V arrive in two separate 64 KB LDS buffers (no time-sharing of one
//   buffer; pegainfer issue 1051, "Description") by direct buffer->LDS loads,
//   one coalesced 1 KB key row per wave instruction, XOR-swizzled per 16 bytes;
//   S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (fp32 accumulators), so that each
//   lane holds one query row's scores;
//   masked keys get -inf (only tiles that cross a row's causal limit or the
//   cache length are masked; tiles past the last row's limit are never loaded);
//   softmax statistics in fp32 with exp2, per 64-key tile (Flash-Decoding for
//   MQA in CUDA, "One KV head breaks the textbook": statistics per tile, not
//   per key), against a per-row reference maximum (see below);
//   P goes to bf16 and O^T += V^T P^T on the same MFMA, V^T read with the
//   gfx950 transposing LDS load.  O accumulates in fp32 across the whole key
//   range (vLLM flash-attention PR 199, commit 3 of the first review).
//
// Within a wave the tile is processed as two 32-key blocks whose chains
// overlap: Q.K^T of block 1 issues on the matrix core while the VALU runs the
// softmax of block 0, and P.V of block 0 while the softmax of block 1 runs.
// The four phases (Q.K^T and P.V of each block) each free one 32-key half of
// the K or V buffer; after the phase's barrier that half is refilled for the
// tile that needs it two phases later, with the wave's 8 row loads spread one
// per four MFMAs over the next phase (a burst of 1 KB buffer->LDS loads would
// stall the wave's instruction issue and starve the matrix core).  A phase's
// last MFMAs go out after the next phase's barrier, beside that phase's first
// operand reads, so that the matrix core has work while they come back.
//
// The same kernel, by template parameters, also covers: an FP8-E4M3 pool
// (512-byte tile rows, bytes widened exactly to bf16 at their MFMA); head dim
// 256 for the sliding-window local layers (512-byte bf16 rows, half the
// MFMAs per tile; A custom attention kernel for Gemma 4 on the RTX PRO 6000,
// "The deployment"), with a window that bounds each row's keys from below and
// a ring cache (Flash-Decoding for MQA in CUDA, "One KV head breaks the
// textbook": slot = position % capacity); and split-K, where workgroups of
// one row block take disjoint key ranges and write unnormalised partials
// that prefill_merge_kernel combines.
#include "device_common.h"
#include "attn_host.h"
#include "prefill_common.h"

#include <type_traits>

namespace attn {

namespace {

constexpr int kRowsPerWaveLoad = kPage / kWaves;  // tile rows each wave moves
constexpr int kPrefetch = 4;  // LDS operand reads in flight ahead of their MFMA
constexpr int kXcds = 8;            // XCDs of a gfx950 part (one work queue each)
constexpr int kCounterStride = 32;  // ints between queue counters (own 128-byte line)
// Row blocks whose first row sees at most this many keys get P in two bf16
// terms in their first tile
constexpr int kLoKeys = 64;
// FP8 operands are widened in registers; one fewer read in flight keeps the
// FP8 kernel inside the 256 VGPRs
template <bool FP8>
constexpr int kPrefetchOf = FP8 ? 3 : kPrefetch;

// K/V tile geometry for a pool element (bf16, or FP8-E4M3 bytes) and a head
// dim D (512 for the global layers, 256 for the sliding-window ones).  Rows
// are 1 KB (bf16 at 512) or 512 bytes (FP8 at 512, bf16 at 256: "narrow").
template <bool FP8, int D = kHeadDim>
struct Kv {
    static_assert(D == 512 || (D == 256 && !FP8), "head dims 512 (bf16, FP8) and 256 (bf16)");
    static constexpr int kRowB = FP8 ? D : 2 * D;
    static constexpr int kTileB = kPage * kRowB;
    static constexpr bool kNarrow = kRowB == 512;
    // buffer->LDS loads per wave per 32-key half refill: 8 rows of 1 KB, or 4
    // loads of two 512-byte rows
    static constexpr int kDmaPerHalf = kNarrow ? 4 : 8;
    static constexpr int kSteps = D / 16;       // Q.K^T MFMAs (k-steps) per 32-key block
    static constexpr int kDimBlocks = D / 32;   // 32-dim output blocks (P.V MFMAs per k-step)
};

// LDS layout of an FP8 tile: row r (a key) is 512 bytes, its 16-byte chunk c
// sits at chunk c ^ (r % 32).  The K operand reads (32 consecutive rows at one
// chunk) and the transposed V reads (8 rows per 16-lane group at one chunk)
// then hit distinct chunks.
__host__ __device__ constexpr int swz8(int r) { return r & 31; }

// LDS layout of a bf16 head-dim-256 tile: row r is 512 bytes, its 16-byte
// chunk c sits at chunk c ^ swzN(r).  swzN swaps the two 2-bit fields of r's
// low nibble (bit 4 kept): a bijection on r mod 16, so 16 consecutive rows
// at one chunk (the K operand reads) hit distinct bank groups, and its bits
// 2..3 separate the 4 rows of an aligned quad, so a transposed V read (4 rows
// x 4 chunks per half wave) does too.
__host__ __device__ constexpr int swzN(int r) {
    return ((r & 3) << 2) | ((r >> 2) & 3) | (r & 16);
}


// Refill of one 32-key half (rows 32 half .. 32 half + 31) of a K or V tile
// buffer from one (page, KV head) tile: each wave moves rows
// 32 half + 8 wave + j, j = 0..7, one buffer->LDS load per row.  The resource
// covers only the tile's `valid` rows, so rows of keys past the cache length
// (whose slots may hold anything) arrive as zeros.  Row 32 half + 8 wave + j
// has swizzle swz(j) ^ 8 (wave & 1), the second term folded into lane_off.
struct HalfDma {
    u32x4 rsrc;
    uint32_t lds_base;  // LDS address of this wave's first row
    uint32_t soff;      // byte offset of this wave's first row in the tile
    bool on;            // wave-uniform: this refill exists
    // Fused append only (app is a compile-time false everywhere else): row J
    // of the wave's 8 is read J * stride bytes past soff, so that rsrc / soff
    // / stride can name either the pool tile (1 KB rows) or the chunk's
    // new-row buffer (rows of one KV head Hkv KB apart).
    bool app;
    int stride;
};

template <bool FP8, int D>
__device__ __forceinline__ HalfDma half_dma(const char* pool, int page, int num_pages, int hkv,
                                            int kvh, int valid, const ATTN_LDS char* buf,
                                            int half, int wave, bool on) {
    constexpr int kRowB = Kv<FP8, D>::kRowB;
    page = page < 0 ? 0 : (page >= num_pages ? num_pages - 1 : page);
    const char* src = pool + ((size_t)page * hkv + kvh) * (size_t)Kv<FP8, D>::kTileB;
    HalfDma d;
    d.rsrc = buffer_rsrc(src, (uint32_t)(valid > 0 ? valid : 0) * kRowB);
    d.soff = (uint32_t)__builtin_amdgcn_readfirstlane((32 * half + 8 * wave) * kRowB);
    d.lds_base = (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)(uintptr_t)buf + d.soff));
    d.on = on;
    d.app = false;
    d.stride = kRowB;
    return d;
}

// One buffer->LDS load of 16 bytes per lane at LDS byte m0 + 16 lane, from
// byte voff + soff of the resource.
__device__ __forceinline__ void dma16(u32x4 rsrc, uint32_t m0, uint32_t soff, int voff) {
    asm volatile(
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %0, %2, %3 offen lds"
        :
        : "v"(voff), "s"(m0), "s"(rsrc), "s"(soff)
        : "memory", "m0");
    race_delay<0>();
}

// Row J of a wave's 8 at J * stride bytes past byte soff of the resource (a
// runtime row stride), to LDS at lds_base + REL, 16-byte chunks placed like
// dma_row's (M0 written first, as there).
template <int SWZ, int J, int REL>
__device__ __forceinline__ void dma_row_strided(u32x4 rsrc, uint32_t lds_base, uint32_t soff,
                                                int stride, int lane_off) {
    int voff;
    asm volatile(
        "s_add_u32 m0, %5, %6\n\t"
        "v_xor_b32 %0, %1, %2\n\t"
        "v_mad_u32_u24 %0, %3, %4, %0\n\t"
        "buffer_load_dwordx4 %0, %7, %8 offen lds"
        : "=&v"(voff)
        : "i"(SWZ), "v"(lane_off), "i"(J), "s"(stride), "s"(lds_base), "i"(REL), "s"(rsrc),
          "s"(soff)
        : "memory", "m0", "scc");
    race_delay<0>();
}

// Row J of a wave's 8 (1 KB rows), as dma_row places it, with M0 written only
// for rows 0 and 4: the buffer instruction's offset field, which the
// hardware adds to both the source and the LDS address, carries (J % 4) KB,
// and the XOR that forms the lane's source offset carries the 4 KB of rows
// 4..7.  The loads of rows 1..3 and 5..7 use the M0 of the row-0 or row-4
// load before them: every refill of a half starts at row 0, nothing else
// in these kernels writes M0, and the asm statements keep their order.
template <int J>
__device__ __forceinline__ void dma_row_m0(u32x4 rsrc, uint32_t lds_base, uint32_t soff,
                                           int lane_off) {
    constexpr int kSwz = (swz(J) << 4) | ((J / 4) * 4096);
    int voff;
    if constexpr (J % 4 == 0) {
        asm volatile(
            "s_add_u32 m0, %3, %2\n\t"
            "v_xor_b32 %0, %4, %1\n\t"
            "buffer_load_dwordx4 %0, %5, %6 offen lds"
            : "=&v"(voff)
            : "v"(lane_off), "i"((J / 4) * 4096), "s"(lds_base), "i"(kSwz), "s"(rsrc), "s"(soff)
            : "memory", "m0", "scc");
    } else {
        asm volatile(
            "v_xor_b32 %0, %2, %1\n\t"
            "buffer_load_dwordx4 %0, %3, %4 offen offset:%5 lds"
            : "=&v"(voff)
            : "v"(lane_off), "i"(kSwz), "s"(rsrc), "s"(soff), "i"((J % 4) * kRowBytes)
            : "memory");
    }
    race_delay<0>();
}

// Refill load J of this wave's share of a half: 1 KB rows, row 8 wave + J of
// the half; narrow rows, rows 8 wave + 2 J and + 1 (lanes 0-31 and 32-63),
// each lane fetching the logical chunk that the swizzle stores at its LDS
// position: chunk (lane % 32) ^ swz8(row) (FP8) or ^ swzN(row) (bf16 at 256).
template <bool FP8, int D, int J>
__device__ __forceinline__ void half_dma_row(const HalfDma& d, int lane_off, int lane, int wave) {
    if constexpr (Kv<FP8, D>::kNarrow) {
        const int rw = 2 * J + (lane >> 5);            // row within the wave's 8
        const int tr = 8 * wave + rw;                  // tile row mod 32 (32 half is 0 mod 32)
        const int f = FP8 ? swz8(tr) : swzN(tr);
        const int voff = rw * 512 + (((lane & 31) ^ f) << 4);
        dma16(d.rsrc, d.lds_base + 2 * J * 512, d.soff, voff);
    } else {
        if (d.app) {
            dma_row_strided<(swz(J) << 4), J, J * kRowBytes>(d.rsrc, d.lds_base, d.soff,
                                                              d.stride, lane_off);
            return;
        }
        dma_row_m0<J>(d.rsrc, d.lds_base, d.soff, lane_off);
    }
}

template <bool FP8, int D>
__device__ __forceinline__ void half_dma_all(const HalfDma& d, int lane_off, int lane, int wave) {
    if (!d.on) return;
    static_for<Kv<FP8, D>::kDmaPerHalf>([&](auto J) {
        half_dma_row<FP8, D, decltype(J)::value>(d, lane_off, lane, wave);
    });
}

// 8 E4M3 bytes -> 8 bf16 (exact: every E4M3 value is a bf16 value)
__device__ __forceinline__ bf16x8 widen8(uint32_t w0, uint32_t w1) {
    const bf16x2 a0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
    const bf16x2 a1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
    const bf16x2 a2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
    const bf16x2 a3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
    return bf16x8{a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]};
}
__device__ __forceinline__ bf16x8 operand(const bf16x8& x) { return x; }
__device__ __forceinline__ bf16x8 operand(const v2i32& x) {
    return widen8((uint32_t)x[0], (uint32_t)x[1]);
}

// Per-lane state of the softmax of one 32-key block.  Scores arrive already
// masked (masked keys -inf) in raw units: x = s * scale_log2.
struct SoftmaxCtx {
    float scale_log2;
    float neg_m_ref;  // -m_ref
    float lo_f;       // 1 when P's second bf16 term is used, else 0 (zero terms)
};

// One softmax element: p = 2^(s * scale - m_ref) (0 for masked keys).  The
// P^T operand takes p one element later (the previous element's p, `pend`,
// is packed here), so that no instruction reads an exp2 result right after
// it is written (that read costs a wait state); softmax_flush finishes the
// block's last element.  The lane's running sum adds the packed bf16 pairs,
// i.e. the same rounded weights P.V multiplies (one v_dot2 per pair), so
// that numerator and denominator agree: a row with one dominant key gets
// that key's value exactly.  Each pair is summed one pair after it is
// packed, so that the v_dot2 never waits for the conversion before it.
// LO (the range's first tile) also packs the residual p - bf16(p) as a
// second bf16 term and sums it the same way, so that P.V sees p to about 16
// significant bits: rows whose few keys all lie in that tile would
// otherwise carry bf16's relative error on each weight.  No running maximum
// is kept: the block's sum bounds every p of the block, which is all the
// overflow check needs.  Elements 0-7 go to p0 (lo0), 8-15 to p1 (lo1).
// The empty asms pin the element to the MFMA step it is issued with (inputs
// taken and running values produced inside the step): without them, IR
// passes gather the softmax arithmetic into one cluster after the MFMA chain
// and the matrix core idles while it runs.  The input side is pinned through
// `sc`, the wave-uniform scale that the caller threads through its elements
// as a chain of SGPR values (an asm that "modifies" it costs nothing), so
// that the score itself is only read: a score still needed afterwards (the
// overflow path recomputes P from the block's scores) is not copied.
// add_pair: the sum of a packed bf16 pair, added to acc in fp32 (one v_dot2
// with 1, 1).
__device__ __forceinline__ float add_pair(const bf16x8& v, int pair, float acc) {
    const bf16x2 x = {v[2 * pair], v[2 * pair + 1]};
    return __builtin_amdgcn_fdot2_f32_bf16(x, bf16x2{(__bf16)1.f, (__bf16)1.f}, acc, false);
}

template <bool LO = false>
__device__ __forceinline__ void softmax_elem(const SoftmaxCtx& c, float& sc, float s, int i,
                                             float& psum, float& pend, bf16x8& p0, bf16x8& p1,
                                             bf16x8& lo0, bf16x8& lo1) {
    asm volatile("" : "+s"(sc));
    const float p = fast_exp2(__builtin_fmaf(s, sc, c.neg_m_ref));
    if (i > 0) {
        const int e = i - 1;                     // the element packed now
        bf16x8& pv = e < 8 ? p0 : p1;
        bf16x8& lv = e < 8 ? lo0 : lo1;
        const __bf16 hi = (__bf16)pend;
        pv[e & 7] = hi;
        if constexpr (LO) lv[e & 7] = (__bf16)((pend - (float)hi) * c.lo_f);
        if (e & 1) {
            // pair e / 2 is complete: pin its packing here, and sum the one
            // completed a pair ago
            asm volatile("" : "+v"(pv));
            if constexpr (LO) asm volatile("" : "+v"(lv));
            const int g = (e >> 1) - 1;
            if (g >= 0) {
                psum = add_pair(g < 4 ? p0 : p1, g & 3, psum);
                if constexpr (LO) psum = add_pair(g < 4 ? lo0 : lo1, g & 3, psum);
            }
        }
    }
    pend = p;
    asm volatile("" : "+v"(psum));
}

// The block's last element (15), and the sums of its last two pairs.
template <bool LO = false>
__device__ __forceinline__ void softmax_flush(const SoftmaxCtx& c, float& psum, float pend,
                                              bf16x8& p1, bf16x8& lo1) {
    const __bf16 hi = (__bf16)pend;
    p1[7] = hi;
    if constexpr (LO) lo1[7] = (__bf16)((pend - (float)hi) * c.lo_f);
    asm volatile("" : "+v"(p1));
    if constexpr (LO) asm volatile("" : "+v"(lo1));
    psum = add_pair(p1, 2, psum);
    if constexpr (LO) psum = add_pair(lo1, 2, psum);
    psum = add_pair(p1, 3, psum);
    if constexpr (LO) psum = add_pair(lo1, 3, psum);
}

// Largest allowed block sum of p before the reference is raised: every p of
// the block is then at most 2^32, far inside fp32 and bf16, and so are O and l.
constexpr float kBlockSumCap = 4294967296.f;   // 2^32

// The overflow guard of the online softmax.  The reference m_ref is a row's
// maximum over its first 32 keys; later keys usually stay near it, so p =
// 2^(x - m_ref) needs no per-tile rescale.  When a block's sum of p passes
// kBlockSumCap on some lane (or is not finite), the wave calls this before
// the block's P.V: every row of the wave takes the exact maximum of its
// block, raises its reference by the whole number of log2 units k >= 0 that
// brings it to at least that maximum, multiplies what it has accumulated (O
// when o_live, l_run, and the sum of the tile's earlier block) by 2^-k,
// which is exact, and recomputes the block's P against the new reference.
// A row whose maximum did not rise keeps k = 0 and its values bit for bit.
// This is the online softmax's rescale, run only for the blocks that need
// it (Flash-Decoding for MQA in CUDA, "One KV head breaks the textbook":
// one rescale per tile, not per key), so any finite score range is handled.
template <bool LO, int NDB>
__device__ __forceinline__ void raise_reference(f32x16 (&o)[NDB], bool o_live, const f32x16& s,
                                                float& m_ref, SoftmaxCtx& c, float& l_run,
                                                float& psum_prev, float& psum, bf16x8& p0,
                                                bf16x8& p1, bf16x8& lo0, bf16x8& lo1) {
    float mx = s[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32)) * c.scale_log2;
    // a row with no visible key yet (window) has m_ref = -inf and p = 0
    float k = m_ref == -__builtin_inff() ? 0.f : __builtin_ceilf(mx - m_ref);
    // NaN and -inf give 0; the cap only keeps the int conversion defined
    // (any k past 150 already makes f = 0)
    k = k > 0.f ? (k < 1073741824.f ? k : 1073741824.f) : 0.f;
    const float f = __builtin_amdgcn_ldexpf(1.f, -(int)k);
    if (o_live) {
        acc_fence(o);
#pragma unroll
        for (int db = 0; db < NDB; ++db) scale_acc(o[db], f);
        acc_fence(o);
    }
    l_run *= f;
    psum_prev *= f;
    m_ref += k;
    c.neg_m_ref = m_ref == -__builtin_inff() ? 0.f : -m_ref;
    psum = 0.f;
    float pend = 0.f;
    float sc = c.scale_log2;
#pragma unroll
    for (int i = 0; i < 16; ++i) softmax_elem<LO>(c, sc, s[i], i, psum, pend, p0, p1, lo0, lo1);
    softmax_flush<LO>(c, psum, pend, p1, lo1);
}

// True when some lane of the wave must raise its reference before the
// block's P.V (a sum past the cap, or not finite).
__device__ __forceinline__ bool block_over(float psum) {
    return __builtin_amdgcn_ballot_w64(!(psum <= kBlockSumCap)) != 0;
}


// Sliding window: a row's reference maximum is the maximum of the first
// 32-key block in which it sees a key (rows start their windows at different
// keys, so the workgroup's first block may be empty for some).  Until then
// m_ref stays -inf and p = 2^(s - 0) = 0 for its (masked) scores.
__device__ __forceinline__ void lazy_reference(const f32x16& s, float scale_log2, float& m_ref,
                                               SoftmaxCtx& c) {
    if (__builtin_amdgcn_ballot_w64(m_ref == -__builtin_inff()) == 0) return;
    float m0 = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < 16; ++i) m0 = fmaxf(m0, s[i]);
    m0 = fmaxf(m0, __shfl_xor(m0, 32)) * scale_log2;
    if (m_ref == -__builtin_inff()) m_ref = m0;
    c.neg_m_ref = m_ref == -__builtin_inff() ? 0.f : -m_ref;
}

// V^T operand reader for the P.V MFMAs (bf16, 1 KB rows): k-step c of the
// tile and dim block db read keys 16c + 8(j/4) + 4h + (j%4) (j = operand
// slot) of output dims 32 db .. 32 db + 31.
struct VReader {
    int voffA[4], voffB[4];
    __device__ __forceinline__ explicit VReader(int lane) {
        const int h = lane >> 5;
        const int grp = lane & 15;
        const int dsub = (lane >> 4) & 1;
        const int krow = 4 * h + (grp >> 2);              // + 16 c (+ 8)
        // 32-dim block db covers chunks 4 db .. 4 db + 3; this lane reads chunk
        // 4 db + cb at byte `within`.  The swizzle permutes chunks within
        // aligned groups of 16, so with db = 4 u + w the offset is voff[w] + 256 u.
        const int cb = 2 * dsub + ((grp & 3) >> 1);
        const int within = 8 * (grp & 1);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            voffA[w] = krow * kRowBytes + (((4 * w + cb) ^ swz(krow)) << 4) + within;
            voffB[w] = (krow + 8) * kRowBytes + (((4 * w + cb) ^ swz(krow + 8)) << 4) + within;
        }
    }
    __device__ __forceinline__ bf16x8 read(const ATTN_LDS char* sV, int c, int db) const {
        const int rel = 16 * c * kRowBytes + 256 * (db >> 2);  // swz(16c + k) == swz(k)
        const bf16x4 va = lds_read_tr16(sV + voffA[db & 3] + rel);
        const bf16x4 vb = lds_read_tr16(sV + voffB[db & 3] + rel);
        return __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7);
    }
};

// The same reader for bf16 head-dim-256 tiles (512-byte rows, swzN): the lane
// reads chunk 4 db + cb of rows krow (+ 8) + 16 c.  krow < 16, so the row's
// swizzle is swzN(krow) ^ 16 (c % 2); with cb < 4 the chunk field is
// (4 db) ^ (cb ^ swizzle), so one address per parity of c takes the dim block
// by XOR (bits 6..8) and the k-step by adding 16 rows.
struct VReaderN {
    int offA[2], offB[2];
    __device__ __forceinline__ explicit VReaderN(int lane) {
        const int h = lane >> 5;
        const int grp = lane & 15;
        const int dsub = (lane >> 4) & 1;
        const int krow = 4 * h + (grp >> 2);
        const int cb = 2 * dsub + ((grp & 3) >> 1);
        const int within = 8 * (grp & 1);
#pragma unroll
        for (int par = 0; par < 2; ++par) {
            offA[par] = krow * 512 + within + ((cb ^ swzN(krow) ^ (16 * par)) << 4);
            offB[par] = (krow + 8) * 512 + within + ((cb ^ swzN(krow + 8) ^ (16 * par)) << 4);
        }
    }
    __device__ __forceinline__ bf16x8 read(const ATTN_LDS char* sV, int c, int db) const {
        const int rel = 16 * c * 512;
        const bf16x4 va = lds_read_tr16(sV + ((offA[c & 1] ^ (64 * db)) + rel));
        const bf16x4 vb = lds_read_tr16(sV + ((offB[c & 1] ^ (64 * db)) + rel));
        return __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7);
    }
};

// FP8 V^T operand reader (ds_read_b64_tr_b8): within each 16-lane group G,
// lane 2 j + hh addresses key row 16 c + 8 (j / 4) + 4 (G / 2) + (j % 4) at
// byte 32 db + 16 (G % 2) + 8 hh, and lane i of the group receives dim
// 32 db + 16 (G % 2) + i of those 8 rows: the A operand of the 32x32x16 MFMA
// (row = lane % 32, k-slot = 8 (lane / 32) + j) with the same keys per slot as
// the bf16 reader, i.e. as the P^T operand.  The row's swizzle is
// (k0 + 16 (c % 2)) for the in-block key k0, so the reader keeps one
// precomputed address per parity of c and XORs in the dim block.
struct VReader8 {
    int w[2];
    __device__ __forceinline__ explicit VReader8(int lane) {
        const int G = lane >> 4, i = lane & 15, j = i >> 1, hh = i & 1;
        const int k0 = 8 * (j >> 2) + 4 * (G >> 1) + (j & 3);
        const int vbase = k0 * kHeadDim + 8 * hh;
#pragma unroll
        for (int par = 0; par < 2; ++par)
            w[par] = vbase | ((((G & 1) ^ swz8(k0 + 16 * par))) << 4);
    }
    // raw E4M3 bytes of the operand (widened to bf16 just before the MFMA)
    __device__ __forceinline__ v2i32 read(const ATTN_LDS char* sV, int c, int db) const {
        return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (ATTN_LDS v2i32*)(sV + 16 * c * kHeadDim + (w[c & 1] ^ (2 * db << 4))));
    }
};

// LDS operand reads of the two products.  A phase's first kPrefetchOf reads
// are issued by the phase before it, right after the barrier that opens the
// phase (see qk_block), into a ring the tile loop owns.
template <bool FP8>
using RawOf = typename std::conditional<FP8, v2i32, bf16x8>::type;

// K operand of k-step ks of 32-key block kb.  bf16 at 512: step ks reads
// chunk 2 ks + h of key row 32 kb + n; with ks = 8 u + v the byte offset is
// koff[v] + 256 u + 32 KiB kb.  bf16 at 256: chunk (2 ks + h) ^ swzN(n) =
// (2 ks) ^ (h ^ swzN(n)): koff[0] ^ (32 ks) + 16 KiB kb.  FP8: bytes 16 ks +
// 8 h of row 32 kb + n, chunk ks at ks ^ n: koff[0] ^ (16 ks) + 16 KiB kb.
// FP8 operands are read as raw bytes and widened at their MFMA.
template <bool FP8, int D>
__device__ __forceinline__ RawOf<FP8> k_operand(const ATTN_LDS char* sK, const int (&koff)[8],
                                                int kb, int ks) {
    if constexpr (FP8)
        return *(const ATTN_LDS v2i32*)(sK + (koff[0] ^ (ks << 4)) + kb * 32 * 512);
    else if constexpr (Kv<FP8, D>::kNarrow)
        return *(const ATTN_LDS bf16x8*)(sK + (koff[0] ^ (ks << 5)) + kb * 32 * 512);
    else
        return *(const ATTN_LDS bf16x8*)(sK + koff[ks & 7] + 256 * (ks >> 3) +
                                          kb * 32 * kRowBytes);
}

// V^T operand of MFMA step st of P.V block kb: k-step 2 kb + st / kDB of the
// tile, dim block st % kDB.
template <bool FP8, int D, typename VR>
__device__ __forceinline__ RawOf<FP8> v_operand(const ATTN_LDS char* sV, const VR& vr, int kb,
                                                int st) {
    constexpr int kDB = Kv<FP8, D>::kDimBlocks;
    return vr.read(sV, 2 * kb + st / kDB, st % kDB);
}

// MFMAs each phase leaves for after the barrier that opens the next phase.
// Their operands are already in registers, so they keep the matrix core busy
// while the barrier releases and the next phase's first operand reads come
// back from LDS, which would otherwise leave it idle at every phase start.
// All phases share one operand ring, and held step i reads slot i (the step
// count minus the held count is a multiple of the ring size), so the next
// phase's read i refills the slot its held MFMA has just taken: no register
// holds more than one operand at a time.  Measured on the 8192- and 2048-row
// chunks, holding the whole ring (4) took 0.7 % and 3 % off the launch time
// on a bf16 pool; the FP8 pool's kernel (ring of 3, so at most 2 held) ran no
// faster and holds none.
template <bool FP8>
constexpr int kHoldOf = FP8 ? 0 : 4;

// Q.K^T of one 32-key block kb: D / 16 MFMAs (VGPR accumulator) over the
// k-steps of head_dim, operands from the ring `kbuf` (filled here unless PRE:
// then the previous phase read them).  When OVERLAP, the 16 softmax elements
// of the previous block's scores `sp` are spread evenly over the MFMAs (one
// after every other at D = 512, one after each at 256); the half-tile refill
// `dma` issues one row load after every fourth MFMA.  `pre` (the previous
// block's masking and reference, which the softmax needs but the chain does
// not) runs after the first MFMA is issued, so that it overlaps the matrix
// pipe.  The last HOLD MFMAs (and the softmax elements beside them) are
// issued after `sync()` (the wait and barrier that open the next phase),
// interleaved with `fill(i)`, the next phase's first operand reads.  Without
// a next phase (tail_on false) there is no barrier to wait for, and the
// reads are still issued (in-bounds LDS reads whose values go unused), so
// that the ring holds one version of its values at every point.
template <bool OVERLAP, bool FP8, int D, bool LO, bool PRE, int HOLD, typename Pre, typename Sync,
          typename Fill>
__device__ __forceinline__ void qk_block(f32x16& s, int kb, const bf16x8 (&qf)[(Kv<FP8, D>::kSteps)],
                                         const ATTN_LDS char* sK, const int (&koff)[8],
                                         RawOf<FP8> (&kbuf)[kPrefetchOf<FP8>],
                                         const f32x16& sp, const SoftmaxCtx& c, float& psum,
                                         bf16x8& pf0, bf16x8& pf1, bf16x8& lo0, bf16x8& lo1,
                                         const HalfDma& dma, int lane_off, int lane, int wave,
                                         Pre&& pre, bool tail_on, Sync&& sync, Fill&& fill) {
    constexpr int kSteps = Kv<FP8, D>::kSteps;
    constexpr int kP = kPrefetchOf<FP8>;
    static_assert(HOLD >= 0 && HOLD <= kP && HOLD < kSteps, "held MFMAs");
    // held step i must read ring slot i (see kHoldOf)
    static_assert(HOLD == 0 || (kSteps - HOLD) % kP == 0, "held steps and ring slots");
    constexpr int kDmaEvery = kSteps / Kv<FP8, D>::kDmaPerHalf;
    constexpr int kSmEvery = kSteps / 16;
    float pend = 0.f;   // p of the previous softmax element
    float sc = c.scale_log2;
    // MFMA of step ks and the softmax element placed after it
    auto step = [&](auto KS) {
        constexpr int ks = decltype(KS)::value;
        const bf16x8 cur = operand(kbuf[ks % kP]);
        if (ks + kP < kSteps) kbuf[ks % kP] = k_operand<FP8, D>(sK, koff, kb, ks + kP);
        if constexpr (FP8) {   // cur was just written by the widening VALU ops
            if constexpr (ks == 0)
                mfma32x32x16_vgpr_first_va(s, cur, qf[0]);
            else
                mfma32x32x16_vgpr_va(s, cur, qf[ks]);
        } else {
            if constexpr (ks == 0)
                mfma32x32x16_vgpr_first(s, cur, qf[0]);
            else
                mfma32x32x16_vgpr(s, cur, qf[ks]);
        }
        if constexpr (ks == 0) pre();
        if constexpr (OVERLAP && (ks % kSmEvery == kSmEvery - 1)) {
            constexpr int i = ks / kSmEvery;
            softmax_elem<LO>(c, sc, sp[i], i, psum, pend, pf0, pf1, lo0, lo1);
        }
    };
    if constexpr (!PRE) {
#pragma unroll
        for (int j = 0; j < kP; ++j) kbuf[j] = k_operand<FP8, D>(sK, koff, kb, j);
    }
    static_for<kSteps>([&](auto KS) {
        constexpr int ks = decltype(KS)::value;
        if constexpr (ks < kSteps - HOLD) step(KS);
        if constexpr (ks % kDmaEvery == 0) {
            if (dma.on) half_dma_row<FP8, D, ks / kDmaEvery>(dma, lane_off, lane, wave);
        }
        __builtin_amdgcn_sched_barrier(0);
    });
    if (tail_on) sync();
    static_for<kP>([&](auto I) {
        constexpr int i = decltype(I)::value;
        if constexpr (i < HOLD) step(std::integral_constant<int, kSteps - HOLD + i>{});
        __builtin_amdgcn_sched_barrier(0);
        fill(I);
        __builtin_amdgcn_sched_barrier(0);
    });
    if constexpr (OVERLAP) softmax_flush<LO>(c, psum, pend, pf1, lo1);
}

// P.V of one 32-key block (k-steps c = 2 kb, 2 kb + 1 of the tile, all D / 32
// dim blocks), operands from the ring `vbuf` (filled here unless PRE).
// FIRST: the tile's first k-step starts O from zero (inline c = 0), so O is
// only ever written by MFMAs.  LO: P carries a second bf16 term (p0lo, p1lo;
// the range's first tile), multiplied into O by a second MFMA on the same V
// operand when lo_on (wave-uniform); LO_NEXT: the overlapped softmax of the
// next block produces its second term too.  When OVERLAP, the 16 softmax
// elements of the next block's scores `sn` are spread evenly over the MFMAs
// (`pre`, run after the first MFMA, readies them); the half-tile refill
// `dma` issues one row load after every fourth MFMA.  HOLD, sync, fill and
// tail_on as in qk_block.
template <bool FIRST, bool OVERLAP, bool FP8, int D, bool LO, bool LO_NEXT, bool PRE, int HOLD,
          typename VR, typename Pre, typename Sync, typename Fill>
__device__ __forceinline__ void pv_block(f32x16 (&o)[(Kv<FP8, D>::kDimBlocks)], int kb,
                                         const bf16x8& p0, const bf16x8& p1,
                                         const bf16x8& p0lo, const bf16x8& p1lo,
                                         const ATTN_LDS char* sV, const VR& vr,
                                         RawOf<FP8> (&vbuf)[kPrefetchOf<FP8>], const f32x16& sn,
                                         const SoftmaxCtx& c, float& psum,
                                         bf16x8& pn0, bf16x8& pn1, bf16x8& ln0, bf16x8& ln1,
                                         const HalfDma& dma, int lane_off, int lane, int wave,
                                         bool lo_on, Pre&& pre, bool tail_on, Sync&& sync,
                                         Fill&& fill) {
    constexpr int kDB = Kv<FP8, D>::kDimBlocks;
    constexpr int kMfma = 2 * kDB;
    constexpr int kP = kPrefetchOf<FP8>;
    static_assert(HOLD >= 0 && HOLD <= kP && HOLD <= kDB, "held MFMAs");
    // held step i must read ring slot i (see kHoldOf)
    static_assert(HOLD == 0 || (kMfma - HOLD) % kP == 0, "held steps and ring slots");
    constexpr int kDmaEvery = kMfma / Kv<FP8, D>::kDmaPerHalf;
    constexpr int kSmEvery = kMfma / 16;
    float pend = 0.f;   // p of the previous softmax element
    float sc = c.scale_log2;
    auto step = [&](auto ST) {
        constexpr int st = decltype(ST)::value;
        const bf16x8 cur = operand(vbuf[st % kP]);
        if (st + kP < kMfma) vbuf[st % kP] = v_operand<FP8, D>(sV, vr, kb, st + kP);
        constexpr int db = st % kDB;
        if constexpr (FIRST && st < kDB)
            o[db] = mfma32x32x16(cur, p0, f32x16{});
        else
            o[db] = mfma32x32x16(cur, st < kDB ? p0 : p1, o[db]);
        if constexpr (LO) {
            if (lo_on) o[db] = mfma32x32x16(cur, st < kDB ? p0lo : p1lo, o[db]);
        }
        if constexpr (st == 0) pre();
        if constexpr (OVERLAP && (st % kSmEvery == kSmEvery - 1)) {
            constexpr int i = st / kSmEvery;
            softmax_elem<LO_NEXT>(c, sc, sn[i], i, psum, pend, pn0, pn1, ln0, ln1);
        }
    };
    if constexpr (!PRE) {
#pragma unroll
        for (int j = 0; j < kP; ++j) vbuf[j] = v_operand<FP8, D>(sV, vr, kb, j);
    }
    static_for<kMfma>([&](auto ST) {
        constexpr int st = decltype(ST)::value;
        if constexpr (st < kMfma - HOLD) step(ST);
        if constexpr (st % kDmaEvery == 0) {
            if (dma.on) half_dma_row<FP8, D, st / kDmaEvery>(dma, lane_off, lane, wave);
        }
        __builtin_amdgcn_sched_barrier(0);
    });
    if (tail_on) sync();
    static_for<kP>([&](auto I) {
        constexpr int i = decltype(I)::value;
        if constexpr (i < HOLD) step(std::integral_constant<int, kMfma - HOLD + i>{});
        __builtin_amdgcn_sched_barrier(0);
        fill(I);
        __builtin_amdgcn_sched_barrier(0);
    });
    if constexpr (OVERLAP) softmax_flush<LO_NEXT>(c, psum, pend, pn1, ln1);
}

// PERSIST: the grid is one workgroup per compute unit, and each workgroup
// takes work units, heaviest first, from counters at a.unit_counter (zeroed
// by prefill_counter_reset on the same stream); otherwise workgroup i does
// unit i.  Units are dealt to the XCDs as the one-per-unit launch deals its
// workgroups (unit u to XCD u % 8, which keeps one KV head's K/V per XCD's
// L2 when the KV head count divides 8): a workgroup drains the queue of the
// XCD it runs on (units x, x + 8, ...), then helps with the other queues, so
// every unit is done whatever the dispatcher's placement.
template <bool OUT_FP32, bool FP8, bool SPLIT, int D = kHeadDim, bool WINDOW = false,
          bool APPEND = false, bool PERSIST = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void prefill_hd512_kernel(PrefillArgs a) {
    static_assert(!(SPLIT && (WINDOW || D != kHeadDim)), "split-K: head dim 512, no window");
    static_assert(!APPEND || (!FP8 && !SPLIT && !WINDOW && D == kHeadDim),
                  "fused append: bf16 pool, head dim 512, single pass");
    static_assert(!PERSIST || (!SPLIT && !WINDOW && !APPEND && D == kHeadDim),
                  "persistent: single pass, head dim 512");
    constexpr int kTileB = Kv<FP8, D>::kTileB;
    constexpr int kD = Kv<FP8, D>::kDmaPerHalf;   // loads per wave per half refill
    constexpr int kSteps = Kv<FP8, D>::kSteps;
    constexpr int kDB = Kv<FP8, D>::kDimBlocks;
    __shared__ __attribute__((aligned(1024))) char smem[2 * kTileB];
    __shared__ int sPage[kPagesInLds];
    ATTN_LDS char* sK = (ATTN_LDS char*)smem;
    ATTN_LDS char* sV = sK + kTileB;

    const int lane0 = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    // One work unit; a unit with nothing to do returns at once.  at_end()
    // runs once the unit's key loop is done, before its epilogue.
    auto run_unit = [&](const int unit, auto&& at_end) {
    // The lane's offsets are derived from an opaque copy of its index, so
    // that a persistent workgroup recomputes them per unit instead of
    // keeping them live across its epilogues and prologues.
    int lane = lane0;
    if constexpr (PERSIST) asm volatile("" : "+v"(lane));
    // ---- work unit: heaviest query tiles first; KV head fastest so that
    // consecutive workgroups (spread round-robin over the XCDs) share a KV
    // head per XCD whenever the KV head count divides 8.
    const int per_rank = a.batch * a.hkv;
    const int per_split = a.wgs_per_seq * per_rank;
    const int split = SPLIT ? unit / per_split : 0;
    const int in_split = unit - split * per_split;
    const int rank = in_split / per_rank;
    const int rem = in_split - rank * per_rank;
    const int kvh = rem % a.hkv;
    const int b = rem / a.hkv;
    const int wg_in_seq = a.wgs_per_seq - 1 - rank;

    int q0 = a.cu_seqlens_q[b];
    int q1 = a.cu_seqlens_q[b + 1];
    q0 = q0 < 0 ? 0 : (q0 > a.total_q ? a.total_q : q0);
    q1 = q1 < q0 ? q0 : (q1 > a.total_q ? a.total_q : q1);
    const int q_len = q1 - q0;
    const int t0 = wg_in_seq * a.tok_per_wg;
    if (t0 >= q_len) return;
    const int t_last = min(t0 + a.tok_per_wg, q_len) - 1;
    int L = a.kv_lens[b];
    // positions index the page table directly unless the cache is a ring
    // (then any tile maps to table entry tile % ring_pages; windowed kernels only)
    const int ring = WINDOW ? a.ring_pages : 0;
    const int L_cap = ring > 0 ? 0x7fffffff - kPage : a.max_pages * kPage;
    L = L < 0 ? 0 : (L > L_cap ? L_cap : L);
    const int qs = max(a.q_start[b], 0);   // every row then sees key 0 (or its window)
    const int n_max = min(qs + t_last + 1, L);   // keys the last row sees
    const int n_min = min(qs + t0 + 1, L);       // keys the first row sees
    // window: row at position p sees keys [p - window + 1, p]; lo_first and
    // lo_last are the first and last rows' lower ends
    const int lo_first = WINDOW ? max(0, qs + t0 - a.window + 1) : 0;
    const int lo_last = WINDOW ? max(0, qs + t_last - a.window + 1) : 0;
    const int ntiles_all = n_max > 0 ? (n_max + kPage - 1) / kPage : 0;
    // this workgroup's key tiles [kt_lo, ntiles): all of them, one split, or
    // those from the first row's window start
    const int kt_lo = SPLIT ? split * a.split_tiles : (WINDOW ? lo_first / kPage : 0);
    const int ntiles = SPLIT ? min(ntiles_all, kt_lo + a.split_tiles) : ntiles_all;
    if (SPLIT && kt_lo >= ntiles) return;   // no row of this unit needs the split

    // ---- this lane's query row: n = column of the MFMA tiles, h = k-half
    const int n = lane & 31;
    const int h = lane >> 5;
    const int r = wave * 32 + n;
    const int tr = r / a.g;
    const bool valid = (tr < a.tok_per_wg) && (t0 + tr <= t_last);
    const int t = valid ? t0 + tr : t_last;      // padding rows shadow the last real token
    const int head = kvh * a.g + (valid ? r - tr * a.g : 0);
    const int n_row = min(qs + t + 1, L);
    const int lo_row = WINDOW ? max(0, qs + t - a.window + 1) : 0;

    // ---- Q^T operand: k-step ks covers head dims 16 ks .. 16 ks + 15; this
    // lane holds dims 16 ks + 8 h .. + 7 of its row.
    bf16x8 qf[kSteps];
    {
        const bf16x8* qp =
            (const bf16x8*)(a.q + ((size_t)(q0 + t) * a.hq + head) * D) + h;
#pragma unroll
        for (int ks = 0; ks < kSteps; ++ks) {
            bf16x8 v = qp[2 * ks];
            qf[ks] = valid ? v : bf16x8{};
        }
    }
    int koff[8];
    if constexpr (FP8) {
        // row n, chunk 0 at n ^ 0, byte 8 h; step ks XORs in 16 ks
        koff[0] = n * 512 + (swz8(n) << 4) + 8 * h;
#pragma unroll
        for (int v = 1; v < 8; ++v) koff[v] = koff[0];
    } else if constexpr (Kv<FP8, D>::kNarrow) {
        // row n, chunk h at h ^ swzN(n); step ks XORs in 32 ks
        koff[0] = n * 512 + ((h ^ swzN(n)) << 4);
#pragma unroll
        for (int v = 1; v < 8; ++v) koff[v] = koff[0];
    } else {
#pragma unroll
        for (int v = 0; v < 8; ++v) koff[v] = n * kRowBytes + (((2 * v + h) ^ swz(n)) << 4);
    }
    using VRd = typename std::conditional<
        FP8, VReader8, typename std::conditional<Kv<FP8, D>::kNarrow, VReaderN, VReader>::type>::type;
    const VRd vr(lane);

    f32x16 o[kDB];  // written first by the range's first P.V
    // Online softmax against a per-row reference maximum: p = 2^(x - m_ref),
    // m_ref starting as the row's maximum over its first 32 keys.  O and l
    // carry the factor 2^(m_true - m_ref), which cancels in O / l.  The
    // reference only moves when a block's sum of p passes kBlockSumCap
    // (raise_reference, before that block's P.V), so the 256 O accumulators
    // (AGPRs, which VALU cannot address) stay out of the loop's VALU code,
    // and the per-element work is one fma, one exp2, one add and a
    // conversion.
    float m_ref = -__builtin_inff();
    float l_run = 0.f;

    const int* ptab = a.page_table + (size_t)b * a.max_pages;
    const int lane16 = lane * 16;
    const int lane_off = lane16 ^ ((wave & 1) << 7);
    const int staged = min(ntiles - kt_lo, kPagesInLds);
    for (int i = threadIdx.x; i < staged; i += kThreads)
        sPage[i] = ptab[ring > 0 ? (kt_lo + i) % ring : kt_lo + i];
    // Fused append.  The chunk's keys are positions [qs, hi).  A wave's 8
    // refill rows (an aligned group of 8 positions) that all lie there come
    // from the new-row buffer; every other group comes from the pool.  This
    // workgroup writes its own tokens' K and V rows into their cache slots,
    // and also the chunk rows of the groups that straddle qs or hi in the
    // tiles it walks: those it then reads from the pool, so it waits for its
    // own writes before the barrier.  Workgroups that write one row write
    // the same bytes, and no workgroup reads a chunk row it has not written.
    if constexpr (APPEND) {
        const int hi = min(qs + q_len, L);
        const int lo8 = min((qs + 7) & ~7, hi);                    // [qs, lo8): first group
        const int hi8 = max(hi & ~7, lo8);                         // [hi8, hi): last group
        const int walked = ntiles_all * kPage;
        const int ntok = t_last - t0 + 1;
        const int nlo = max(lo8 - qs, 0);                          // none when hi <= qs
        const int nhi = max(min(hi, walked) - hi8, 0);
        const int nrow = ntok + nlo + nhi;
        // wave w moves rows w, w + 4, ... (one 1 KB row per wave instruction,
        // 16 bytes a lane), four rows of K and V in flight per batch; a row's
        // position and page are wave-uniform
        for (int r0 = wave; r0 < nrow; r0 += 16) {
            u32x4 kr[4], vr4[4];
            size_t dst[4];
            bool ok[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rr = r0 + 4 * i;
                const int pos = rr < ntok ? qs + t0 + rr
                                          : (rr < ntok + nlo ? qs + rr - ntok : hi8 + rr - ntok - nlo);
                const int pg = rr < nrow && pos / kPage < a.max_pages ? ptab[pos / kPage] : -1;
                ok[i] = pg >= 0 && pg < a.num_pages;
                dst[i] = (((size_t)pg * a.hkv + kvh) * kPage + pos % kPage) * kRowBytes + lane16;
                const size_t src = ((size_t)(q0 + pos - qs) * a.hkv + kvh) * kRowBytes + lane16;
                if (ok[i]) {
                    kr[i] = *(const u32x4*)(a.k_new + src);
                    vr4[i] = *(const u32x4*)(a.v_new + src);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (ok[i]) {
                    *(u32x4*)((char*)a.k_pages + dst[i]) = kr[i];
                    *(u32x4*)((char*)a.v_pages + dst[i]) = vr4[i];
                }
            }
        }
        // the straddling rows must be in memory before this workgroup's
        // refills read them; its own rows need no wait (their stores are
        // older than every refill load, so the loop's counted waits stay safe)
        if (nlo + nhi > 0) wait_vmcnt<0>();
    }
    race_delay<2>();
    __syncthreads();
    auto page_of = [&](int tile) -> int {
        return tile - kt_lo < kPagesInLds ? __builtin_amdgcn_readfirstlane(sPage[tile - kt_lo])
                                          : load_uniform(ptab, ring > 0 ? tile % ring : tile);
    };

    // Fused append: a group of 8 refill rows starting at position p comes
    // from the new-row buffer when qs <= p and p + 8 <= hi, i.e. when
    // p - qs_g <= g_lim unsigned (qs_g pushed out of reach when no group
    // qualifies); its bytes start (p - qs) * n_stride + n_base into the buffer.
    int qs_g = 0, g_lim = 0, n_stride = kRowBytes;
    uint32_t n_base = 0, n_bytes = 0;
    if constexpr (APPEND) {
        const int hi = min(qs + q_len, L);
        qs_g = __builtin_amdgcn_readfirstlane(hi - 8 - qs >= 0 ? qs : 0x40000000);
        g_lim = __builtin_amdgcn_readfirstlane(max(hi - 8 - qs, 0));
        n_stride = __builtin_amdgcn_readfirstlane(a.hkv * kRowBytes);
        n_base = (uint32_t)__builtin_amdgcn_readfirstlane(
            (int)(((uint32_t)q0 * (uint32_t)a.hkv + (uint32_t)kvh) * kRowBytes));
        n_bytes = (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)a.total_q * a.hkv * kRowBytes));
    }
    // refill descriptor of half `half` of tile `tile` (K or V)
    auto refill = [&](bool is_k, int page, int valid_rows, int tile, int half, bool on) -> HalfDma {
        if constexpr (!APPEND) {
            return half_dma<FP8, D>(is_k ? a.k_pages : a.v_pages, page, a.num_pages, a.hkv, kvh,
                                    valid_rows, is_k ? sK : sV, half, wave, on);
        } else {
            // the pool descriptor half_dma would build, then the source chosen
            // by scalar selects on one compare (written out so that the choice
            // costs no branch in the loop)
            const HalfDma pd = half_dma<FP8, D>(is_k ? a.k_pages : a.v_pages, page, a.num_pages,
                                                a.hkv, kvh, valid_rows, is_k ? sK : sV, half,
                                                wave, on);
            const int p = tile * kPage + 32 * half + 8 * wave;
            const uint32_t nsoff = (uint32_t)__builtin_amdgcn_readfirstlane(
                (int)((uint32_t)(p - qs) * (uint32_t)n_stride + n_base));
            const uint64_t np = (uint64_t)(uintptr_t)(is_k ? a.k_new : a.v_new);
            const uint32_t n0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)np);
            const uint32_t n1 = (uint32_t)__builtin_amdgcn_readfirstlane((int)((np >> 32) & 0xffffu));
            const uint32_t pos = (uint32_t)__builtin_amdgcn_readfirstlane(p);
            HalfDma d = pd;
            uint32_t t;
            asm volatile(
                "s_sub_u32 %[t], %[pos], %[qsg]\n\t"
                "s_cmp_le_u32 %[t], %[glim]\n\t"
                "s_cselect_b32 %[r0], %[n0], %[p0]\n\t"
                "s_cselect_b32 %[r1], %[n1], %[p1]\n\t"
                "s_cselect_b32 %[r2], %[nb], %[p2]\n\t"
                "s_cselect_b32 %[so], %[nso], %[pso]\n\t"
                "s_cselect_b32 %[st], %[nst], %[pst]"
                : [t] "=&s"(t), [r0] "=&s"(d.rsrc[0]), [r1] "=&s"(d.rsrc[1]),
                  [r2] "=&s"(d.rsrc[2]), [so] "=&s"(d.soff), [st] "=&s"(d.stride)
                : [pos] "s"(pos), [qsg] "s"(qs_g), [glim] "s"(g_lim), [n0] "s"(n0),
                  [p0] "s"(pd.rsrc[0]), [n1] "s"(n1), [p1] "s"(pd.rsrc[1]), [nb] "s"(n_bytes),
                  [p2] "s"(pd.rsrc[2]), [nso] "s"(nsoff), [pso] "s"(pd.soff),
                  [nst] "s"(n_stride), [pst] "s"(pd.stride)
                : "scc");
            d.app = true;
            return d;
        }
    };

    // Vector-memory accounting: every wave issues its half-tile refills in the
    // order V1(j) [during QK0(j)], K0(j+1) [QK1(j)], K1(j+1) [PV0(j)],
    // V0(j+1) [PV1(j)], kD loads each; before each phase the half it reads was
    // issued two refills (2 kD loads) before the newest.  The last tile's
    // successor refills are issued too, into halves nothing reads again, so
    // that every refill site is unconditional and every count the same; the
    // loop's end waits for them.  They re-read the last tile's own rows (its
    // page, which is page_n there), already in the L2: loads over an empty
    // range would fetch nothing, but measured slower than real ones (a copy
    // whose refills all had no records ran 22 % slower than the kernel).
    // P in two bf16 terms in the first tile (see the tile below)
    const bool lo_on = n_min - max(kt_lo * kPage, lo_first) <= kLoKeys;
    int page_cur = ntiles > kt_lo ? page_of(kt_lo) : 0;              // page of tile kt
    int page_nx = kt_lo + 1 < ntiles ? page_of(kt_lo + 1) : page_cur;  // of tile kt + 1
    if (ntiles > kt_lo) {
        const int page0 = page_cur;
        const int v0 = min(L - kt_lo * kPage, kPage);
        half_dma_all<FP8, D>(refill(true, page0, v0, kt_lo, 0, true), lane_off, lane, wave);
        half_dma_all<FP8, D>(refill(true, page0, v0, kt_lo, 1, true), lane_off, lane, wave);
        half_dma_all<FP8, D>(refill(false, page0, v0, kt_lo, 0, true), lane_off, lane, wave);
    }
    // The operand ring `opr` of the phases (each phase's first reads are issued by
    // the phase before it), and the wait and barrier that open every phase: before each phase the half
    // it reads was issued two refills (2 kD loads) before the newest.
    constexpr int kHold = kHoldOf<FP8>;
    RawOf<FP8> opr[kPrefetchOf<FP8>];
    auto sync = [&] {
        wait_vmcnt<2 * kD>();
        lds_barrier();
    };
    // One 64-key tile.  kFirst (the range's first tile, peeled off the loop):
    // the reference maximum is taken, P.V starts O from zero, and P can carry
    // its second bf16 term, which it does when the block's first row sees at
    // most kLoKeys keys of the range (lo_on; bf16 P's relative error per
    // weight only shows in rows with few keys): otherwise the second terms
    // are zero and their MFMAs are skipped.
    auto tile = [&](auto first_tag, int kt) {
        constexpr bool kFirst = decltype(first_tag)::value;
        constexpr bool kLo = kFirst;
        const bool more = kt + 1 < ntiles;
        const int key0 = kt * kPage;
        const int valid = min(L - key0, kPage);
        // the last tile's successor refills re-read its own rows (see above)
        const int valid_n = more ? min(L - key0 - kPage, kPage) : valid;
        const int page = page_cur;
        const int page_n = page_nx;
        // page id of tile kt + 2: the LDS read is issued here and its value
        // taken after QK0, so that its latency hides under QK0's MFMAs (the
        // index is clamped into the staged range; past it the id comes from
        // the table after QK0)
        const int t2 = kt + 2;
        const bool t2_staged = t2 - kt_lo < kPagesInLds;
        const int page_nn_raw = sPage[min(t2 - kt_lo, kPagesInLds - 1)];
        // the tile crosses a row's causal limit (or a row's window start)
        const bool mask = key0 + kPage > n_min || (WINDOW && key0 < lo_last);
        SoftmaxCtx c0{a.scale_log2, WINDOW && m_ref == -__builtin_inff() ? 0.f : -m_ref,
                      lo_on ? 1.f : 0.f};
        float psum0 = 0.f, psum1 = 0.f;   // the lane's sums of p of blocks 0 and 1
        bf16x8 pf[4];
        bf16x8 pl[4];                     // second terms (kLo only)
        f32x16 s0, s1;

        // ---- QK0: reads K rows 0..31 of tile kt; V rows 32..63 of kt refill.
        // Past the range's first tile the barrier that opens QK0 was taken at
        // the end of the previous tile's PV1, which also read QK0's first
        // operands into `opr` and issued its own last MFMAs after it.  Every
        // phase ends the same way: its last kHold MFMAs go out after the next
        // phase's barrier, beside that phase's first operand reads.  Each
        // refill is named after the barrier of the phase that issues it,
        // where those held MFMAs cover the address work.
        if constexpr (kFirst) sync();
        const HalfDma dv1 = refill(false, page, valid, kt, 1, true);
        qk_block<false, FP8, D, false, !kFirst, kHold>(
            s0, 0, qf, sK, koff, opr, s0, c0, psum0, pf[0], pf[1], pl[0], pl[1], dv1, lane_off,
            lane, wave, [] {}, true, sync,
            [&](auto I) { opr[decltype(I)::value] = k_operand<FP8, D>(sK, koff, 1, I); });
        page_cur = page_n;
        page_nx = t2 >= ntiles ? page_n
                : (t2_staged ? __builtin_amdgcn_readfirstlane(page_nn_raw)
                             : load_uniform(ptab, ring > 0 ? t2 % ring : t2));

        // ---- QK1 with block 0's softmax; K rows 0..31 of tile kt+1 refill.
        // Block 0's masking and reference run after QK1's first MFMA.
        const HalfDma dk0 = refill(true, page_n, valid_n, kt + 1, 0, true);
        qk_block<true, FP8, D, kLo, true, kHold>(
            s1, 1, qf, sK, koff, opr, s0, c0, psum0, pf[0], pf[1], pl[0], pl[1], dk0, lane_off,
            lane, wave,
            [&] {
                mfma_vgpr_drain(s0);
                if (mask) mask_block<WINDOW>(s0, key0 + 4 * h, n_row, lo_row);
                if constexpr (WINDOW) lazy_reference(s0, a.scale_log2, m_ref, c0);
                if constexpr (!WINDOW && kFirst) {
                    // reference maximum: the row's maximum over the range's
                    // first 32 keys.  Without split-K key 0 is visible to
                    // every row, so it is finite; a split can start past a
                    // row's causal limit, and that row then takes 0 (every
                    // p = 0, an empty partial).
                    float m0 = -__builtin_inff();
#pragma unroll
                    for (int i = 0; i < 16; ++i) m0 = fmaxf(m0, s0[i]);
                    m0 = fmaxf(m0, __shfl_xor(m0, 32)) * a.scale_log2;
                    m0 = m0 == -__builtin_inff() ? 0.f : m0;
                    m_ref = m0;
                    c0.neg_m_ref = -m0;
                }
            },
            true, sync,
            [&](auto I) { opr[decltype(I)::value] = v_operand<FP8, D>(sV, vr, 0, I); });
        // block 0's P must be representable before its P.V (O is still
        // unwritten in the first tile)
        const bool over0 = block_over(psum0);

        // ---- PV0 with block 1's softmax; K rows 32..63 of tile kt+1 refill.
        // Block 1's masking runs after PV0's first MFMA (the last MFMAs of
        // its Q.K^T went out after the barrier).
        if (__builtin_expect(over0, 0)) {
            float none = 0.f;
            raise_reference<kLo>(o, !kFirst, s0, m_ref, c0, l_run, none, psum0, pf[0], pf[1],
                                    pl[0], pl[1]);
        }
        const HalfDma dk1 = refill(true, page_n, valid_n, kt + 1, 1, true);
        pv_block<kFirst, true, FP8, D, kLo, kLo, true, kHold>(
            o, 0, pf[0], pf[1], pl[0], pl[1], sV, vr, opr, s1, c0, psum1, pf[2], pf[3], pl[2],
            pl[3], dk1, lane_off, lane, wave, lo_on,
            [&] {
                mfma_vgpr_drain(s1);
                if (mask) mask_block<WINDOW>(s1, key0 + 32 + 4 * h, n_row, lo_row);
                if constexpr (WINDOW) lazy_reference(s1, a.scale_log2, m_ref, c0);
            },
            true, sync,
            [&](auto I) { opr[decltype(I)::value] = v_operand<FP8, D>(sV, vr, 1, I); });
        // block 1's P likewise (O now holds block 0 of this tile as well)
        const bool over1 = block_over(psum1);

        // ---- PV1; V rows 0..31 of tile kt+1 refill.  Its tail opens the
        // next tile's QK0 (there is none after the range's last tile).
        if (__builtin_expect(over1, 0))
            raise_reference<kLo>(o, true, s1, m_ref, c0, l_run, psum0, psum1, pf[2], pf[3],
                                    pl[2], pl[3]);
        const HalfDma dv0 = refill(false, page_n, valid_n, kt + 1, 0, true);
        pv_block<false, false, FP8, D, kLo, false, true, kHold>(
            o, 1, pf[2], pf[3], pl[2], pl[3], sV, vr, opr, s1, c0, psum1, pf[2], pf[3], pl[2],
            pl[3], dv0, lane_off, lane, wave, lo_on, [] {}, more, sync,
            [&](auto I) { opr[decltype(I)::value] = k_operand<FP8, D>(sK, koff, 0, I); });
        l_run += psum0 + psum1;
    };
    if (ntiles > kt_lo) {
        tile(std::true_type{}, kt_lo);
        for (int kt = kt_lo + 1; kt < ntiles; ++kt) tile(std::false_type{}, kt);
    }
    wait_vmcnt<0>();   // the empty refills past the last tile

    at_end();

    // ---- epilogue: outputs (or split-K partials) of the workgroup's rows
    constexpr bool kStageOut = !OUT_FP32 && 2 * kTileB >= kWaves * 32 * D * 2;
    prefill_epilogue<OUT_FP32, SPLIT, D, kStageOut, FP8>(
        a, o, l_run, m_ref, ntiles > kt_lo,
        RowSlot{q0, q0 + t, head, t0, t_last, kvh, split, valid}, (ATTN_LDS char*)smem, lane,
        wave);
    };

    if constexpr (PERSIST) {
        // HW_REG_XCC_ID (hardware register 20), bits 0..3: this XCD
        const int xcd = (int)(__builtin_amdgcn_s_getreg((3 << 11) | 20) & 7);
        // Thread 0 takes the next unit: from this XCD's queue, then from the
        // others in turn once a queue's counter has passed the last unit;
        // a.total_units when all are drained.
        int qi = 0;
        auto take = [&]() -> int {
            while (qi < kXcds) {
                const int queue = (xcd + qi) & (kXcds - 1);
                const int u =
                    queue + kXcds * atomicAdd(a.unit_counter + kCounterStride * queue, 1);
                if (u < a.total_units) return u;
                ++qi;
            }
            return a.total_units;
        };
        // The next unit is taken when the current one's key loop is done, so
        // that the atomic's round trip overlaps the epilogue (taken earlier,
        // heavy units would no longer pair with light ones).  Every wave
        // reads the index from LDS after the barrier that ends the unit, and
        // all leave the loop together.
        __shared__ int sUnit;
        if (threadIdx.x == 0) sUnit = take();
        race_delay<2>();
        __syncthreads();
        for (;;) {
            const int unit = sUnit;
            if (unit >= a.total_units) break;
            bool taken = false;
            run_unit(unit, [&] {
                if (threadIdx.x == 0) sUnit = take();   // every wave has read sUnit by now
                taken = true;
            });
            if (!taken && threadIdx.x == 0) sUnit = take();   // a unit with no work
            // the next unit rewrites the page ids and tile buffers only after
            // every wave is done with them (the unit's loads have all landed;
            // its output stores may still be in flight: they only lengthen the
            // next unit's counted waits, which then cover older operations)
            race_delay<2>();
            __syncthreads();
        }
    } else {
        run_unit(blockIdx.x, [] {});
    }
}

// Zeroes the persistent prefill's unit counters (a kernel, not a memset, so
// that the pair can also be recorded into a graph).
__global__ void prefill_counter_reset(int* counter) {
    if (threadIdx.x < kXcds) counter[kCounterStride * threadIdx.x] = 0;
}


// Merge of the split-K partials of one (query row, query head): the partial
// of split s is O_s (times v_scale), m_s (log2 units) and l_s, with O_s and
// l_s relative to 2^{m_s}; the row's result is sum_s 2^{m_s - top} O_s /
// (2^{sink - top} + sum_s 2^{m_s - top} l_s), top the largest exponent.
// Grid: one 128-lane workgroup per (row, head); lane i owns dims 4i .. 4i+3.
template <bool OUT_FP32>
__global__ __launch_bounds__(128) void prefill_merge_kernel(PrefillArgs a, int rows_cap) {
    const int head = blockIdx.x % a.hq;
    const int row = blockIdx.x / a.hq;
    auto cu = [&](int i) {
        const int v = a.cu_seqlens_q[i];
        return v < 0 ? 0 : (v > a.total_q ? a.total_q : v);
    };
    // the sequence holding the row: the last b with cu[b] <= row
    int lo = 0, hi = a.batch - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cu(mid) <= row) lo = mid; else hi = mid - 1;
    }
    const int b = lo;
    const int q0 = cu(b);
    const int q1 = max(q0, cu(b + 1));
    const int t = row - q0;
    if (row < q0 || row >= q1 || t >= rows_cap) return;   // a row the split kernel skipped
    int L = a.kv_lens[b];
    L = L < 0 ? 0 : (L > a.max_pages * kPage ? a.max_pages * kPage : L);
    const int n_row = min(max(a.q_start[b], 0) + t + 1, L);
    const int split_keys = a.split_tiles * kPage;
    const int ns = min((n_row + split_keys - 1) / split_keys, a.nsplit);
    const size_t slot0 = (size_t)row * a.hq + head;
    const size_t stride = (size_t)a.total_q * a.hq;
    const float sink2 = a.sinks ? a.sinks[head] * 1.4426950408889634f : -__builtin_inff();
    float top = sink2;
    for (int s = 0; s < ns; ++s) top = fmaxf(top, a.part_ml[2 * (slot0 + s * stride)]);
    f32x4 acc = f32x4{};
    float den = 0.f;
    const int d0 = 4 * threadIdx.x;
    if (top != -__builtin_inff()) {
        for (int s = 0; s < ns; ++s) {
            const size_t slot = slot0 + s * stride;
            const float m = a.part_ml[2 * slot];
            if (m == -__builtin_inff()) continue;   // a split the row saw no key of
            const float w = fast_exp2(m - top);
            den += w * a.part_ml[2 * slot + 1];
            acc += w * *(const f32x4*)(a.part_o + slot * kHeadDim + d0);
        }
        den += fast_exp2(sink2 - top);   // 0 without a sink
    }
    // IEEE division as in the single-pass epilogue; no key and no sink gives 0
    const float dd = den > 0.f ? den : 1.f;
    const size_t obase = slot0 * kHeadDim + d0;
    const f32x4 v = {acc[0] / dd, acc[1] / dd, acc[2] / dd, acc[3] / dd};
    if constexpr (OUT_FP32) {
        *(f32x4*)((float*)a.out + obase) = v;
    } else {
        *(bf16x4*)((__bf16*)a.out + obase) =
            bf16x4{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
    }
    if (a.lse && threadIdx.x == 0)
        a.lse[slot0] = den > 0.f ? (top + __builtin_log2f(den)) * 0.6931471805599453f
                                 : -__builtin_inff();
}

}  // namespace

}  // namespace attn

namespace attn {
namespace {

// Split-K plan of a prefill launch: nsplit ranges of split_tiles key tiles.
// A workgroup fills a compute unit (its LDS and registers), so a launch of
// u equal workgroups takes ceil(u / kCus) rounds of one workgroup's time,
// which shrinks as 1 / nsplit.  The default picks the split count that
// minimises ceil(u / kCus) / u, charged kSplitCost per range for the
// partial traffic, the merge and each range's pipeline start; ranges keep
// at least kMinSplitTiles tiles.  One range means the single-pass kernel.
constexpr int kCus = 256;               // compute units of a gfx950 part
// the persistent launch's queue counters, one 128-byte line each
constexpr size_t kPersistWorkspace = sizeof(int) * kCounterStride * kXcds;
constexpr int kMinSplitTiles = 8;
constexpr int kMaxAutoSplits = 64;
constexpr double kSplitCost = 0.02;

struct SplitPlanK {
    int nsplit, split_tiles;
};

SplitPlanK prefill_split_plan(long long base_wgs, int max_kv_len, int keys_per_split) {
    const int max_tiles = (max_kv_len + kPage - 1) / kPage;
    if (max_tiles < 1 || base_wgs < 1) return {1, max_tiles > 0 ? max_tiles : 1};
    int st = max_tiles;
    if (keys_per_split > 0) {
        st = keys_per_split / kPage;
    } else {
        const int cap = min(kMaxAutoSplits, max(1, max_tiles / kMinSplitTiles));
        double best = 0.0;
        for (int ns = 1; ns <= cap; ++ns) {
            const int t = (max_tiles + ns - 1) / ns;
            const int real = (max_tiles + t - 1) / t;   // ranges after rounding
            if (real != ns) continue;
            const double u = (double)base_wgs * ns;
            const double rounds = (double)((long long)(u + kCus - 1) / kCus);
            const double cost = rounds / u * (ns == 1 ? 1.0 : 1.0 + kSplitCost * ns);
            if (ns == 1 || cost < best) {
                best = cost;
                st = t;
            }
        }
    }
    return {(max_tiles + st - 1) / st, st};
}

template <bool FP8, int D, bool WINDOW>
void launch_single(const PrefillArgs& a, bool out_fp32, dim3 gd, hipStream_t stream) {
    if (out_fp32)
        hipLaunchKernelGGL((prefill_hd512_kernel<true, FP8, false, D, WINDOW>), gd, dim3(kThreads),
                           0, stream, a);
    else
        hipLaunchKernelGGL((prefill_hd512_kernel<false, FP8, false, D, WINDOW>), gd,
                           dim3(kThreads), 0, stream, a);
}

int prefill_launch(const void* q, const void* k_pages, const void* v_pages, bool fp8,
                   float k_scale, float v_scale, const int32_t* page_table,
                   const int32_t* cu_seqlens_q, const int32_t* q_start_pos,
                   const int32_t* kv_lens, int batch, int total_q, int max_q_len,
                   int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                   int num_pages, int max_pages_per_seq, float softmax_scale,
                   const float* sinks, void* out, int out_dtype, float* lse,
                   bool splitk, int max_kv_len, int keys_per_split, void* workspace,
                   size_t workspace_bytes, bool swa, int window, int ring_pages,
                   const void* k_new, const void* v_new, bool fp8_mma, hipStream_t stream,
                   bool persist = false, bool check_only = false) {
    // check_only: every check runs, nothing is launched
    // the sliding-window entry is bf16 and single-pass; so is the fused append
    // (given both new-row buffers or neither), at head dim 512 with no window;
    // the FP8-MFMA form is FP8, single-pass, at head dim 512
    const bool append = k_new || v_new;
    if (persist && (splitk || swa || append || fp8_mma)) return ATTN_ERR_UNSUPPORTED;
    if (fp8_mma && (!fp8 || swa || append)) return ATTN_ERR_UNSUPPORTED;
    if (swa && (fp8 || splitk)) return ATTN_ERR_UNSUPPORTED;
    if (append && (!k_new || !v_new)) return ATTN_ERR_NULL;
    if (append && (fp8 || splitk || swa)) return ATTN_ERR_UNSUPPORTED;
    if (!q || !k_pages || !v_pages || !page_table || !cu_seqlens_q || !q_start_pos ||
        !kv_lens || !out)
        return ATTN_ERR_NULL;
    if (batch < 1 || total_q < 0 || max_q_len < 0 || num_q_heads < 1 || num_kv_heads < 1 ||
        num_pages < 1 || max_pages_per_seq < 1 || !(softmax_scale == softmax_scale))
        return ATTN_ERR_SHAPE;
    if (fp8 && (!(k_scale > 0.f) || !(v_scale > 0.f))) return ATTN_ERR_SHAPE;
    if (num_q_heads % num_kv_heads) return ATTN_ERR_SHAPE;
    if (window < 0 || ring_pages < 0 || ring_pages > max_pages_per_seq) return ATTN_ERR_SHAPE;
    if (page_size != kPage) return ATTN_ERR_UNSUPPORTED;
    // head dim 256, windows and rings come only through attn_prefill_swa
    if (head_dim != kHeadDim && (head_dim != 256 || !swa)) return ATTN_ERR_UNSUPPORTED;
    if (!swa && (window != 0 || ring_pages != 0)) return ATTN_ERR_UNSUPPORTED;
    if (ring_pages > 0 && window == 0) return ATTN_ERR_SHAPE;   // a ring needs a window
    const int g = num_q_heads / num_kv_heads;
    if (g > kRowsPerWg) return ATTN_ERR_UNSUPPORTED;
    if (out_dtype != ATTN_BF16 && out_dtype != ATTN_FP32) return ATTN_ERR_UNSUPPORTED;
    if ((long long)max_pages_per_seq * kPage > 0x7fffffffLL) return ATTN_ERR_SHAPE;
    if (splitk && (max_kv_len < 1 || keys_per_split < 0 || keys_per_split % kPage ||
                   (long long)max_kv_len > (long long)max_pages_per_seq * kPage))
        return ATTN_ERR_SHAPE;
    if (total_q == 0 || max_q_len == 0) return ATTN_OK;
    if (max_q_len > total_q) return ATTN_ERR_SHAPE;

    PrefillArgs a;
    a.q = (const __bf16*)q;
    a.k_pages = (const char*)k_pages;
    a.v_pages = (const char*)v_pages;
    a.page_table = page_table;
    a.cu_seqlens_q = cu_seqlens_q;
    a.q_start = q_start_pos;
    a.kv_lens = kv_lens;
    a.out = out;
    a.batch = batch;
    a.total_q = total_q;
    a.hq = num_q_heads;
    a.hkv = num_kv_heads;
    a.g = g;
    a.max_pages = max_pages_per_seq;
    a.num_pages = num_pages;
    a.tok_per_wg = kRowsPerWg / g;
    a.wgs_per_seq = (max_q_len + a.tok_per_wg - 1) / a.tok_per_wg;
    a.scale_log2 = softmax_scale * 1.4426950408889634f * (fp8 ? k_scale : 1.f);
    a.v_scale = fp8 ? v_scale : 1.f;
    a.sinks = sinks;
    a.lse = lse;
    a.nsplit = 1;
    a.split_tiles = 0;
    a.part_o = nullptr;
    a.part_ml = nullptr;
    a.window = window;
    a.ring_pages = ring_pages;
    a.k_new = (const char*)k_new;
    a.v_new = (const char*)v_new;
    a.unit_counter = nullptr;
    a.total_units = 0;
    // the new-row buffers are addressed by 32-bit buffer offsets
    if (append && (long long)total_q * num_kv_heads * kRowBytes > 0xffffffffLL)
        return ATTN_ERR_SHAPE;
    const long long base = (long long)a.wgs_per_seq * batch * num_kv_heads;
    if (splitk) {
        const SplitPlanK sp = prefill_split_plan(base, max_kv_len, keys_per_split);
        if (sp.nsplit > 1) {
            const size_t slots = (size_t)sp.nsplit * total_q * num_q_heads;
            if (!workspace || workspace_bytes < slots * (kHeadDim + 2) * sizeof(float))
                return ATTN_ERR_WORKSPACE;
            a.nsplit = sp.nsplit;
            a.split_tiles = sp.split_tiles;
            a.part_o = (float*)workspace;
            a.part_ml = (float*)workspace + slots * kHeadDim;
            const long long grid = base * sp.nsplit;
            const long long mgrid = (long long)total_q * num_q_heads;
            if (grid > 0x7fffffffLL || mgrid > 0x7fffffffLL) return ATTN_ERR_SHAPE;
            if (check_only) return ATTN_OK;
            if (fp8_mma)
                launch_prefill_fp8mma(a, false, true, (unsigned)grid, stream);
            else if (fp8)
                hipLaunchKernelGGL((prefill_hd512_kernel<false, true, true>), dim3((unsigned)grid),
                                   dim3(kThreads), 0, stream, a);
            else
                hipLaunchKernelGGL((prefill_hd512_kernel<false, false, true>), dim3((unsigned)grid),
                                   dim3(kThreads), 0, stream, a);
            const int rows_cap = a.wgs_per_seq * a.tok_per_wg;
            if (out_dtype == ATTN_FP32)
                hipLaunchKernelGGL(prefill_merge_kernel<true>, dim3((unsigned)mgrid), dim3(128), 0,
                                   stream, a, rows_cap);
            else
                hipLaunchKernelGGL(prefill_merge_kernel<false>, dim3((unsigned)mgrid), dim3(128), 0,
                                   stream, a, rows_cap);
            return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
        }
    }
    const long long grid = base;
    if (grid > 0x7fffffffLL) return ATTN_ERR_SHAPE;
    if (check_only && !persist) return ATTN_OK;
    const dim3 gd((unsigned)grid);
    const bool f32 = out_dtype == ATTN_FP32;
    if (persist) {
        if (!workspace) return ATTN_ERR_NULL;
        if (workspace_bytes < kPersistWorkspace) return ATTN_ERR_WORKSPACE;
        // one workgroup per compute unit of the stream's device
        int dev = -1, cus = 0;
        if (stream) {
            hipDevice_t d;
            if (hipStreamGetDevice(stream, &d) != hipSuccess) return ATTN_ERR_HIP;
            dev = (int)d;
        } else if (hipGetDevice(&dev) != hipSuccess) {
            return ATTN_ERR_HIP;
        }
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus < 1)
            return ATTN_ERR_HIP;
        if (check_only) return ATTN_OK;
        a.unit_counter = (int*)workspace;
        a.total_units = (int)grid;
        const dim3 pg((unsigned)(grid < cus ? grid : cus));
        hipLaunchKernelGGL(prefill_counter_reset, dim3(1), dim3(64), 0, stream, a.unit_counter);
        if (fp8 && f32)
            hipLaunchKernelGGL((prefill_hd512_kernel<true, true, false, kHeadDim, false, false, true>),
                               pg, dim3(kThreads), 0, stream, a);
        else if (fp8)
            hipLaunchKernelGGL((prefill_hd512_kernel<false, true, false, kHeadDim, false, false, true>),
                               pg, dim3(kThreads), 0, stream, a);
        else if (f32)
            hipLaunchKernelGGL((prefill_hd512_kernel<true, false, false, kHeadDim, false, false, true>),
                               pg, dim3(kThreads), 0, stream, a);
        else
            hipLaunchKernelGGL((prefill_hd512_kernel<false, false, false, kHeadDim, false, false, true>),
                               pg, dim3(kThreads), 0, stream, a);
        return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
    }
    if (fp8_mma) {
        launch_prefill_fp8mma(a, f32, false, (unsigned)grid, stream);
    } else if (append) {
        if (f32)
            hipLaunchKernelGGL((prefill_hd512_kernel<true, false, false, kHeadDim, false, true>),
                               gd, dim3(kThreads), 0, stream, a);
        else
            hipLaunchKernelGGL((prefill_hd512_kernel<false, false, false, kHeadDim, false, true>),
                               gd, dim3(kThreads), 0, stream, a);
    } else if (fp8)
        launch_single<true, kHeadDim, false>(a, f32, gd, stream);
    else if (head_dim == 256)
        (window > 0 ? launch_single<false, 256, true> : launch_single<false, 256, false>)(a, f32, gd, stream);
    else
        (window > 0 ? launch_single<false, kHeadDim, true> : launch_single<false, kHeadDim, false>)(a, f32, gd, stream);
    return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

}  // namespace
}  // namespace attn

extern "C" int attn_prefill_hd512(const void* q, const void* k_pages, const void* v_pages,
                                  const int32_t* page_table, const int32_t* cu_seqlens_q,
                                  const int32_t* q_start_pos, const int32_t* kv_lens, int batch,
                                  int total_q, int max_q_len, int num_q_heads,
                                  int num_kv_heads, int head_dim, int page_size,
                                  int num_pages, int max_pages_per_seq, float softmax_scale,
                                  void* out, int out_dtype, hipStream_t stream) {
    return attn::prefill_launch(q, k_pages, v_pages, false, 1.f, 1.f, page_table, cu_seqlens_q,
                                q_start_pos, kv_lens, batch, total_q, max_q_len, num_q_heads,
                                num_kv_heads, head_dim, page_size, num_pages, max_pages_per_seq,
                                softmax_scale, nullptr, out, out_dtype, nullptr, false, 0, 0, nullptr,
                                0, false, 0, 0, nullptr, nullptr, false, stream);
}

extern "C" int attn_prefill_hd512_e4m3(const void* q, const void* k_pages, const void* v_pages,
                                       float k_scale, float v_scale, const int32_t* page_table,
                                       const int32_t* cu_seqlens_q, const int32_t* q_start_pos,
                                       const int32_t* kv_lens, int batch, int total_q,
                                       int max_q_len, int num_q_heads, int num_kv_heads,
                                       int head_dim, int page_size, int num_pages,
                                       int max_pages_per_seq, float softmax_scale, void* out,
                                       int out_dtype, hipStream_t stream) {
    return attn::prefill_launch(q, k_pages, v_pages, true, k_scale, v_scale, page_table,
                                cu_seqlens_q, q_start_pos, kv_lens, batch, total_q, max_q_len,
                                num_q_heads, num_kv_heads, head_dim, page_size, num_pages,
                                max_pages_per_seq, softmax_scale, nullptr, out, out_dtype,
                                nullptr, false, 0, 0, nullptr, 0, false, 0, 0, nullptr, nullptr, false, stream);
}

extern "C" int attn_prefill_hd512_ex(const void* q, const void* k_pages, const void* v_pages,
                                     int kv_dtype, float k_scale, float v_scale,
                                     const int32_t* page_table, const int32_t* cu_seqlens_q,
                                     const int32_t* q_start_pos, const int32_t* kv_lens,
                                     int batch, int total_q, int max_q_len, int num_q_heads,
                                     int num_kv_heads, int head_dim, int page_size,
                                     int num_pages, int max_pages_per_seq, float softmax_scale,
                                     const float* sinks, void* out, int out_dtype, float* lse,
                                     hipStream_t stream) {
    using namespace attn;
    if (kv_dtype != ATTN_BF16 && kv_dtype != ATTN_FP8_E4M3) return ATTN_ERR_UNSUPPORTED;
    const bool fp8 = kv_dtype == ATTN_FP8_E4M3;
    return prefill_launch(q, k_pages, v_pages, fp8, fp8 ? k_scale : 1.f, fp8 ? v_scale : 1.f,
                          page_table, cu_seqlens_q, q_start_pos, kv_lens, batch, total_q,
                          max_q_len, num_q_heads, num_kv_heads, head_dim, page_size, num_pages,
                          max_pages_per_seq, softmax_scale, sinks, out, out_dtype, lse, false, 0,
                          0, nullptr, 0, false, 0, 0, nullptr, nullptr, false, stream);
}

extern "C" size_t attn_prefill_hd512_splitk_workspace_size(int batch, int max_q_len,
                                                           int total_q, int num_q_heads,
                                                           int num_kv_heads, int max_kv_len,
                                                           int keys_per_split) {
    using namespace attn;
    if (batch < 1 || max_q_len < 1 || total_q < max_q_len || num_q_heads < 1 ||
        num_kv_heads < 1 || num_q_heads % num_kv_heads || max_kv_len < 1 ||
        keys_per_split < 0 || keys_per_split % kPage)
        return 0;
    const int g = num_q_heads / num_kv_heads;
    if (g > kRowsPerWg) return 0;
    const int tok = kRowsPerWg / g;
    const long long base = (long long)((max_q_len + tok - 1) / tok) * batch * num_kv_heads;
    const SplitPlanK sp = prefill_split_plan(base, max_kv_len, keys_per_split);
    if (sp.nsplit < 2) return 0;
    return (size_t)sp.nsplit * total_q * num_q_heads * (kHeadDim + 2) * sizeof(float);
}

extern "C" int attn_prefill_hd512_splitk(const void* q, const void* k_pages, const void* v_pages,
                                         int kv_dtype, float k_scale, float v_scale,
                                         const int32_t* page_table, const int32_t* cu_seqlens_q,
                                         const int32_t* q_start_pos, const int32_t* kv_lens,
                                         int batch, int total_q, int max_q_len, int num_q_heads,
                                         int num_kv_heads, int head_dim, int page_size,
                                         int num_pages, int max_pages_per_seq, int max_kv_len,
                                         int keys_per_split, float softmax_scale,
                                         const float* sinks, void* workspace,
                                         size_t workspace_bytes, void* out, int out_dtype,
                                         float* lse, hipStream_t stream) {
    using namespace attn;
    if (kv_dtype != ATTN_BF16 && kv_dtype != ATTN_FP8_E4M3) return ATTN_ERR_UNSUPPORTED;
    const bool fp8 = kv_dtype == ATTN_FP8_E4M3;
    return prefill_launch(q, k_pages, v_pages, fp8, fp8 ? k_scale : 1.f, fp8 ? v_scale : 1.f,
                          page_table, cu_seqlens_q, q_start_pos, kv_lens, batch, total_q,
                          max_q_len, num_q_heads, num_kv_heads, head_dim, page_size, num_pages,
                          max_pages_per_seq, softmax_scale, sinks, out, out_dtype, lse, true,
                          max_kv_len, keys_per_split, workspace, workspace_bytes, false, 0, 0, nullptr,
                          nullptr, false, stream);
}

extern "C" int attn_prefill_swa(const void* q, const void* k_pages, const void* v_pages,
                                const int32_t* page_table, const int32_t* cu_seqlens_q,
                                const int32_t* q_start_pos, const int32_t* kv_lens, int batch,
                                int total_q, int max_q_len, int num_q_heads, int num_kv_heads,
                                int head_dim, int page_size, int num_pages,
                                int max_pages_per_seq, int window, int ring_pages,
                                float softmax_scale, void* out, int out_dtype,
                                hipStream_t stream) {
    return attn::prefill_launch(q, k_pages, v_pages, false, 1.f, 1.f, page_table, cu_seqlens_q,
                                q_start_pos, kv_lens, batch, total_q, max_q_len, num_q_heads,
                                num_kv_heads, head_dim, page_size, num_pages, max_pages_per_seq,
                                softmax_scale, nullptr, out, out_dtype, nullptr, false, 0, 0,
                                nullptr, 0, true, window, ring_pages, nullptr, nullptr, false, stream);
}

extern "C" int attn_prefill_hd512_append(const void* q, const void* k_new, const void* v_new,
                                         void* k_pages, void* v_pages,
                                         const int32_t* page_table, const int32_t* cu_seqlens_q,
                                         const int32_t* q_start_pos, const int32_t* kv_lens,
                                         int batch, int total_q, int max_q_len, int num_q_heads,
                                         int num_kv_heads, int head_dim, int page_size,
                                         int num_pages, int max_pages_per_seq,
                                         float softmax_scale, const float* sinks, void* out,
                                         int out_dtype, float* lse, hipStream_t stream) {
    if (!k_new || !v_new) return ATTN_ERR_NULL;
    return attn::prefill_launch(q, k_pages, v_pages, false, 1.f, 1.f, page_table, cu_seqlens_q,
                                q_start_pos, kv_lens, batch, total_q, max_q_len, num_q_heads,
                                num_kv_heads, head_dim, page_size, num_pages, max_pages_per_seq,
                                softmax_scale, sinks, out, out_dtype, lse, false, 0, 0, nullptr,
                                0, false, 0, 0, k_new, v_new, false, stream);
}

extern "C" int attn_prefill_hd512_e4m3_mma_append(
    const void* q, const void* k_new, const void* v_new, void* k_pages, void* v_pages,
    float k_scale, float v_scale, const int32_t* page_table, const int32_t* cu_seqlens_q,
    const int32_t* q_start_pos, const int32_t* kv_lens, int batch, int total_q, int max_q_len,
    int num_q_heads, int num_kv_heads, int head_dim, int page_size, int num_pages,
    int max_pages_per_seq, float softmax_scale, const float* sinks, void* out, int out_dtype,
    float* lse, hipStream_t stream) {
    if (!k_new || !v_new) return ATTN_ERR_NULL;
    // every check of both steps runs before the first launch (the append's
    // are a subset of the prefill's), so a call that fails leaves the pool
    // as it was
    int rc = attn::prefill_launch(q, k_pages, v_pages, true, k_scale, v_scale, page_table,
                                  cu_seqlens_q, q_start_pos, kv_lens, batch, total_q, max_q_len,
                                  num_q_heads, num_kv_heads, head_dim, page_size, num_pages,
                                  max_pages_per_seq, softmax_scale, sinks, out, out_dtype, lse,
                                  false, 0, 0, nullptr, 0, false, 0, 0, nullptr, nullptr, true,
                                  stream, false, true);
    if (rc != ATTN_OK || total_q == 0 || max_q_len == 0) return rc;
    rc = attn_append_kv(k_new, v_new, ATTN_FP8_E4M3, k_scale, v_scale, page_table, cu_seqlens_q,
                        q_start_pos, batch, total_q, num_kv_heads, head_dim, page_size, num_pages,
                        max_pages_per_seq, k_pages, v_pages, stream);
    if (rc != ATTN_OK) return rc;
    return attn::prefill_launch(q, k_pages, v_pages, true, k_scale, v_scale, page_table,
                                cu_seqlens_q, q_start_pos, kv_lens, batch, total_q, max_q_len,
                                num_q_heads, num_kv_heads, head_dim, page_size, num_pages,
                                max_pages_per_seq, softmax_scale, sinks, out, out_dtype, lse,
                                false, 0, 0, nullptr, 0, false, 0, 0, nullptr, nullptr, true,
                                stream);
}

extern "C" size_t attn_prefill_hd512_persistent_workspace_size(void) {
    return attn::kPersistWorkspace;
}

extern "C" int attn_prefill_hd512_persistent(const void* q, const void* k_pages,
                                             const void* v_pages, int kv_dtype, float k_scale,
                                             float v_scale, const int32_t* page_table,
                                             const int32_t* cu_seqlens_q,
                                             const int32_t* q_start_pos, const int32_t* kv_lens,
                                             int batch, int total_q, int max_q_len,
                                             int num_q_heads, int num_kv_heads, int head_dim,
                                             int page_size, int num_pages, int max_pages_per_seq,
                                             float softmax_scale, const float* sinks,
                                             void* workspace, size_t workspace_bytes, void* out,
                                             int out_dtype, float* lse, hipStream_t stream) {
    using namespace attn;
    if (kv_dtype != ATTN_BF16 && kv_dtype != ATTN_FP8_E4M3) return ATTN_ERR_UNSUPPORTED;
    const bool fp8 = kv_dtype == ATTN_FP8_E4M3;
    return prefill_launch(q, k_pages, v_pages, fp8, fp8 ? k_scale : 1.f, fp8 ? v_scale : 1.f,
                          page_table, cu_seqlens_q, q_start_pos, kv_lens, batch, total_q,
                          max_q_len, num_q_heads, num_kv_heads, head_dim, page_size, num_pages,
                          max_pages_per_seq, softmax_scale, sinks, out, out_dtype, lse, false, 0,
                          0, workspace, workspace_bytes, false, 0, 0, nullptr, nullptr, false,
                          stream, true);
}

extern "C" int attn_prefill_hd512_e4m3_mma(const void* q, const void* k_pages,
                                           const void* v_pages, float k_scale, float v_scale,
                                           const int32_t* page_table,
                                           const int32_t* cu_seqlens_q,
                                           const int32_t* q_start_pos, const int32_t* kv_lens,
                                           int batch, int total_q, int max_q_len,
                                           int num_q_heads, int num_kv_heads, int head_dim,
                                           int page_size, int num_pages, int max_pages_per_seq,
                                           float softmax_scale, const float* sinks, void* out,
                                           int out_dtype, float* lse, hipStream_t stream) {
    return attn::prefill_launch(q, k_pages, v_pages, true, k_scale, v_scale, page_table,
                                cu_seqlens_q, q_start_pos, kv_lens, batch, total_q, max_q_len,
                                num_q_heads, num_kv_heads, head_dim, page_size, num_pages,
                                max_pages_per_seq, softmax_scale, sinks, out, out_dtype, lse,
                                false, 0, 0, nullptr, 0, false, 0, 0, nullptr, nullptr, true,
                                stream);
}

extern "C" int attn_prefill_hd512_splitk_e4m3_mma(
    const void* q, const void* k_pages, const void* v_pages, float k_scale, float v_scale,
    const int32_t* page_table, const int32_t* cu_seqlens_q, const int32_t* q_start_pos,
    const int32_t* kv_lens, int batch, int total_q, int max_q_len, int num_q_heads,
    int num_kv_heads, int head_dim, int page_size, int num_pages, int max_pages_per_seq,
    int max_kv_len, int keys_per_split, float softmax_scale, const float* sinks,
    void* workspace, size_t workspace_bytes, void* out, int out_dtype, float* lse,
    hipStream_t stream) {
    return attn::prefill_launch(q, k_pages, v_pages, true, k_scale, v_scale, page_table,
                                cu_seqlens_q, q_start_pos, kv_lens, batch, total_q, max_q_len,
                                num_q_heads, num_kv_heads, head_dim, page_size, num_pages,
                                max_pages_per_seq, softmax_scale, sinks, out, out_dtype, lse, true,
                                max_kv_len, keys_per_split, workspace, workspace_bytes, false, 0,
                                0, nullptr, nullptr, true, stream);
}
