// Chunked causal GQA/MQA prefill at head_dim 512 over a paged FP8-E4M3 KV
// cache with both products on the gfx950 block-scaled FP8 matrix core
// (v_mfma_scale_f32_32x32x64_f8f6f4), the FP8-MMA form of vLLM flash-attention
// PR 199 ("Summary": FP8 paged KV and FP8 QK/PV MMA).
//
// The pages' accuracy safeguards for that form, and what they become here:
//   * Q and P each enter as two E4M3 terms, a high part and a residual (second
//     review, commits 4 and 5 and finding F1: P as e4m3(256 p) plus a residual
//     scaled by 32).  Here every term carries a power-of-two scale in the
//     MFMA itself: the instruction applies one E8M0 exponent per 32
//     contraction elements of each row of A and column of B.  Q is scaled per
//     32 head dims of its row (so no fixed range limit: finding F2 caps |q| at
//     448 with a fixed scale), and P per 32-key block of its row by that
//     block's own maximum, so both terms of every P element lie in
//     [2^-9, 256] relative to 2^(e - 7) and the residual (x 32, as in F1)
//     keeps keys down to about 2^-21 of the block maximum.
//   * FP8 products are accumulated in fp32 by the matrix core (the Hopper
//     path accumulated below fp32 and needed commit 3's per-block promotion
//     and commit 5's split QK sum); O accumulates over the whole key range in
//     the fp32 accumulators, as in the bf16 kernel.
//   * The residual term is issued before the high term (commit 4); with fp32
//     accumulation the order only changes rounding.
// k_scale folds into the softmax scale and v_scale multiplies O at the end, as
// in the widened FP8 path.
//
// Work unit, softmax bookkeeping (a per-row reference maximum, raised by
// whole log2 units only for blocks that would overflow against it), masking
// and output are those of prefill_hd512_kernel.  The tile
// pipeline differs, because one 32x32x64 MFMA of P.V spans the whole 64-key
// tile: per tile j the wave runs Q.K^T of block 0 (16 MFMAs) under block 1's
// softmax of tile j - 1, which completes P(j - 1); then P.V of tile j - 1
// (32 MFMAs); then Q.K^T of block 1 under block 0's softmax of tile j.  Only
// one P operand pair is ever live, which keeps the kernel inside 256 VGPRs
// beside the 256 O accumulators.  E4M3 tiles are 32 KB, so K and V are
// double-buffered (128 KB of LDS) and each refill is issued a phase or more
// ahead of the barrier that waits for it.  A split-K form (one key range per
// workgroup, partials merged by prefill_merge_kernel) shares the code.
#include "device_common.h"
#include "prefill_common.h"

namespace attn {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kRow8 = 512;                  // one E4M3 row of 512 dims
constexpr int kTile8 = kPage * kRow8;       // 32 KB
constexpr int kVRegion = 2 * kTile8;        // V buffers follow the two K buffers
constexpr int kTileArea = 4 * kTile8;       // K0 K1 V0 V1
constexpr int kSmem8 = kTileArea + kPagesInLds * 4;
constexpr int kBufBit = kTile8;             // offset bit that selects buffer 1
static_assert(kBufBit == 1 << 15, "buffers 32 KB apart");
// E8M0 encodings: 2^(e - 7) for a high term, 2^(e - 12) for a residual that
// was scaled by 32
constexpr int kE8Hi = 127 - 7;
constexpr int kE8Lo = 127 - 12;
constexpr int kE8One = 127;

// LDS layout of an E4M3 tile: row r is 512 bytes; its 16-byte chunk c sits at
// chunk c ^ sw8m(r), which permutes only the low 3 chunk bits.  Eight
// consecutive rows at one chunk (the K operand reads) and the 8 rows of a
// transposed V read (keys {0..3, 8..11} + 4 h of 16) both land on 8
// distinct chunk positions, and the chunk bits above 2 stay additive, so the
// k-step and dim-block offsets fold into the instructions' immediates.
__host__ __device__ constexpr int sw8m(int r) { return (r & 7) ^ (((r >> 3) & 1) << 2); }

// Refill of one whole tile: wave w moves rows 16 w .. 16 w + 15, two 512-byte
// rows per buffer->LDS load (lanes 0-31 row 2 J, lanes 32-63 row 2 J + 1).
// The resource covers the tile's valid rows only, so keys past the cache
// length arrive as zeros.
struct TileDma {
    u32x4 rsrc;
    uint32_t lds_base;  // LDS address of this wave's first row
    uint32_t soff;      // byte offset of this wave's first row in the tile
};

__device__ __forceinline__ TileDma tile_dma(const char* pool, int page, int num_pages, int hkv,
                                            int kvh, int valid, uint32_t buf, int wave) {
    page = page < 0 ? 0 : (page >= num_pages ? num_pages - 1 : page);
    const char* src = pool + ((size_t)page * hkv + kvh) * (size_t)kTile8;
    TileDma d;
    d.rsrc = buffer_rsrc(src, (uint32_t)(valid > 0 ? valid : 0) * kRow8);
    d.soff = (uint32_t)__builtin_amdgcn_readfirstlane(wave * 16 * kRow8);
    d.lds_base = (uint32_t)__builtin_amdgcn_readfirstlane((int)(buf + d.soff));
    return d;
}

// Load J of a wave's 8.  Lane l lands at LDS chunk l % 32 of row 2 J + l / 32
// (relative to the wave's rows), so it fetches logical chunk
// (l % 32) ^ sw8m(2 J + l / 32) = (l % 32) ^ (l / 32) ^ c_J: lane_off8 holds
// the lane's part, c_J and the row pair's 1 KB offset are immediates.
template <int J>
__device__ __forceinline__ void tile_rows(const TileDma& d, int lane_off8) {
    constexpr int cJ = ((2 * J) & 6) ^ (J >= 4 ? 4 : 0);
    static_assert(sw8m(2 * J) == cJ && sw8m(2 * J + 1) == (cJ ^ 1), "row-pair swizzle");
    dma_row<(cJ << 4), kRowBytes * J>(d.rsrc, d.lds_base, d.soff, lane_off8);
}

template <int... Js>
__device__ __forceinline__ void tile_rows_all(const TileDma& d, int lane_off8,
                                              std::integer_sequence<int, Js...>) {
    (tile_rows<Js>(d, lane_off8), ...);
}

// acc += a b on the block-scaled FP8 MFMA with a VGPR accumulator (the Q.K^T
// chain, read by the softmax); A unscaled, B scaled by byte SB of sb.  The
// asm is opaque to the hazard recognizer: its operands are written long
// before (Q) or by LDS reads, which the compiler waits for.
template <int SB>
__device__ __forceinline__ void mfma8_vgpr(f32x16& acc, const i32x8& a, const i32x8& b, int sa,
                                           int sb) {
    asm volatile(
        "v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel:[0,%5,0] op_sel_hi:[0,%6,0]"
        : "+v"(acc)
        : "v"(a), "v"(b), "v"(sa), "v"(sb), "i"(SB & 1), "i"(SB >> 1));
}
template <int SB>
__device__ __forceinline__ void mfma8_vgpr_first(f32x16& acc, const i32x8& a, const i32x8& b,
                                                 int sa, int sb) {
    asm volatile(
        "v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, 0, %3, %4 op_sel:[0,%5,0] op_sel_hi:[0,%6,0]"
        : "=&v"(acc)
        : "v"(a), "v"(b), "v"(sa), "v"(sb), "i"(SB & 1), "i"(SB >> 1));
}

// Maximum of x over the lane pair (l, l ^ 32) that holds one query row.
__device__ __forceinline__ float pair_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Two E4M3 terms of values already scaled into [0, 256] (|x| < 256): bytes
// (i, i + 1) of dword dw of hi take e4m3(x), those of lo take e4m3(32 (x -
// hi)), whose magnitude is at most 32 x half an E4M3 step at 256 = 256.
template <bool WORD>
__device__ __forceinline__ void split_pair(float xa, float xb, int& hi, int& lo) {
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(xa, xb, hi, WORD);
    const f32x2 h32 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hi, 32.f, WORD);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_fmaf(xa, 32.f, -h32[0]),
                                         __builtin_fmaf(xb, 32.f, -h32[1]), lo, WORD);
}

// floor of the row's block maximum in log2 units relative to the reference.
// Clamped below at -100 (masked rows and NaN give a finite exponent; weights
// under 2^-100 of the reference vanish either way) and above only where the
// int conversion needs it: a block far above the reference gets its true
// exponent, so its weights p' stay in [0, 256), and rebase_blocks brings the
// exponent back into the E8M0 range before the block's P.V.
__device__ __forceinline__ int block_exponent(const f32x16& s, float scale_log2, float neg_m_ref) {
    float m = s[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) m = fmaxf(m, s[i]);
    m = pair_max(m);
    const float xl = __builtin_fmaf(m, scale_log2, neg_m_ref);
    return (int)__builtin_floorf(fminf(fmaxf(xl, -100.f), 1073741824.f));
}

// Largest block exponent a P.V takes: the block's scale 2^(e - 7) stays
// encodable, and O and l (at most 2^(e + 1) per key and value) far inside fp32.
constexpr int kMaxBlockExp = 32;

// True when a row of the wave has a block of the tile whose P.V is next
// above kMaxBlockExp.
__device__ __forceinline__ bool blocks_over(int e0, int e1) {
    return __builtin_amdgcn_ballot_w64(e0 > kMaxBlockExp || e1 > kMaxBlockExp) != 0;
}

// The reference raise of the online softmax (Flash-Decoding for MQA in CUDA,
// "One KV head breaks the textbook": one rescale per tile, not per key), run
// only when a block would pass kMaxBlockExp: every row of the wave raises
// m_ref by k = max(e0, e1, 0) whole log2 units, multiplies O and l_run by
// 2^-k (exact), and lowers both block exponents by k.  The blocks' weights
// p' are relative to their own exponents, so they do not change.  A block
// left more than 100 log2 units below the new reference takes exponent -100,
// as block_exponent does, which keeps its E8M0 scale encodable (its weights
// are then below 2^-92 of the row's largest, in O and in l alike).
__device__ __forceinline__ void rebase_blocks(f32x16 (&o)[16], float& m_ref, float& l_run,
                                              int& e0, int& e1) {
    const int k = max(max(e0, e1), 0);
    const float f = __builtin_amdgcn_ldexpf(1.f, -k);
    acc_fence(o);
#pragma unroll
    for (int db = 0; db < 16; ++db) scale_acc(o[db], f);
    acc_fence(o);
    l_run *= f;
    m_ref += (float)k;
    e0 = max(e0 - k, -100);
    e1 = max(e1 - k, -100);
}

// Softmax of elements i, i + 1 (i even) of a block with exponent offset c
// (= 7 - e - m_ref), in two halves that go into the two gaps of a k-step's
// dependent MFMA pair (issued after the first MFMA and after the second, so
// that neither gap's VALU work outlasts the MFMA it hides under):
// softmax_exp gives p' = 2^(s scale_log2 + c) in [0, 256); softmax_split
// writes the two E4M3 terms into dword DW of the P operands and adds the
// pair's represented weights hi + lo / 32 (exact in f16: at most 9
// significant bits) to the lane's block sum, so that l sums the same
// weights P.V multiplies: a row with one dominant key gets that key's value
// up to the output rounding.  The empty asms pin the work to its step.
template <int I>
__device__ __forceinline__ void softmax_exp(const f32x16& s, float scale_log2, float c, float& pa,
                                            float& pb) {
    float sa = s[I], sb = s[I + 1];
    asm volatile("" : "+v"(sa), "+v"(sb));
    pa = fast_exp2(__builtin_fmaf(sa, scale_log2, c));
    pb = fast_exp2(__builtin_fmaf(sb, scale_log2, c));
    asm volatile("" : "+v"(pa), "+v"(pb));
}
template <int I, int DW>
__device__ __forceinline__ void softmax_split(float pa, float pb, i32x8& phi, i32x8& plo,
                                              float& psum) {
    constexpr bool kWord = ((I >> 1) & 1) != 0;
    int hi = phi[DW], lo = plo[DW];
    split_pair<kWord>(pa, pb, hi, lo);
    phi[DW] = hi;
    plo[DW] = lo;
    const f16x2 rep = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.f, kWord) +
                      __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 0.03125f, kWord);
    psum = __builtin_amdgcn_fdot2(rep, f16x2{(_Float16)1.f, (_Float16)1.f}, psum, false);
    asm volatile("" : "+v"(hi), "+v"(lo), "+v"(psum));
}
template <int I, int DW>
__device__ __forceinline__ void softmax_pair(const f32x16& s, float scale_log2, float c, float& psum,
                                             i32x8& phi, i32x8& plo) {
    float pa, pb;
    softmax_exp<I>(s, scale_log2, c, pa, pb);
    softmax_split<I, DW>(pa, pb, phi, plo, psum);
}

template <bool OUT_FP32, bool SPLIT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void prefill_fp8mma_kernel(PrefillArgs a) {
    __shared__ __attribute__((aligned(1024))) char smem[kSmem8];
    ATTN_LDS char* const lds = (ATTN_LDS char*)smem;
    ATTN_LDS int* const sPage = (ATTN_LDS int*)(lds + kTileArea);

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    // ---- work unit (as in prefill_hd512_kernel): heaviest query tiles first,
    // KV head fastest; split-K ranges outermost
    const int per_rank = a.batch * a.hkv;
    const int per_split = a.wgs_per_seq * per_rank;
    const int split = SPLIT ? blockIdx.x / per_split : 0;
    const int in_split = blockIdx.x - split * per_split;
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
    const int L_cap = a.max_pages * kPage;
    L = L < 0 ? 0 : (L > L_cap ? L_cap : L);
    const int qs = max(a.q_start[b], 0);
    const int n_max = min(qs + t_last + 1, L);
    const int n_min = min(qs + t0 + 1, L);
    const int ntiles_all = n_max > 0 ? (n_max + kPage - 1) / kPage : 0;
    // this workgroup's key tiles [kt_lo, kt_lo + ntiles): all of them, or one
    // split's range (below, tile j means absolute tile kt_lo + j)
    const int kt_lo = SPLIT ? split * a.split_tiles : 0;
    const int ntiles = SPLIT ? min(ntiles_all, kt_lo + a.split_tiles) - kt_lo : ntiles_all;
    if (SPLIT && ntiles <= 0) return;   // no row of this unit needs the split

    const int n = lane & 31;
    const int h = lane >> 5;
    const int r = wave * 32 + n;
    const int tr = r / a.g;
    const bool valid = (tr < a.tok_per_wg) && (t0 + tr <= t_last);
    const int t = valid ? t0 + tr : t_last;
    const int head = kvh * a.g + (valid ? r - tr * a.g : 0);
    const int n_row = min(qs + t + 1, L);

    // ---- Q^T operands.  k-step ks covers dims 64 ks .. 64 ks + 63; byte s of
    // lane (n, h) is dim 64 ks + 32 (s / 16) + 16 h + s % 16 (the MFMA's k
    // order), and the 32 dims of each half (s / 16) share one exponent eq,
    // whose E8M0 scale the lane of that half's h supplies.
    i32x8 qhi[8], qlo[8];
    int qsc[4] = {0, 0, 0, 0};   // bytes 4 (ks / 2) + 2 (ks % 2) + {0 hi, 1 lo}
    {
        const __bf16* qp = a.q + ((size_t)(q0 + t) * a.hq + head) * kHeadDim;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            float v[32];
#pragma unroll
            for (int part = 0; part < 2; ++part) {
                // padding rows read their shadow row (t, head are in range)
                // and are zeroed after the load
                const bf16x8* src = (const bf16x8*)(qp + 64 * ks + 32 * part + 16 * h);
                bf16x8 x0 = src[0], x1 = src[1];
                if (!valid) x0 = x1 = bf16x8{};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    v[16 * part + e] = (float)x0[e];
                    v[16 * part + 8 + e] = (float)x1[e];
                }
            }
            int eq[2];
#pragma unroll
            for (int part = 0; part < 2; ++part) {
                float m = 0.f;
#pragma unroll
                for (int e = 0; e < 16; ++e) m = fmaxf(m, __builtin_fabsf(v[16 * part + e]));
                m = pair_max(m);
                const int ex = m > 0.f ? __builtin_amdgcn_frexp_expf(m) - 1 : 0;
                eq[part] = ex < -110 ? -110 : (ex > 127 ? 127 : ex);
            }
#pragma unroll
            for (int part = 0; part < 2; ++part) {
#pragma unroll
                for (int dw = 0; dw < 4; ++dw) {
                    const float* x = v + 16 * part + 4 * dw;
                    const int sh = 7 - eq[part];
                    int hi = 0, lo = 0;
                    split_pair<false>(__builtin_amdgcn_ldexpf(x[0], sh),
                                      __builtin_amdgcn_ldexpf(x[1], sh), hi, lo);
                    split_pair<true>(__builtin_amdgcn_ldexpf(x[2], sh),
                                     __builtin_amdgcn_ldexpf(x[3], sh), hi, lo);
                    qhi[ks][4 * part + dw] = hi;
                    qlo[ks][4 * part + dw] = lo;
                }
            }
            const int own = h ? eq[1] : eq[0];
            qsc[ks >> 1] |= ((kE8Hi + own) | ((kE8Lo + own) << 8)) << (16 * (ks & 1));
            __builtin_amdgcn_sched_barrier(0);   // one k-step's loads live at a time
        }
    }

    // ---- LDS operand offsets (buffer 0; bit 15 selects buffer 1)
    // K: k-step ks = 2 k' + k0 of block kb, half j: row 32 kb + n, logical
    // chunk 4 ks + 2 j + h = 8 k' + (4 k0 + 2 j + h)
    int kx[4];
    {
        const int sw = sw8m(n);
#pragma unroll
        for (int k0 = 0; k0 < 2; ++k0)
#pragma unroll
            for (int j = 0; j < 2; ++j) kx[2 * k0 + j] = n * kRow8 + (((4 * k0 + 2 * j + h) ^ sw) << 4);
    }
    // V^T (ds_read_b64_tr_b8, as the widened FP8 path's reader): in 16-lane
    // group G, lane 2 jj + hh addresses key row 16 c + r0, r0 = 8 (jj / 4) +
    // 4 (G / 2) + jj % 4, at the 8-byte half hh of logical chunk 2 db + G % 2;
    // read c (0..3) fills bytes 8 c .. 8 c + 7 of the A operand, i.e. keys
    // 16 c + 8 (jj / 4) + 4 h + jj % 4, the key of P^T byte 8 c + jj.  With
    // db = 4 u + w the offset is vx[w] + 128 u + 8192 c.
    int vx[4];
    {
        const int G = lane >> 4, jj = (lane & 15) >> 1, hh = lane & 1;
        const int r0 = 8 * (jj >> 2) + 4 * (G >> 1) + (jj & 3);
        const int sw = sw8m(r0);
#pragma unroll
        for (int w = 0; w < 4; ++w)
            vx[w] = kVRegion + r0 * kRow8 + (((2 * w + (G & 1)) ^ sw) << 4) + 8 * hh;
    }
    auto kread = [&](int kb, int ks) -> i32x8 {
        const int imm = 16384 * kb + 128 * (ks >> 1);
        const u32x4 x = *(const ATTN_LDS u32x4*)(lds + kx[2 * (ks & 1)] + imm);
        const u32x4 y = *(const ATTN_LDS u32x4*)(lds + kx[2 * (ks & 1) + 1] + imm);
        return i32x8{(int)x[0], (int)x[1], (int)x[2], (int)x[3],
                     (int)y[0], (int)y[1], (int)y[2], (int)y[3]};
    };
    auto vread = [&](int db) -> i32x8 {
        const ATTN_LDS char* p = lds + vx[db & 3] + 128 * (db >> 2);
        const v2i32 x0 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((ATTN_LDS v2i32*)(p));
        const v2i32 x1 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((ATTN_LDS v2i32*)(p + 8192));
        const v2i32 x2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((ATTN_LDS v2i32*)(p + 16384));
        const v2i32 x3 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((ATTN_LDS v2i32*)(p + 24576));
        return i32x8{x0[0], x0[1], x1[0], x1[1], x2[0], x2[1], x3[0], x3[1]};
    };

    const int* ptab = a.page_table + (size_t)b * a.max_pages;
    const int staged = min(ntiles, kPagesInLds);
    for (int i = threadIdx.x; i < staged; i += kThreads) sPage[i] = ptab[kt_lo + i];
    race_delay<2>();
    __syncthreads();
    auto page_of = [&](int tile) -> int {
        return tile < kPagesInLds ? __builtin_amdgcn_readfirstlane(sPage[tile])
                                  : load_uniform(ptab, kt_lo + tile);
    };
    const int lane_off8 = (h << 9) | (((lane & 31) ^ h) << 4);
    const uint32_t lds_u = (uint32_t)(uintptr_t)lds;
    // refill descriptor: tile `tile` (empty past the last one) of K or V into
    // buffer `buf`
    auto tdma = [&](bool is_k, int tile, int buf) -> TileDma {
        const bool in = tile < ntiles;
        const int page = in ? page_of(tile) : 0;
        const int nv = in ? min(L - (kt_lo + tile) * kPage, kPage) : 0;
        return tile_dma(is_k ? a.k_pages : a.v_pages, page, a.num_pages, a.hkv, kvh, nv,
                        lds_u + (is_k ? 0 : kVRegion) + buf * kTile8, wave);
    };
    const int sa = kE8One;

    f32x16 o[16];
    f32x16 s0, s1;                 // scores of blocks 0 and 1 (raw, then masked)
    i32x8 phi = {}, plo = {};      // P operands: bytes 0-15 block 0, 16-31 block 1
    float m_ref = -__builtin_inff();
    float l_run = 0.f;

    // Per tile j the wave runs, in order: Q.K^T of block 0 of tile j under
    // block 1's softmax of tile j - 1 (which completes P(j - 1)); P.V of tile
    // j - 1; Q.K^T of block 1 of tile j under block 0's softmax of tile j.
    // So the P operands are built just before their P.V and only one copy
    // is ever live.
    //
    // Vector-memory accounting per wave: refills are issued in the order
    // K(0), V(-1) (empty) before the loop, then K(j + 1) under Q.K^T of block
    // 0 of tile j and V(j) under that of block 1, 8 loads each.  Tile j's
    // first phase needs K(j) and its P.V phase V(j - 1): each was issued one
    // refill (8 loads) before the newest.  Refills past the last tile are
    // issued too (empty: they land zeros in buffers nothing reads again), so
    // that every count is the same; the last P.V waits for all.
    // Q.K^T of block kb of the tile in the current K buffer into acc, one
    // refill row pair after each k-step's first MFMA and softmax pair i of
    // block sp (of the other block) over both of its MFMAs.  `prologue`
    // (the other block's masking and exponent; it returns the softmax offset
    // c) runs after the first MFMA is issued, so that it overlaps the matrix
    // pipe instead of delaying the chain.
    auto qk_phase = [&](auto KB, f32x16& acc, const TileDma& d, const f32x16& sp, auto prologue,
                        float& psum, auto DWB) {
        constexpr int kb = decltype(KB)::value;
        constexpr int dwb = decltype(DWB)::value;
        float c = 0.f;
        // one k-step's operand read ahead: two 64-cycle MFMAs cover its latency
        i32x8 knext = kread(kb, 0);
        static_for<8>([&](auto KS) {
            constexpr int ks = decltype(KS)::value;
            const i32x8 cur = knext;
            if constexpr (ks + 1 < 8) knext = kread(kb, ks + 1);
            if constexpr (ks == 0)
                mfma8_vgpr_first<2 * (ks & 1) + 1>(acc, cur, qlo[ks], sa, qsc[ks >> 1]);
            else
                mfma8_vgpr<2 * (ks & 1) + 1>(acc, cur, qlo[ks], sa, qsc[ks >> 1]);
            tile_rows<ks>(d, lane_off8);
            if constexpr (ks == 0) c = prologue();
            float pa, pb;
            softmax_exp<2 * ks>(sp, a.scale_log2, c, pa, pb);
            __builtin_amdgcn_sched_barrier(0);
            mfma8_vgpr<2 * (ks & 1)>(acc, cur, qhi[ks], sa, qsc[ks >> 1]);
            softmax_split<2 * ks, dwb + ks / 2>(pa, pb, phi, plo, psum);
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    // P.V of the tile whose P operands are complete, from V buffer vbuf
    auto pv_phase = [&](int vbuf, int psc) {
        const int vflip = vbuf * kBufBit;
#pragma unroll
        for (int w = 0; w < 4; ++w) vx[w] ^= vflip;
        // two operand buffers; each is refilled (two dim blocks ahead) right
        // after its last MFMA, so a read has two steps (four MFMAs) to land
        i32x8 vb0 = vread(0), vb1 = vread(1);
        static_for<16>([&](auto DB) {
            constexpr int db = decltype(DB)::value;
            const i32x8 vop = (db & 1) ? vb1 : vb0;
            o[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vop, plo, o[db], 0, 0, 0, sa,
                                                                    1, psc);
            o[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vop, phi, o[db], 0, 0, 0, sa,
                                                                    0, psc);
            // keeps each step's MFMAs and operand read in their step (without
            // it the compiler may hoist all 16 reads above MFMAs sunk to the
            // epilogue and run out of registers)
            asm volatile("" : "+a"(o[db]) :: "memory");
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (db + 2 < 16) {
                if constexpr (db & 1) vb1 = vread(db + 2); else vb0 = vread(db + 2);
            }
            __builtin_amdgcn_sched_barrier(0);
        });
#pragma unroll
        for (int w = 0; w < 4; ++w) vx[w] ^= vflip;
    };

    // Per tile j the wave runs, in order: Q.K^T of block 0 of tile j under
    // block 1's softmax of tile j - 1 (which completes P(j - 1)); P.V of tile
    // j - 1; Q.K^T of block 1 of tile j under block 0's softmax of tile j.
    // So the P operands are built just before their P.V and only one copy
    // is ever live.  The last tile's block-1 softmax and P.V follow the loop.
    //
    // Vector-memory accounting per wave: refills are issued in the order
    // K(0), V(-1) (empty) before the loop, then K(j + 1) under Q.K^T of block
    // 0 of tile j and V(j) under that of block 1, 8 loads each.  Tile j's
    // first phase needs K(j) and its P.V phase V(j - 1): each was issued one
    // refill (8 loads) before the newest.  Refills past the last tile are
    // issued too (empty: they land zeros in buffers nothing reads again), so
    // that every count is the same; the last P.V waits for all.
    if (ntiles > 0) {
#pragma unroll
        for (int db = 0; db < 16; ++db) o[db] = f32x16{};
        tile_rows_all(tdma(true, 0, 0), lane_off8, std::make_integer_sequence<int, 8>{});
        tile_rows_all(tdma(false, ntiles, 1), lane_off8, std::make_integer_sequence<int, 8>{});
        s1 = f32x16{};   // tile 0's first phase runs a softmax whose results are unused
        int e0 = 0;      // block 0's exponent of the tile being built
        float ps0 = 0.f; // its lane sum of p'
        for (int j = 0; j < ntiles; ++j) {
            const int key0 = (kt_lo + j) * kPage;
            // ---- block 1's softmax of tile j - 1 (completing P(j - 1)) under
            // Q.K^T of block 0 of tile j; K(j + 1) refill
            const float neg_m = -m_ref;
            const TileDma dk = tdma(true, j + 1, (j + 1) & 1);
            wait_vmcnt<8>();
            lds_barrier();
            int e1 = 0;
            float ps1 = 0.f;   // block sums of the represented weights, in units of p'
            qk_phase(std::integral_constant<int, 0>{}, s0, dk, s1, [&]() {
                mfma_vgpr_drain(s1);
                if (j > 0 && key0 > n_min)
                    mask_block<false>(s1, key0 - kPage + 32 + 4 * h, n_row, 0);
                e1 = block_exponent(s1, a.scale_log2, neg_m);
                return neg_m + (float)(7 - e1);
            }, ps1, std::integral_constant<int, 4>{});
            // ---- P.V of tile j - 1
            if (j > 0) {
                // the vote is taken before the wait and acted on after it
                const bool over = blocks_over(e0, e1);
                wait_vmcnt<8>();
                lds_barrier();
                if (__builtin_expect(over, 0)) rebase_blocks(o, m_ref, l_run, e0, e1);
                const int own = h ? e1 : e0;
                l_run += __builtin_amdgcn_ldexpf(ps0, e0 - 7) + __builtin_amdgcn_ldexpf(ps1, e1 - 7);
                pv_phase((j - 1) & 1, (kE8Hi + own) | ((kE8Lo + own) << 8));
            }
            // ---- block 0's softmax of tile j under Q.K^T of block 1; V(j) refill
            ps0 = 0.f;
            qk_phase(std::integral_constant<int, 1>{}, s1, tdma(false, j, j & 1), s0, [&]() {
                mfma_vgpr_drain(s0);
                if (key0 + kPage > n_min) mask_block<false>(s0, key0 + 4 * h, n_row, 0);
                float neg_m0 = -m_ref;   // after any raise above
                if (j == 0) {
                    // reference maximum: the row's maximum over the range's first
                    // 32 keys (without split-K key 0 is visible to every row; a
                    // split can start past a row's causal limit, and that row
                    // then takes 0: every p = 0, an empty partial)
                    float m0 = s0[0];
#pragma unroll
                    for (int i = 1; i < 16; ++i) m0 = fmaxf(m0, s0[i]);
                    m0 = pair_max(m0) * a.scale_log2;
                    m0 = m0 == -__builtin_inff() ? 0.f : m0;
                    m_ref = m0;
                    neg_m0 = -m0;
                }
                e0 = block_exponent(s0, a.scale_log2, neg_m0);
                return neg_m0 + (float)(7 - e0);
            }, ps0, std::integral_constant<int, 0>{});
            // the next tile reads the other K buffer
#pragma unroll
            for (int i = 0; i < 4; ++i) kx[i] ^= kBufBit;
        }
        // ---- the last tile: block 1's softmax and P.V
        {
            mfma_vgpr_drain(s1);
            const int key0 = (kt_lo + ntiles) * kPage;
            if (key0 > n_min) mask_block<false>(s1, key0 - kPage + 32 + 4 * h, n_row, 0);
            const float neg_m = -m_ref;
            int e1 = block_exponent(s1, a.scale_log2, neg_m);
            const float c1 = neg_m + (float)(7 - e1);
            float ps1 = 0.f;
            static_for<8>([&](auto I) {
                constexpr int i = 2 * decltype(I)::value;
                softmax_pair<i, 4 + i / 4>(s1, a.scale_log2, c1, ps1, phi, plo);
            });
            const bool over = blocks_over(e0, e1);
            wait_vmcnt<0>();
            lds_barrier();
            if (__builtin_expect(over, 0)) rebase_blocks(o, m_ref, l_run, e0, e1);
            const int own = h ? e1 : e0;
            l_run += __builtin_amdgcn_ldexpf(ps0, e0 - 7) + __builtin_amdgcn_ldexpf(ps1, e1 - 7);
            pv_phase((ntiles - 1) & 1, (kE8Hi + own) | ((kE8Lo + own) << 8));
        }
    }

    // ---- epilogue (shared with prefill_hd512_kernel): O in the true scale of p.
    // The row's token and head are derived again from the lane index, which
    // is itself recounted here (mbcnt) rather than read from the thread
    // index: kept from the prologue, either would stay live across the key
    // loop, where every register is taken, and spill.
    static_assert(kWaves * 32 * kHeadDim * 2 <= kTileArea, "staging fits the tile buffers");
    const int lane_e = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    const int r_e = wave * 32 + (lane_e & 31);
    const int tr_e = r_e / a.g;
    const bool valid_e = (tr_e < a.tok_per_wg) && (t0 + tr_e <= t_last);
    const int t_e = valid_e ? t0 + tr_e : t_last;
    const int head_e = kvh * a.g + (valid_e ? r_e - tr_e * a.g : 0);
    prefill_epilogue<OUT_FP32, SPLIT, kHeadDim, !OUT_FP32, true>(
        a, o, l_run, m_ref, ntiles > 0,
        RowSlot{q0, q0 + t_e, head_e, t0, t_last, kvh, split, valid_e}, lds, lane_e, wave);
}

}  // namespace

void launch_prefill_fp8mma(const PrefillArgs& a, bool out_fp32, bool split, unsigned grid,
                           hipStream_t stream) {
    if (split)
        hipLaunchKernelGGL((prefill_fp8mma_kernel<false, true>), dim3(grid), dim3(kThreads), 0,
                           stream, a);
    else if (out_fp32)
        hipLaunchKernelGGL((prefill_fp8mma_kernel<true, false>), dim3(grid), dim3(kThreads), 0,
                           stream, a);
    else
        hipLaunchKernelGGL((prefill_fp8mma_kernel<false, false>), dim3(grid), dim3(kThreads), 0,
                           stream, a);
}

}  // namespace attn
