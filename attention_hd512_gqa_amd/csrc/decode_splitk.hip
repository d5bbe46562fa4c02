// Split-K (Flash-Decoding) decode at head_dim 512 over a paged KV cache, for
// gfx950 (MI355X): q_len query tokens per sequence at its last positions
// (1 for plain decode; more for verifying drafted tokens), GQA/MQA.
//
// A single KV head per sequence would give one workgroup per (sequence, KV
// head) and leave most CUs idle, so the key range is cut into splits of
// `keys_per_split` keys, each handled by one workgroup that writes
// unnormalised partials (O, m, l) for the (token, query head) columns of the
// group; a merge kernel then combines the partials with the online-softmax
// rule (Flash-Decoding for MQA in CUDA, "One KV head breaks the textbook").
// Only the live band [0, kv_len) is read (same page, "The starting point").
// Every KV byte is read once per call, with the non-temporal cache policy.
//
// The q_len * g columns of a KV head are the (zero-padded) 16-column blocks
// of v_mfma_f32_16x16x32_bf16 products: S^T = K Q^T and O^T += V^T P^T, O in
// fp32 per key block (vLLM flash-attention PR 199, commit 3 of the first
// review).  Decode moves ~2 bytes per flop per column block: HBM bandwidth,
// not the MFMA rate, bounds it, and the padded MFMA columns cost issue slots
// that are free at that ratio.
//
// Tile kernel (bf16 pool; FP8 pool with 2 or 3 column blocks): one 64-key tile
// (= one page of one KV head) at a time per workgroup of 4 waves.  K and V
// tiles are DMA'd to separate LDS buffers (swizzled rows); wave w computes
// the scores and probabilities of keys 16 w .. 16 w + 15 for every column
// block, the probabilities meet in a small LDS buffer, and every wave
// accumulates its own 128 of the 512 output dims over all 64 keys.  Up to 3
// blocks (48 columns: e.g. 5 tokens at g = 8) keep Q in registers; wider
// calls run as split-K prefill.
//
// Half-page kernel (FP8-E4M3 pool, one column block): a split workgroup is
// one wave (the kernel takes any number of waves, each on its own 32-key
// half pages and writing its own partial), so the loop has no workgroup
// barrier and four independent waves per CU hide each other's start-up.
// Each wave DMAs raw E4M3 half pages of K and V into its own two LDS buffers
// and reads K back row-wise, V transposed (ds_read_b64_tr_b8).
//
// FP8 values are widened exactly to bf16 (every E4M3 value is a bf16 value)
// just before their MFMA, k_scale is folded into the softmax scale and
// v_scale into the partial (vLLM flash-attention PR 199, "Summary": FP8 KV
// with 16-bit MMA).  Both kernels keep a reference maximum per column and
// rescale O only when a score exceeds it by more than a margin (log2 units),
// so the O accumulators are rarely touched by the softmax.
#include "device_common.h"
#include "attn_host.h"

#include <mutex>

namespace attn {

namespace {

constexpr int kDecRows = 16;        // query heads of one group, zero-padded
constexpr int kDecWaves = 4;
constexpr int kDecThreads = 64 * kDecWaves;
constexpr int kDefaultTargetWgs = 4096;
constexpr int kFp8Waves = 1;       // waves per FP8 split workgroup, one partial each
constexpr int kMaxSub = 4;          // partials per split workgroup (FP8: one per wave)
constexpr int kHalfKeys = 32;       // FP8: keys per wave step
constexpr int kHalfBytes = kHalfKeys * kHeadDim;   // FP8 rows are 512 bytes
constexpr float kRefMargin = 10.f;  // FP8: allowed excess of a score over the reference max
constexpr int kRoutedMaxGroup = 128;  // largest group the prefill takes (128 packed rows)
constexpr int kMaxColBlocks = 3;    // 16-column blocks of a decode split (Q stays in registers)
constexpr int kDecCols = kDecRows * kMaxColBlocks;   // wider calls run as split-K prefill

struct DecodeArgs {
    const __bf16* q;
    const char* k_pages;
    const char* v_pages;
    const int* page_table;
    const int* kv_lens;
    float* part_o;      // [batch][hkv][max_splits][sub][g][512]
    float* part_ml;     // [batch][hkv][max_splits][sub][g][2]  (m in log2 units, l)
    int batch, hq, hkv, g, max_pages, num_pages;
    int q_len;          // query tokens per sequence, at positions kv_len - q_len ..
    int cols;           // q_len * g MFMA columns: column c = token c / g, head c % g
    int max_splits, tiles_per_split, sub;
    float scale_log2;   // softmax_scale * log2(e) * k_scale
    float v_scale;
    const float* sinks; // per query head sink logit (natural-log units), or null
    float* lse;         // [batch * q_len][hq] natural-log log-sum-exp, or null
};

// The key range of one split workgroup and where its tiles live.
struct SplitPlan {
    int b, kvh, split;
    int k_begin, k_end, ntiles;
    int L;              // the sequence's cache length
    const int* ptab;    // this sequence's row of the page table
};

// Split-major launch order: consecutive workgroups take the same split index
// of different (sequence, KV head) pairs.  Workgroups are dealt round-robin
// to the 8 XCDs, so each XCD gets the same mix of split indices (a split
// index fixed per XCD would give some XCDs mostly empty late splits), and the
// late, often empty splits come last.
__device__ __forceinline__ bool plan_split(const DecodeArgs& a, SplitPlan& p) {
    const int pairs = a.batch * a.hkv;
    p.split = blockIdx.x / pairs;
    const int rest = blockIdx.x - p.split * pairs;
    p.kvh = rest % a.hkv;
    p.b = rest / a.hkv;
    int L = __builtin_amdgcn_readfirstlane(a.kv_lens[p.b]);   // wave-uniform
    L = L < 0 ? 0 : (L > a.max_pages * kPage ? a.max_pages * kPage : L);
    p.k_begin = p.split * a.tiles_per_split * kPage;
    if (p.k_begin >= L) return false;  // empty split: the merge never reads it
    p.k_end = min(p.k_begin + a.tiles_per_split * kPage, L);
    p.ntiles = (p.k_end - p.k_begin + kPage - 1) / kPage;
    p.L = L;
    p.ptab = a.page_table + (size_t)p.b * a.max_pages;
    return true;
}

// Physical page of split tile t (clamped to the split's tiles, then to the
// pool).
__device__ __forceinline__ int split_page(const DecodeArgs& a, const SplitPlan& p, int t) {
    const int tile = p.k_begin / kPage + min(max(t, 0), p.ntiles - 1);
    const int page = load_uniform(p.ptab, tile);
    return page < 0 ? 0 : (page >= a.num_pages ? a.num_pages - 1 : page);
}
__device__ __forceinline__ const char* tile_base(const char* pool, const DecodeArgs& a, int page,
                                                 int kvh, int tile_bytes) {
    return pool + ((size_t)page * a.hkv + kvh) * (size_t)tile_bytes;
}

// MFMA column c of a split: token c / g at position L - q_len + c / g and
// query head kvh g + c % g.  Columns past q_len g are zero padding.
struct Column {
    bool ok;            // a real (token, head)
    size_t q_row;       // row of q / out: (b q_len + token) hq + head
    int k_lim;          // keys of the split this column may see: [k_begin, k_lim)
};

__device__ __forceinline__ Column column_of(const DecodeArgs& a, const SplitPlan& p, int c) {
    Column col;
    col.ok = c < a.cols;
    const int t = col.ok ? c / a.g : 0;
    const int h = col.ok ? c - t * a.g : 0;
    col.q_row = ((size_t)p.b * a.q_len + t) * a.hq + (size_t)p.kvh * a.g + h;
    // causal: the token at position L - q_len + t sees keys j <= that position
    col.k_lim = col.ok ? min(p.k_end, p.L - a.q_len + t + 1) : p.k_end;
    return col;
}

// exp2 reference that is finite whenever possible: a column that has seen
// no key yet keeps m = -inf, and its p = 2^(-inf - 0) = 0, alpha = 1.
__device__ __forceinline__ float finite_or_zero(float m) { return m == -__builtin_inff() ? 0.f : m; }

// Unnormalised partial of column c: O^T element i of block db is dim
// 16 db + 4 kq + i (db over NB blocks, starting at dim d0); l sums over the
// four k-groups.
template <int NB>
__device__ __forceinline__ void write_partial(const DecodeArgs& a, size_t slot, int c, int kq,
                                              int d0, const f32x4 (&o)[NB], float m, float l) {
    float l_row = l + __shfl_xor(l, 16);
    l_row += __shfl_xor(l_row, 32);
    if (c < a.cols) {
        float* dst = a.part_o + slot * kHeadDim + d0 + 4 * kq;
#pragma unroll
        for (int db = 0; db < NB; ++db) *(f32x4*)(dst + 16 * db) = o[db] * a.v_scale;
        if (kq == 0 && d0 == 0) {
            a.part_ml[2 * slot] = m;
            a.part_ml[2 * slot + 1] = l_row;
        }
    }
}

// ====================== tile kernel (bf16 and wide FP8) ======================

// LDS layout of E4M3 rows: row r (a key) is 512 bytes, its 16-byte chunk c
// sits at chunk c ^ swz8(r).  swz8 is a bijection on r mod 16, so the 16 rows
// of one K operand read land on 16 distinct chunk positions (all 64 banks),
// and so do the rows of each transposed V read (8 consecutive rows from a
// multiple of 8; in the half-page kernel rows 4 kq .. 4 kq + 3 and 16 + 4 kq
// .. 16 + 4 kq + 3).
__host__ __device__ constexpr int swz8(int r) { return (r & 15) ^ (((r >> 4) & 1) << 2); }

// Eight E4M3 bytes (two words, low byte first) widened exactly to bf16.
__device__ __forceinline__ bf16x8 widen8(uint32_t w0, uint32_t w1) {
    const bf16x2 a0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
    const bf16x2 a1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
    const bf16x2 a2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
    const bf16x2 a3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
    return bf16x8{a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]};
}

// x *= f for an f32x4 accumulator held in AGPRs, one element at a time
// through one VGPR (VALU cannot read AGPRs), as asm so that the accumulators
// stay in AGPRs (with Q's registers beside them, VGPRs would not hold them).
__device__ __forceinline__ void scale_acc4(f32x4& acc, float f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float x = acc[i];
        float t;
        asm volatile(
            "v_accvgpr_read_b32 %1, %0\n\t"
            "v_mul_f32 %1, %1, %2\n\t"
            "v_accvgpr_write_b32 %0, %1"
            : "+a"(x), "=&v"(t)
            : "v"(f));
        acc[i] = x;
    }
}

// Wait states around scale_acc4, tied to the 8 accumulators of one column
// block so that no MFMA moves across them: an MFMA's result is written before
// v_accvgpr_read reads it, and a v_accvgpr_write before an MFMA reads the
// register as its C operand (the asm is opaque to the hazard recognizer).
__device__ __forceinline__ void acc_fence8(f32x4 (&o)[8]) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]), "+a"(o[4]), "+a"(o[5]),
                   "+a"(o[6]), "+a"(o[7]));
}

// Load I of an E4M3 row-pair refill: rows 2 I and 2 I + 1 of a block (lanes
// 0-31 and 32-63), 16 bytes per lane, landing at LDS bytes 1024 I + 16 lane
// past `lds` and fetched from block byte 1024 I + 512 (lane / 32) + 16 c,
// c = (lane % 32) ^ swz8(row).  For rows 2 I + h (h = lane / 32) of a block
// that starts at a multiple of 32 rows, swz8 is h OR (2 (I % 8) ^ 4 (I / 8)),
// so the whole per-lane offset is lane_base XOR a constant; a block starting
// at 16 mod 32 (the tile kernel's odd waves) takes bit 2 of swz8 into
// lane_base.  M0 is written for every fourth load: the instruction's offset
// field, which the hardware adds to both the source and the LDS address,
// carries (I % 4) KB; it also enters the resource's range check, so rows past
// the record count still arrive as zeros.  The SALU write of M0 and the load
// that reads it are one VALU op apart.
template <int I>
__device__ __forceinline__ void dma_row_pair(u32x4 rsrc, uint32_t lds, int lane_base) {
    constexpr int kC = (((2 * (I % 8)) ^ (4 * (I / 8))) << 4) | ((I / 4) * 4096);
    int voff;
    if constexpr (I % 4 == 0) {
        asm volatile(
            "s_add_u32 m0, %3, %2\n\t"
            "v_xor_b32 %0, %4, %1\n\t"
            "buffer_load_dwordx4 %0, %5, 0 offen nt lds"
            : "=&v"(voff)
            : "v"(lane_base), "i"((I / 4) * 4096), "s"(lds), "i"(kC), "s"(rsrc)
            : "memory", "m0", "scc");
    } else {
        asm volatile(
            "v_xor_b32 %0, %2, %1\n\t"
            "buffer_load_dwordx4 %0, %3, 0 offen offset:%4 nt lds"
            : "=&v"(voff)
            : "v"(lane_base), "i"(kC), "s"(rsrc), "i"((I % 4) * 2 * kHeadDim)
            : "memory");
    }
}

// This wave's 16 rows (16 wave .. 16 wave + 15) of a 64-key tile -> LDS, rows
// past `valid` as zeros.  bf16: 1 KB rows, one per DMA, swizzled by swz.
// E4M3: 512-byte rows, two per DMA, 16-byte chunk c of row r stored at chunk
// c ^ swz8(r) (the FP8 half pages' layout below).
template <bool FP8>
__device__ __forceinline__ void issue_tile(const char* src, int valid, ATTN_LDS char* buf,
                                           int wave, int lane) {
    if constexpr (!FP8) {
        rows16_to_lds<true>(buffer_rsrc(src, (uint32_t)valid * kRowBytes), buf, wave, lane * 16);
    } else {
        // rows 16 wave + 2 i + h: the wave's block starts 16 wave rows in
        const u32x4 rsrc = buffer_rsrc(src, (uint32_t)valid * kHeadDim);
        const uint32_t lds = (uint32_t)__builtin_amdgcn_readfirstlane(
            (int)((uint32_t)(uintptr_t)buf + (uint32_t)wave * 16 * kHeadDim));
        const int hl = lane >> 5;
        const int lane_base = (wave * 16 * kHeadDim) | (hl << 9) |
                              ((((lane & 31) ^ hl) ^ (4 * (wave & 1))) << 4);
        static_for<8>([&](auto I) { dma_row_pair<decltype(I)::value>(rsrc, lds, lane_base); });
        race_delay<0>();
    }
}

// S^T += K Q^T on v_mfma_f32_16x16x32_bf16 with the score accumulator in
// VGPRs and the Q operand in AGPRs (QA) or VGPRs.  With two or three column
// blocks Q takes 64 registers per block; holding blocks 1.. in AGPRs, read
// by the MFMA directly, leaves the VGPRs for operand reads in flight.  The
// asm is opaque to the hazard recognizer, so: FIRST starts the chain from an
// inline zero accumulator (no VALU write feeds it), NOP puts 5 wait states
// in front for a K operand a VALU op (the E4M3 widening) has just written,
// and qk_drain waits out the MFMAs' passes before the scores are read.
#define ATTN_QK_MFMA(PRE, C) PRE "v_mfma_f32_16x16x32_bf16 %0, %1, %2, " C
template <bool QA, bool FIRST, bool NOP>
__device__ __forceinline__ void qk_mfma(f32x4& acc, const bf16x8& k, const bf16x8& q) {
    // the wait states sit in the same asm as the MFMA, so that nothing is
    // scheduled between them
    if constexpr (FIRST && NOP && QA)
        asm volatile(ATTN_QK_MFMA("s_nop 4\n\t", "0") : "=&v"(acc) : "v"(k), "a"(q));
    else if constexpr (FIRST && NOP)
        asm volatile(ATTN_QK_MFMA("s_nop 4\n\t", "0") : "=&v"(acc) : "v"(k), "v"(q));
    else if constexpr (FIRST && QA)
        asm volatile(ATTN_QK_MFMA("", "0") : "=&v"(acc) : "v"(k), "a"(q));
    else if constexpr (FIRST)
        asm volatile(ATTN_QK_MFMA("", "0") : "=&v"(acc) : "v"(k), "v"(q));
    else if constexpr (NOP && QA)
        asm volatile(ATTN_QK_MFMA("s_nop 4\n\t", "%0") : "+v"(acc) : "v"(k), "a"(q));
    else if constexpr (NOP)
        asm volatile(ATTN_QK_MFMA("s_nop 4\n\t", "%0") : "+v"(acc) : "v"(k), "v"(q));
    else if constexpr (QA)
        asm volatile(ATTN_QK_MFMA("", "%0") : "+v"(acc) : "v"(k), "a"(q));
    else
        asm volatile(ATTN_QK_MFMA("", "%0") : "+v"(acc) : "v"(k), "v"(q));
}
#undef ATTN_QK_MFMA
template <int NC>
__device__ __forceinline__ void qk_drain(f32x4 (&s)[NC]) {
    if constexpr (NC == 2)
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s[0]), "+v"(s[1]));
    else
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s[0]), "+v"(s[1]), "+v"(s[2]));
}

// One 64-key tile (= one page of one KV head) at a time per workgroup of 4
// waves, NC blocks of 16 (token, head) columns.  Wave w DMAs keys 16 w ..
// 16 w + 15 of each K and V tile into LDS; it alone reads those K rows, so
// it refills them as soon as its own reads have returned.  It computes its
// keys' scores for every column block (one K operand read serves all NC
// blocks) and their probabilities, which it writes to LDS as bf16; after a
// barrier it accumulates its own 128 of the 512 output dims over all 64
// keys, reading each V operand once for all blocks.  A column's
// probabilities are taken against a reference maximum that moves only when
// a tile's maximum exceeds it by more than kTileMargin (log2 units), so the
// accumulators are rarely rescaled; l sums the bf16 probabilities the PV
// products use.  The probabilities are written against the current
// references at once, with each wave's vote on whether one of its scores
// passes the margin; only when a vote is cast (every column's first tile,
// then rarely) do the waves exchange per-column maxima, move references,
// rescale and write the probabilities again, two barriers more.  bf16: a
// second barrier per tile frees the V buffer for the next tile.  FP8: the
// tiles hold E4M3 bytes, widened exactly to bf16 as each operand is read
// (k_scale is in the softmax scale, v_scale in the partial); their 32 KB
// tiles fit twice over, so K(t + 2) loads while tile t is consumed, and V(t +
// 1) goes out after tile t's barrier (every wave is then past P.V of tile
// t - 1, whose buffer it takes): one barrier per tile.
constexpr float kTileMargin = 8.f;
constexpr int kPStride = 2 * kPage + 16;   // bytes per column row of the P buffer

__device__ __forceinline__ float pair_sum(const bf16x8& v, float acc) {
    const bf16x2 one = {(__bf16)1.f, (__bf16)1.f};
#pragma unroll
    for (int j = 0; j < 4; ++j)
        acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{v[2 * j], v[2 * j + 1]}, one, acc, false);
    return acc;
}

template <bool FP8, int NC>
__global__ __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_split_tile_kernel(DecodeArgs a) {
    constexpr int kTB = FP8 ? kPage * kHeadDim : kTileBytes;   // one K or V tile
    constexpr int kLoads = FP8 ? kPage / 8 : kPage / kDecWaves;  // DMAs per wave per tile
    constexpr int kCols = NC * kDecRows;
    constexpr int kDepth = FP8 ? 2 : 1;   // tiles in flight per operand
    constexpr int kPBytes = kCols * kPStride;   // one P buffer
    __shared__ __attribute__((aligned(1024)))
        char smem[2 * kDepth * kTB + 2 * kPBytes + kCols * kDecWaves * 4 + 2 * kDecWaves * 4];
    SplitPlan p;
    if (!plan_split(a, p)) return;
    ATTN_LDS char* sK0 = (ATTN_LDS char*)smem;                  // K buffers, then V buffers
    ATTN_LDS char* sV0 = sK0 + kDepth * kTB;
    ATTN_LDS char* sP0 = sV0 + kDepth * kTB;                     // 2 x [column][64 keys] bf16
    ATTN_LDS float* sM = (ATTN_LDS float*)(sP0 + 2 * kPBytes);   // [column][wave]
    ATTN_LDS int* sVote = (ATTN_LDS int*)(sM + kCols * kDecWaves);  // 2 x [wave]
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15;   // MFMA column within a block
    const int kq = lane >> 4;  // k-group

    // Q^T operand of block cb, k-step ks: bf16 dims 32 ks + 8 kq .. + 7; FP8
    // dims 64 (ks / 2) + 16 kq + 8 (ks % 2) .. + 7, the order in which one
    // 16-byte K read delivers two k-steps
    Column col[NC];
    bf16x8 qf[NC][16];
#pragma unroll
    for (int cb = 0; cb < NC; ++cb) {
        col[cb] = column_of(a, p, 16 * cb + n);
        const __bf16* qrow = a.q + col[cb].q_row * kHeadDim;
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) {
            const int d = FP8 ? 64 * (ks >> 1) + 16 * kq + 8 * (ks & 1) : 32 * ks + 8 * kq;
            const bf16x8 v = *(const bf16x8*)(qrow + d);
            qf[cb][ks] = col[cb].ok ? v : bf16x8{};
        }
    }
    // K operand: key row 16 wave + n (the tile layouts of issue_tile).  bf16:
    // chunk 4 ks + kq, with ks = 4 u + v at byte koff[v] + 256 u.  FP8: read i
    // (chunk 4 i + kq) at krow + ((4 i + kq) ^ ksw) * 16.
    int koff[4];
#pragma unroll
    for (int v = 0; v < 4; ++v)
        koff[v] = (16 * wave + n) * kRowBytes + (((4 * v + kq) ^ swz(n)) << 4);
    const int krow = (16 * wave + n) * kHeadDim;
    const int ksw = swz8(16 * wave + n);
    // V^T operand (transposing reads).  bf16: key row 32 c + 8 kq + (n >> 2)
    // (+4 for the second read), dims 128 wave + 16 db + 4 (n & 3), i.e. logical
    // chunk 16 wave + 2 db + (n & 3) / 2 at byte 8 (n & 1); rows of different c
    // share the swizzle (32 c is a multiple of 16).  FP8: lane pair n = 2 j +
    // h of group kq addresses key row 32 c + 8 kq + j at byte 8 h of dim chunk
    // 8 wave + db, and lane n receives dim 16 (8 wave + db) + n of those 8
    // keys.  Either way the keys are 32 c + 8 kq .. + 7, those of this lane's
    // P^T operand, in its order.
    int vrow[2], vsw[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        vrow[h] = (8 * kq + (n >> 2) + 4 * h) * kRowBytes + 8 * (n & 1);
        vsw[h] = swz(8 * kq + (n >> 2) + 4 * h);
    }
    const int vchunk0 = 16 * wave + ((n & 3) >> 1);
    const int vr8 = 8 * kq + (n >> 1);
    const int vrow8 = vr8 * kHeadDim + 8 * (n & 1);
    const int vsw8 = swz8(vr8);   // the same for rows 32 c + vr8

    f32x4 o[NC][8];
    float m_ref[NC], l_run[NC];
#pragma unroll
    for (int cb = 0; cb < NC; ++cb) {
#pragma unroll
        for (int db = 0; db < 8; ++db) o[cb][db] = f32x4{};
        m_ref[cb] = -__builtin_inff();
        l_run[cb] = 0.f;
    }

    constexpr int kPoolTile = FP8 ? kTileBytes / 2 : kTileBytes;
    // keys of tile t below k_end (0 past the split: such loads are
    // zero-length, so with kDepth 2 every step issues the same loads)
    auto valid_of = [&](int t) { return max(min(p.k_end - (p.k_begin + t * kPage), kPage), 0); };
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
        const int pg = split_page(a, p, d);
        issue_tile<FP8>(tile_base(a.k_pages, a, pg, p.kvh, kPoolTile), valid_of(d),
                        sK0 + d * kTB, wave, lane);
        issue_tile<FP8>(tile_base(a.v_pages, a, pg, p.kvh, kPoolTile), valid_of(d),
                        sV0 + d * kTB, wave, lane);
    }
    for (int t = 0; t < p.ntiles; ++t) {
        const int key0 = p.k_begin + t * kPage;
        const bool more = t + 1 < p.ntiles;
        const int buf = kDepth == 2 ? (t & 1) : 0;
        const ATTN_LDS char* sK = sK0 + buf * kTB;
        const ATTN_LDS char* sV = sV0 + buf * kTB;
        // the tile this step's refills bring: t + kDepth
        const int pg_next = split_page(a, p, t + kDepth);
        // this wave's K(t) rows are in.  kDepth 1: V(t), issued after them,
        // may still be in flight.  kDepth 2 (the issue order is K0 V0 K1 V1,
        // then per step t: K(t + 2), and V(t + 1) from t = 1): of the loads
        // after K(t), V(t - 1) has landed and at most K(t + 1), V(t) remain
        // (on the first step also V0 is waited for)
        wait_vmcnt<(kDepth == 2 ? 2 : 1) * kLoads>();

        // S^T[16 keys of this wave][16 columns] per block, over 512 dims
        f32x4 s[NC];
        if constexpr (NC == 1) {
            s[0] = f32x4{};
            if constexpr (FP8) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const u32x4 w =
                        *(const ATTN_LDS u32x4*)(sK + krow + (((4 * i + kq) ^ ksw) << 4));
                    s[0] = mfma16x16x32(widen8(w[0], w[1]), qf[0][2 * i], s[0]);
                    s[0] = mfma16x16x32(widen8(w[2], w[3]), qf[0][2 * i + 1], s[0]);
                }
            } else {
#pragma unroll
                for (int ks = 0; ks < 16; ++ks) {
                    const bf16x8 kv =
                        *(const ATTN_LDS bf16x8*)(sK + koff[ks & 3] + 256 * (ks >> 2));
                    s[0] = mfma16x16x32(kv, qf[0][ks], s[0]);
                }
            }
        } else {
            // block 0's Q in VGPRs, the others' in AGPRs.  The asm MFMAs are
            // scheduling boundaries, so the K operand reads are prefetched
            // kAhead k-steps ahead here (E4M3: 8 raw bytes per step, widened
            // just before its MFMAs)
            using Raw = typename std::conditional<FP8, unsigned long long, bf16x8>::type;
            constexpr int kAhead = FP8 ? 4 : 3;
            auto kread = [&](int ks) -> Raw {
                if constexpr (FP8)
                    return *(const ATTN_LDS unsigned long long*)(sK + krow + 8 * (ks & 1) +
                                                    (((2 * (ks & ~1) + kq) ^ ksw) << 4));
                else
                    return *(const ATTN_LDS bf16x8*)(sK + koff[ks & 3] + 256 * (ks >> 2));
            };
            Raw kb[kAhead];
#pragma unroll
            for (int j = 0; j < kAhead; ++j) kb[j] = kread(j);
            static_for<16>([&](auto KS) {
                constexpr int ks = decltype(KS)::value;
                const Raw raw = kb[ks % kAhead];
                if constexpr (ks + kAhead < 16) kb[ks % kAhead] = kread(ks + kAhead);
                bf16x8 kv;
                if constexpr (FP8)
                    kv = widen8(unsigned(raw), unsigned(raw >> 32));
                else
                    kv = raw;
                static_for<NC>([&](auto CB) {
                    constexpr int cb = decltype(CB)::value;
                    qk_mfma<(cb > 0), (ks == 0), (FP8 && cb == 0)>(s[cb], kv, qf[cb][ks]);
                });
            });
            qk_drain<NC>(s);
        }
        // this wave's K rows are free once its reads have returned
        wait_lgkmcnt0();
        __builtin_amdgcn_sched_barrier(0);
        if (kDepth == 2 || more)
            issue_tile<FP8>(tile_base(a.k_pages, a, pg_next, p.kvh, kPoolTile),
                            valid_of(t + kDepth), sK0 + buf * kTB, wave, lane);

        // element i: key 16 wave + 4 kq + i of column 16 cb + n, in log2
        // units; keys a column may not see are -inf (only in the tiles that
        // reach past k_end - q_len: earlier keys are visible to every column).
        // The wave votes to move the references when one of its scores is
        // above its column's reference by more than the margin.
        const bool edge = key0 + kPage > p.k_end - a.q_len;
        const int mykey = key0 + 16 * wave + 4 * kq;
        bool over = false;
#pragma unroll
        for (int cb = 0; cb < NC; ++cb) {
            const float lim = m_ref[cb] + kTileMargin;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float v = s[cb][i] * a.scale_log2;
                if (edge && mykey + i >= col[cb].k_lim) v = -__builtin_inff();
                s[cb][i] = v;
                over |= v > lim;
            }
        }
        // probabilities of this wave's keys against the references -> P
        // buffer t % 2 (two buffers: a wave may write tile t + 1's while
        // another still reads tile t's)
        ATTN_LDS char* sP = sP0 + (t & 1) * kPBytes;
        auto write_p = [&] {
#pragma unroll
            for (int cb = 0; cb < NC; ++cb) {
                const float m_use = finite_or_zero(m_ref[cb]);
                bf16x4 pw;
#pragma unroll
                for (int i = 0; i < 4; ++i) pw[i] = (__bf16)fast_exp2(s[cb][i] - m_use);
                *(ATTN_LDS bf16x4*)(sP + (16 * cb + n) * kPStride + (16 * wave + 4 * kq) * 2) = pw;
            }
        };
        write_p();
        const bool vote = __builtin_amdgcn_ballot_w64(over) != 0;
        if (lane == 0) sVote[(t & 1) * kDecWaves + wave] = vote;

        // this wave's V(t) rows are in.  kDepth 1: after them were issued
        // K(t + 1) (none on the last tile).  kDepth 2 (issue order K0 V0 K1
        // V1, then per step t: K(t + 2), and V(t + 1) from t = 1): after V(t)
        // only K(t + 2) from t = 2 on (the first two steps wait for a little
        // more than they need)
        if constexpr (kDepth == 2) {
            wait_vmcnt<kLoads>();
        } else {
            if (more) wait_vmcnt<kLoads>(); else wait_vmcnt<0>();
        }
        lds_barrier();  // P, the votes and every wave's V(t) rows visible
        // kDepth 2: every wave is past P.V of tile t - 1, so its V buffer
        // takes tile t + 1 (zero-length past the split)
        if (kDepth == 2 && t >= 1)
            issue_tile<FP8>(tile_base(a.v_pages, a, split_page(a, p, t + 1), p.kvh, kPoolTile),
                            valid_of(t + 1), sV0 + ((t + 1) & 1) * kTB, wave, lane);

        const u32x4 votes = *(const ATTN_LDS u32x4*)(sVote + (t & 1) * kDecWaves);
        if (__builtin_expect((votes[0] | votes[1] | votes[2] | votes[3]) != 0, 0)) {
            // Some score is above its reference by more than the margin (the
            // first tile with a visible key always is, against m_ref = -inf):
            // the waves exchange their per-column maxima, a column's reference
            // moves to its tile maximum when that exceeds it by more than the
            // margin (alpha = 0 on the zero O the first time), and the waves
            // write their probabilities again.  Every wave takes the same
            // decisions, so O, l and P are those of a tile-by-tile exchange.
#pragma unroll
            for (int cb = 0; cb < NC; ++cb) {
                float mt = fmaxf(fmaxf(s[cb][0], s[cb][1]), fmaxf(s[cb][2], s[cb][3]));
                mt = fmaxf(mt, __shfl_xor(mt, 16));
                mt = fmaxf(mt, __shfl_xor(mt, 32));
                if (kq == 0) sM[(16 * cb + n) * kDecWaves + wave] = mt;
            }
            lds_barrier();  // column maxima visible
            bool up_any = false;
            float alpha[NC];
#pragma unroll
            for (int cb = 0; cb < NC; ++cb) {
                const f32x4 mm = *(const ATTN_LDS f32x4*)(sM + (16 * cb + n) * kDecWaves);
                const float mt = fmaxf(fmaxf(mm[0], mm[1]), fmaxf(mm[2], mm[3]));
                const bool up = mt > m_ref[cb] + kTileMargin;
                alpha[cb] = up ? fast_exp2(m_ref[cb] - mt) : 1.f;
                m_ref[cb] = up ? mt : m_ref[cb];
                up_any |= up;
            }
            if (__builtin_amdgcn_ballot_w64(up_any)) {
#pragma unroll
                for (int cb = 0; cb < NC; ++cb) {
                    l_run[cb] *= alpha[cb];
                    if constexpr (NC == 1) {
#pragma unroll
                        for (int db = 0; db < 8; ++db) o[cb][db] *= alpha[cb];
                    } else {
                        acc_fence8(o[cb]);
#pragma unroll
                        for (int db = 0; db < 8; ++db) scale_acc4(o[cb][db], alpha[cb]);
                        acc_fence8(o[cb]);
                    }
                }
            }
            write_p();
            lds_barrier();  // the new P visible
        }

        // P^T operand: keys 32 c + 8 kq .. + 7 of column 16 cb + n
        bf16x8 pf[NC][2];
#pragma unroll
        for (int cb = 0; cb < NC; ++cb) {
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                pf[cb][c] = *(const ATTN_LDS bf16x8*)(sP + (16 * cb + n) * kPStride +
                                                      (32 * c + 8 * kq) * 2);
                l_run[cb] = pair_sum(pf[cb][c], l_run[cb]);
            }
        }
        // O^T[128 dims of this wave][16 columns] += V^T P^T per block
#pragma unroll
        for (int c = 0; c < 2; ++c) {
#pragma unroll
            for (int db = 0; db < 8; ++db) {
                bf16x8 vt;
                if constexpr (FP8) {
                    const v2i32 t8 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                        (ATTN_LDS v2i32*)(sV + 32 * c * kHeadDim + vrow8 +
                                          (((8 * wave + db) ^ vsw8) << 4)));
                    vt = widen8((uint32_t)t8[0], (uint32_t)t8[1]);
                } else {
                    const int ch = vchunk0 + 2 * db;
                    const ATTN_LDS char* base = sV + 32 * c * kRowBytes;
                    const bf16x4 va = lds_read_tr16(base + vrow[0] + ((ch ^ vsw[0]) << 4));
                    const bf16x4 vb = lds_read_tr16(base + vrow[1] + ((ch ^ vsw[1]) << 4));
                    vt = __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7);
                }
#pragma unroll
                for (int cb = 0; cb < NC; ++cb) o[cb][db] = mfma16x16x32(vt, pf[cb][c], o[cb][db]);
            }
        }
        if constexpr (kDepth == 1) {
            lds_barrier();  // every wave is done with the V buffer
            if (more)
                issue_tile<FP8>(tile_base(a.v_pages, a, pg_next, p.kvh, kPoolTile),
                                valid_of(t + 1), sV0, wave, lane);
        }
    }
    if constexpr (kDepth == 2) wait_vmcnt<0>();   // the zero-length loads past the split
    const size_t slot0 = (((size_t)p.b * a.hkv + p.kvh) * a.max_splits + p.split) * a.sub * a.cols;
#pragma unroll
    for (int cb = 0; cb < NC; ++cb)
        write_partial<8>(a, slot0 + 16 * cb + n, 16 * cb + n, kq, 128 * wave, o[cb], m_ref[cb],
                         l_run[cb]);
}

// ============================== FP8 pool ===================================


// K or V half page (32 rows of 512 E4M3 bytes) -> this wave's LDS buffer by
// DMA, 2 whole rows (8 full 128-byte lines) per instruction: lane l lands at
// LDS byte 16 l of rows 2 i, 2 i + 1, i.e. row 2 i + l / 32 at chunk position
// l % 32, and so fetches logical chunk (l % 32) ^ swz8(row).  Rows past
// `rows` arrive as zeros.
__device__ __forceinline__ void dma_half(const char* src, int rows, ATTN_LDS char* buf,
                                           int lane) {
    const u32x4 rsrc = buffer_rsrc(src, (uint32_t)rows * kHeadDim);
    const uint32_t lds = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uintptr_t)buf);
    const int hl = lane >> 5;
    const int lane_base = (hl << 9) | (((lane & 31) ^ hl) << 4);
    static_for<kHalfKeys / 2>([&](auto I) { dma_row_pair<decltype(I)::value>(rsrc, lds, lane_base); });
    race_delay<0>();
}

// K operand of key group gm (keys 16 gm .. 16 gm + 15), read i: key
// 16 gm + n, bytes 64 i + 16 kq .. + 15 (logical chunk 4 i + kq), i.e. the
// lane's operands of k-steps 2 i and 2 i + 1 (8 dims each).  Within each 8
// lanes of one read the rows differ in their low 3 bits, so swz8 puts their
// chunks in distinct bank groups.
__device__ __forceinline__ u32x4 k_read(const ATTN_LDS char* sk, int gm, int i, int n, int kq) {
    const int row = 16 * gm + n;
    return *(const ATTN_LDS u32x4*)(sk + row * kHeadDim + (((4 * i + kq) ^ swz8(row)) << 4));
}


// Per wave step (half page u of this wave; one K and one V half-page buffer
// in LDS, both filled by whole-row DMA):
//   wait for K(u), QK(u) from the K buffer, then K(u + NW) -> the K buffer
//   (its reads have returned); softmax; wait for V(u), PV(u) from the V
//   buffer, then V(u + NW) -> the V buffer.  Every wait leaves exactly the
//   other buffer's kHalfKeys / 2 loads in flight.  Past the split's end the
//   loads are zero-length.
template <int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_split_fp8_kernel(DecodeArgs a) {
    __shared__ __attribute__((aligned(1024))) char smem[NW * 2 * kHalfBytes];
    SplitPlan p;
    if (!plan_split(a, p)) return;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15;   // query head of the group (MFMA column)
    const int kq = lane >> 4;  // k-group
    // this wave's K and V half-page buffers
    ATTN_LDS char* sk = (ATTN_LDS char*)smem + wave * 2 * kHalfBytes;
    ATTN_LDS char* sv = sk + kHalfBytes;

    // Q^T operand of k-step ks: dims 64 (ks / 2) + 16 kq + 8 (ks % 2) .. + 7,
    // the order in which the K loads deliver them
    const Column col = column_of(a, p, n);
    bf16x8 qf[16];
    {
        const __bf16* qrow = a.q + col.q_row * kHeadDim;
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) {
            const bf16x8 v = *(const bf16x8*)(qrow + 64 * (ks >> 1) + 16 * kq + 8 * (ks & 1));
            qf[ks] = col.ok ? v : bf16x8{};
        }
    }
    // V^T operand, read transposed: within each 16-lane group kq, lane
    // 2 j + h addresses key row r_j = (j < 4 ? 4 kq + j : 16 + 4 kq + j - 4) at
    // byte 16 db + 8 h, and lane i receives dim 16 db + i of rows r_0 .. r_7:
    // the same keys, in the same order, as this lane's P^T operand (the QK
    // accumulators of key groups 0 and 1).
    const int tj = n >> 1;
    const int vr = tj < 4 ? 4 * kq + tj : 16 + 4 * kq + tj - 4;
    const int vrow = vr * kHeadDim + 8 * (n & 1);
    const int vsw = swz8(vr);

    f32x4 o[32];
#pragma unroll
    for (int db = 0; db < 32; ++db) o[db] = f32x4{};
    float m_ref = -__builtin_inff();
    float l_run = 0.f;

    const int nhalf = (p.k_end - p.k_begin + kHalfKeys - 1) / kHalfKeys;
    const int count = nhalf > wave ? (nhalf - wave + NW - 1) / NW : 0;
    // half page u of the split: rows past its end (or past the split) are
    // zero-length loads, so every step issues the same count
    auto issue = [&](int u, bool is_k) {
        int rows = p.k_end - (p.k_begin + u * kHalfKeys);
        rows = rows < 0 ? 0 : (rows > kHalfKeys ? kHalfKeys : rows);
        const int pg = split_page(a, p, u >> 1);
        const int off = (u & 1) * kHalfBytes;
        dma_half(tile_base(is_k ? a.k_pages : a.v_pages, a, pg, p.kvh, kTileBytes / 2) + off,
                 rows, is_k ? sk : sv, lane);
    };
    issue(wave, true);
    issue(wave, false);
    for (int c = 0; c < count; ++c) {
        const int u = wave + NW * c;
        const int key0 = p.k_begin + u * kHalfKeys;
        // K(u) landed; V(u), issued after it, may still be in flight
        wait_vmcnt<kHalfKeys / 2>();
        // S^T[32 keys][16 heads]: key group gm = keys 16 gm .. 16 gm + 15
        f32x4 s[2];
#pragma unroll
        for (int gm = 0; gm < 2; ++gm) {
            f32x4 s0 = f32x4{}, s1 = f32x4{};
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const u32x4 w = k_read(sk, gm, i, n, kq);
                s0 = mfma16x16x32(widen8(w[0], w[1]), qf[2 * i], s0);
                s1 = mfma16x16x32(widen8(w[2], w[3]), qf[2 * i + 1], s1);
            }
            s[gm] = s0 + s1;   // element i: key 16 gm + 4 kq + i of head n
        }
        // the K buffer is free once its reads have returned: refill it with
        // this wave's next half page (one wave per buffer, so no barrier)
        wait_lgkmcnt0();
        __builtin_amdgcn_sched_barrier(0);
        issue(u + NW, true);

        // softmax against the reference maximum
        float x[8];
        float mt = -__builtin_inff();
#pragma unroll
        for (int gm = 0; gm < 2; ++gm)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = key0 + 16 * gm + 4 * kq + i;
                const float v = key < col.k_lim ? s[gm][i] * a.scale_log2 : -__builtin_inff();
                x[4 * gm + i] = v;
                mt = fmaxf(mt, v);
            }
        mt = fmaxf(mt, __shfl_xor(mt, 16));
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        // the first half page with a visible key moves the reference (alpha
        // = 0 on the zero O); before it mt = m_ref = -inf and nothing changes
        // (a later token of a multi-token decode can see keys an earlier one
        // cannot)
        const bool up = mt > m_ref + kRefMargin;
        if (__builtin_amdgcn_ballot_w64(up)) {
            const float m_new = up ? mt : m_ref;
            const float alpha = up ? fast_exp2(m_ref - m_new) : 1.f;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < 32; ++db) o[db] *= alpha;
            m_ref = m_new;
        }
        bf16x8 pf;
        float psum = 0.f;
        const float m_use = finite_or_zero(m_ref);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float pv = fast_exp2(x[j] - m_use);
            psum += pv;
            pf[j] = (__bf16)pv;
        }
        l_run += psum;

        // O^T[512 dims][16 heads] += V^T P^T over the 32 keys; V(u) landed
        // (K(u + NW), issued after it, may still be in flight)
        wait_vmcnt<kHalfKeys / 2>();
#pragma unroll
        for (int db = 0; db < 32; ++db) {
            const v2i32 t8 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (ATTN_LDS v2i32*)(sv + vrow + ((db ^ vsw) << 4)));
            o[db] = mfma16x16x32(widen8((uint32_t)t8[0], (uint32_t)t8[1]), pf, o[db]);
            // bound the operands in flight
            if ((db & 7) == 7 && db < 31) __builtin_amdgcn_sched_barrier(0);
        }
        // the V buffer is free once its reads have returned
        wait_lgkmcnt0();
        __builtin_amdgcn_sched_barrier(0);
        issue(u + NW, false);
    }
    wait_vmcnt<0>();   // the last (zero-length) loads
    const size_t slot =
        ((((size_t)p.b * a.hkv + p.kvh) * a.max_splits + p.split) * a.sub + wave) * a.cols + n;
    write_partial<32>(a, slot, n, kq, 0, o, m_ref, l_run);
}

// One workgroup per (sequence, token, query head): combine the partials,
// mu = max(m_i, sink), o = sum 2^(m_i - mu) O_i / (sum 2^(m_i - mu) l_i +
// 2^(sink - mu)), in log2 units (m_i already are; the sink logit is scaled by
// log2(e)).  A partial that saw no key (m = -inf, l = 0, O = 0) adds nothing;
// with no key at all the output is 0 and the log-sum-exp is the sink logit,
// or -inf without a sink (vLLM flash-attention PR 199, second review,
// finding F4).
template <bool OUT_FP32>
__global__ __launch_bounds__(128) void decode_merge_kernel(DecodeArgs a, void* out) {
    const int h = blockIdx.x % a.hq;
    const int bt = blockIdx.x / a.hq;     // b q_len + token
    const int b = bt / a.q_len;
    const int t = bt - b * a.q_len;
    const int kvh = h / a.g;
    const int c = t * a.g + (h - kvh * a.g);
    int L = a.kv_lens[b];
    L = L < 0 ? 0 : (L > a.max_pages * kPage ? a.max_pages * kPage : L);
    const int split_keys = a.tiles_per_split * kPage;
    int ns = (L + split_keys - 1) / split_keys;
    ns = (ns > a.max_splits ? a.max_splits : ns) * a.sub;   // every non-empty split wrote a.sub
    const size_t slot0 = (((size_t)b * a.hkv + kvh) * a.max_splits) * a.sub * a.cols + c;
    const float sink2 = a.sinks ? a.sinks[h] * 1.4426950408889634f : -__builtin_inff();
    float mu = sink2;
    for (int i = 0; i < ns; ++i) mu = fmaxf(mu, a.part_ml[2 * (slot0 + (size_t)i * a.cols)]);
    f32x4 acc = f32x4{};
    float den = 0.f;
    const int d0 = 4 * threadIdx.x;
    if (mu != -__builtin_inff()) {
        for (int i = 0; i < ns; ++i) {
            const size_t slot = slot0 + (size_t)i * a.cols;
            const float m = a.part_ml[2 * slot];
            if (m == -__builtin_inff()) continue;   // empty partial
            const float w = fast_exp2(m - mu);
            den += w * a.part_ml[2 * slot + 1];
            acc += w * *(const f32x4*)(a.part_o + slot * kHeadDim + d0);
        }
        den += fast_exp2(sink2 - mu);   // 0 without a sink
    }
    // IEEE division, as in prefill; no key and no sink gives 0
    const float dd = den > 0.f ? den : 1.f;
    const size_t obase = ((size_t)bt * a.hq + h) * kHeadDim + d0;
    const f32x4 v = {acc[0] / dd, acc[1] / dd, acc[2] / dd, acc[3] / dd};
    if constexpr (OUT_FP32) {
        *(f32x4*)((float*)out + obase) = v;
    } else {
        *(bf16x4*)((__bf16*)out + obase) = bf16x4{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
    }
    if (a.lse && threadIdx.x == 0)
        a.lse[(size_t)bt * a.hq + h] =
            den > 0.f ? (mu + __builtin_log2f(den)) * 0.6931471805599453f : -__builtin_inff();
}

// Scratch of attn_decode_splitk_ex_noalloc: the partials live in this
// device array instead of a caller workspace.  Host code never uses the
// array's name as an address (on the host it is only a stand-in for the
// symbol): each device's address comes from hipGetSymbolAddress, taken once
// per device with that device current, and is kept in scratch_dev.
constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kMaxScratchDevices = 64;
std::mutex scratch_mu;
void* scratch_dev[kMaxScratchDevices] = {};

}  // namespace
}  // namespace attn

static __device__ __align__(256) char scratch[attn::kScratchBytes];

namespace attn {
namespace {

// The scratch address on the device `stream` belongs to (the current device
// for the null stream).
int scratch_for_stream(hipStream_t stream, void** out) {
    int dev = -1;
    if (stream) {
        hipDevice_t d;
        if (hipStreamGetDevice(stream, &d) != hipSuccess) return ATTN_ERR_HIP;
        dev = (int)d;
    } else if (hipGetDevice(&dev) != hipSuccess) {
        return ATTN_ERR_HIP;
    }
    if (dev < 0 || dev >= kMaxScratchDevices) return ATTN_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_dev[dev]) {
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess) return ATTN_ERR_HIP;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return ATTN_ERR_HIP;
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev && hipSetDevice(cur) != hipSuccess) return ATTN_ERR_HIP;
        if (e != hipSuccess || !p) return ATTN_ERR_HIP;
        scratch_dev[dev] = p;
    }
    *out = scratch_dev[dev];
    return ATTN_OK;
}

// Bytes of the routed path's argument arrays at the head of the workspace
// (2 batch + 1 ints, rounded up to 256 so the partials stay aligned).
size_t routed_meta_bytes(int batch) {
    return ((size_t)(2 * batch + 1) * sizeof(int) + 255) / 256 * 256;
}

// Default split: about kDefaultTargetWgs splits over the largest key ranges.
// A split with two or three 16-column blocks (a multi-token decode) pays
// about three times the fixed cost per split of a one-block split (Q of up
// to 48 columns, their 96 KB of partials, the first tile's reference
// exchange, the pipeline fill), so its splits are made twice as long.
int default_keys_per_split(int batch, int hkv, int max_kv_len, int col_blocks) {
    const long long total = (long long)batch * hkv * max_kv_len;
    const int target = col_blocks > 1 ? kDefaultTargetWgs / 2 : kDefaultTargetWgs;
    long long s = (total + target - 1) / target;
    s = (s + kPage - 1) / kPage * kPage;
    if (s < 4 * kPage) s = 4 * kPage;
    return (int)s;
}

// Key ranges of a routed call: the caller's, else the decode default (the
// prefill's own plan counts compute rounds and keeps one range for decode
// shapes; here the work is the KV stream, and the ranges balance the
// sequences' different lengths).
int routed_keys_per_split(int batch, int hkv, int max_kv_len, int keys_per_split) {
    return keys_per_split ? keys_per_split : default_keys_per_split(batch, hkv, max_kv_len, 1);
}

}  // namespace

}  // namespace attn

extern "C" size_t attn_decode_splitk_ex_workspace_size(int batch, int q_len, int num_q_heads,
                                                       int num_kv_heads, int max_kv_len,
                                                       int keys_per_split) {
    using namespace attn;
    if (batch < 1 || q_len < 1 || num_q_heads < 1 || num_kv_heads < 1 || max_kv_len < 1 ||
        num_q_heads % num_kv_heads || keys_per_split < 0 || keys_per_split % kPage)
        return 0;
    if ((long long)q_len * (num_q_heads / num_kv_heads) > kDecCols) {
        // routed to the split-K prefill: row offsets and chunk starts, then
        // the prefill's partials
        if ((long long)batch * q_len > 0x7fffffffLL) return 0;
        return routed_meta_bytes(batch) +
               attn_prefill_hd512_splitk_workspace_size(
                   batch, q_len, batch * q_len, num_q_heads, num_kv_heads, max_kv_len,
                   routed_keys_per_split(batch, num_kv_heads, max_kv_len, keys_per_split));
    }
    const int nc = (q_len * (num_q_heads / num_kv_heads) + kDecRows - 1) / kDecRows;
    const int kps = keys_per_split ? keys_per_split
                                   : default_keys_per_split(batch, num_kv_heads, max_kv_len, nc);
    const size_t splits = (size_t)(max_kv_len + kps - 1) / kps;
    // hkv * (q_len * g) columns = q_len * hq
    const size_t slots = (size_t)batch * q_len * num_q_heads * splits * kMaxSub;
    return slots * (kHeadDim + 2) * sizeof(float);
}

extern "C" size_t attn_decode_splitk_workspace_size(int batch, int num_q_heads, int num_kv_heads,
                                                    int max_kv_len, int keys_per_split) {
    return attn_decode_splitk_ex_workspace_size(batch, 1, num_q_heads, num_kv_heads, max_kv_len,
                                                keys_per_split);
}

namespace attn {
namespace {

// Multi-token decode with more (token, head) columns than the decode tile's
// 16 (e.g. 5 tokens at g = 8: a draft of 4 plus the current token) is the
// prefill of q_len rows per sequence at positions kv_len - q_len ..
// kv_len - 1: it runs as the split-K prefill (which reads each K/V tile once
// for every row of the group), after this kernel has written the prefill's
// device-side arguments: cu[b] = b q_len (b = 0 .. batch) and
// qs[b] = kv_len[b] - q_len.
__global__ __launch_bounds__(256) void decode_route_meta(const int* kv_lens, int batch,
                                                         int q_len, int* cu, int* qs) {
    for (int b = threadIdx.x; b <= batch; b += blockDim.x) {
        cu[b] = b * q_len;
        if (b < batch) qs[b] = kv_lens[b] - q_len;
    }
}

int decode_as_prefill(const void* q, const void* k_pages, const void* v_pages, int kv_dtype,
                      float k_scale, float v_scale, const int32_t* page_table,
                      const int32_t* kv_lens, int batch, int q_len, int num_q_heads,
                      int num_kv_heads, int head_dim, int page_size, int num_pages,
                      int max_pages_per_seq, int max_kv_len, int keys_per_split,
                      float softmax_scale, const float* sinks, void* workspace,
                      size_t workspace_bytes, bool noalloc, void* out, int out_dtype,
                      float* lse, hipStream_t stream) {
    // every check the split-K prefill makes runs here, before the kernel
    // below is launched (the caller has checked pointers, sizes and layout)
    if ((long long)batch * q_len > 0x7fffffffLL) return ATTN_ERR_SHAPE;
    if ((long long)batch * q_len * num_q_heads > 0x7fffffffLL) return ATTN_ERR_SHAPE;
    if ((long long)max_pages_per_seq * kPage > 0x7fffffffLL) return ATTN_ERR_SHAPE;
    if (num_q_heads / num_kv_heads > kRoutedMaxGroup) return ATTN_ERR_UNSUPPORTED;
    if (kv_dtype != ATTN_BF16 && kv_dtype != ATTN_FP8_E4M3) return ATTN_ERR_UNSUPPORTED;
    if (out_dtype != ATTN_BF16 && out_dtype != ATTN_FP32) return ATTN_ERR_UNSUPPORTED;
    if (kv_dtype == ATTN_FP8_E4M3 && (!(k_scale > 0.f) || !(v_scale > 0.f))) return ATTN_ERR_SHAPE;
    const int total = batch * q_len;
    const size_t meta = routed_meta_bytes(batch);
    keys_per_split = routed_keys_per_split(batch, num_kv_heads, max_kv_len, keys_per_split);
    const size_t part = attn_prefill_hd512_splitk_workspace_size(
        batch, q_len, total, num_q_heads, num_kv_heads, max_kv_len, keys_per_split);
    if (noalloc) {
        if (meta + part > kScratchBytes) return ATTN_ERR_WORKSPACE;
        const int rc = scratch_for_stream(stream, &workspace);
        if (rc != ATTN_OK) return rc;
        workspace_bytes = kScratchBytes;
    } else if (!workspace || workspace_bytes < meta + part) {
        return ATTN_ERR_WORKSPACE;
    }
    int* cu = (int*)workspace;
    int* qs = cu + batch + 1;
    hipLaunchKernelGGL(decode_route_meta, dim3(1), dim3(256), 0, stream, kv_lens, batch, q_len,
                       cu, qs);
    if (hipGetLastError() != hipSuccess) return ATTN_ERR_HIP;
    return attn_prefill_hd512_splitk(q, k_pages, v_pages, kv_dtype, k_scale, v_scale, page_table,
                                     cu, qs, kv_lens, batch, total, q_len, num_q_heads,
                                     num_kv_heads, head_dim, page_size, num_pages,
                                     max_pages_per_seq, max_kv_len, keys_per_split,
                                     softmax_scale, sinks, part ? (char*)workspace + meta : nullptr,
                                     part ? workspace_bytes - meta : 0, out, out_dtype, lse,
                                     stream);
}

// Validation and launch shared by the caller-workspace entry point and the
// one that allocates nothing.  workspace == nullptr asks for the library's
// static scratch (attn_decode_splitk_ex_noalloc).
int decode_launch(const void* q, const void* k_pages, const void* v_pages, int kv_dtype,
                  float k_scale, float v_scale, const int32_t* page_table,
                  const int32_t* kv_lens, int batch, int q_len, int num_q_heads,
                  int num_kv_heads, int head_dim, int page_size, int num_pages,
                  int max_pages_per_seq, int max_kv_len, int keys_per_split,
                  float softmax_scale, const float* sinks, void* workspace,
                  size_t workspace_bytes, bool noalloc, void* out, int out_dtype, float* lse,
                  hipStream_t stream) {
    if (!q || !k_pages || !v_pages || !page_table || !kv_lens || !out) return ATTN_ERR_NULL;
    if (batch < 1 || q_len < 1 || num_q_heads < 1 || num_kv_heads < 1 || num_pages < 1 ||
        max_pages_per_seq < 1 || max_kv_len < 1 || keys_per_split < 0 ||
        !(softmax_scale == softmax_scale))
        return ATTN_ERR_SHAPE;
    if (num_q_heads % num_kv_heads || keys_per_split % kPage) return ATTN_ERR_SHAPE;
    if ((long long)max_kv_len > (long long)max_pages_per_seq * kPage) return ATTN_ERR_SHAPE;
    if (head_dim != kHeadDim || page_size != kPage) return ATTN_ERR_UNSUPPORTED;
    const int g = num_q_heads / num_kv_heads;
    if ((long long)q_len * g > kDecCols)
        return decode_as_prefill(q, k_pages, v_pages, kv_dtype, k_scale, v_scale, page_table,
                                 kv_lens, batch, q_len, num_q_heads, num_kv_heads, head_dim,
                                 page_size, num_pages, max_pages_per_seq, max_kv_len,
                                 keys_per_split, softmax_scale, sinks, workspace,
                                 workspace_bytes, noalloc, out, out_dtype, lse, stream);
    if (kv_dtype != ATTN_BF16 && kv_dtype != ATTN_FP8_E4M3) return ATTN_ERR_UNSUPPORTED;
    if (out_dtype != ATTN_BF16 && out_dtype != ATTN_FP32) return ATTN_ERR_UNSUPPORTED;
    if (kv_dtype == ATTN_FP8_E4M3 && (!(k_scale > 0.f) || !(v_scale > 0.f))) return ATTN_ERR_SHAPE;
    const bool fp8 = kv_dtype == ATTN_FP8_E4M3;
    const int nc = (q_len * g + kDecRows - 1) / kDecRows;   // 16-column blocks
    const int kps = keys_per_split ? keys_per_split
                                   : default_keys_per_split(batch, num_kv_heads, max_kv_len, nc);
    // FP8 with one block: the half-page kernel (a partial per wave)
    const int sub = fp8 && nc == 1 ? kFp8Waves : 1;
    const int max_splits = (max_kv_len + kps - 1) / kps;
    // partial slots the launch writes and reads: (O, m, l) per split, partial
    // of the split and (token, query head)
    const size_t slots = (size_t)batch * q_len * num_q_heads * max_splits * sub;
    if (noalloc) {
        if (slots * (kHeadDim + 2) * sizeof(float) > kScratchBytes) return ATTN_ERR_WORKSPACE;
        const int rc = scratch_for_stream(stream, &workspace);
        if (rc != ATTN_OK) return rc;
    } else {
        const size_t need = attn_decode_splitk_ex_workspace_size(batch, q_len, num_q_heads,
                                                                 num_kv_heads, max_kv_len,
                                                                 keys_per_split);
        if (!workspace || workspace_bytes < need || need == 0) return ATTN_ERR_WORKSPACE;
    }

    DecodeArgs a;
    a.q = (const __bf16*)q;
    a.k_pages = (const char*)k_pages;
    a.v_pages = (const char*)v_pages;
    a.page_table = page_table;
    a.kv_lens = kv_lens;
    a.batch = batch;
    a.hq = num_q_heads;
    a.hkv = num_kv_heads;
    a.g = g;
    a.q_len = q_len;
    a.cols = q_len * g;
    a.max_pages = max_pages_per_seq;
    a.num_pages = num_pages;
    a.max_splits = max_splits;
    a.tiles_per_split = kps / kPage;
    a.part_o = (float*)workspace;
    a.part_ml = (float*)workspace + slots * kHeadDim;
    a.sub = sub;
    a.scale_log2 = softmax_scale * 1.4426950408889634f * (fp8 ? k_scale : 1.f);
    a.v_scale = fp8 ? v_scale : 1.f;
    a.sinks = sinks;
    a.lse = lse;
    const long long grid = (long long)batch * num_kv_heads * a.max_splits;
    const long long mgrid = (long long)batch * q_len * num_q_heads;
    if (grid > 0x7fffffffLL || mgrid > 0x7fffffffLL) return ATTN_ERR_SHAPE;
    const dim3 tg((unsigned)grid), tb(kDecThreads);
    if (fp8) {
        if (nc == 1)
            hipLaunchKernelGGL(decode_split_fp8_kernel<kFp8Waves>, dim3((unsigned)grid),
                               dim3(64 * kFp8Waves), 0, stream, a);
        else if (nc == 2)
            hipLaunchKernelGGL((decode_split_tile_kernel<true, 2>), tg, tb, 0, stream, a);
        else
            hipLaunchKernelGGL((decode_split_tile_kernel<true, 3>), tg, tb, 0, stream, a);
    } else {
        if (nc == 1)
            hipLaunchKernelGGL((decode_split_tile_kernel<false, 1>), tg, tb, 0, stream, a);
        else if (nc == 2)
            hipLaunchKernelGGL((decode_split_tile_kernel<false, 2>), tg, tb, 0, stream, a);
        else
            hipLaunchKernelGGL((decode_split_tile_kernel<false, 3>), tg, tb, 0, stream, a);
    }
    if (hipGetLastError() != hipSuccess) return ATTN_ERR_HIP;
    if (out_dtype == ATTN_FP32)
        hipLaunchKernelGGL(decode_merge_kernel<true>, dim3((unsigned)mgrid), dim3(128), 0, stream,
                           a, out);
    else
        hipLaunchKernelGGL(decode_merge_kernel<false>, dim3((unsigned)mgrid), dim3(128), 0,
                           stream, a, out);
    return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

}  // namespace
}  // namespace attn

extern "C" int attn_decode_splitk_ex(const void* q, const void* k_pages, const void* v_pages,
                                     int kv_dtype, float k_scale, float v_scale,
                                     const int32_t* page_table, const int32_t* kv_lens,
                                     int batch, int q_len, int num_q_heads, int num_kv_heads,
                                     int head_dim, int page_size, int num_pages,
                                     int max_pages_per_seq, int max_kv_len, int keys_per_split,
                                     float softmax_scale, const float* sinks, void* workspace,
                                     size_t workspace_bytes, void* out, int out_dtype,
                                     float* lse, hipStream_t stream) {
    return attn::decode_launch(q, k_pages, v_pages, kv_dtype, k_scale, v_scale, page_table,
                               kv_lens, batch, q_len, num_q_heads, num_kv_heads, head_dim,
                               page_size, num_pages, max_pages_per_seq, max_kv_len,
                               keys_per_split, softmax_scale, sinks, workspace, workspace_bytes,
                               false, out, out_dtype, lse, stream);
}

extern "C" int attn_decode_splitk_ex_noalloc(const void* q, const void* k_pages,
                                             const void* v_pages, int kv_dtype, float k_scale,
                                             float v_scale, const int32_t* page_table,
                                             const int32_t* kv_lens, int batch, int q_len,
                                             int num_q_heads, int num_kv_heads, int head_dim,
                                             int page_size, int num_pages,
                                             int max_pages_per_seq, int max_kv_len,
                                             int keys_per_split, float softmax_scale,
                                             const float* sinks, void* out, int out_dtype,
                                             float* lse, hipStream_t stream) {
    return attn::decode_launch(q, k_pages, v_pages, kv_dtype, k_scale, v_scale, page_table,
                               kv_lens, batch, q_len, num_q_heads, num_kv_heads, head_dim,
                               page_size, num_pages, max_pages_per_seq, max_kv_len,
                               keys_per_split, softmax_scale, sinks, nullptr, 0, true, out,
                               out_dtype, lse, stream);
}

extern "C" int attn_decode_splitk(const void* q, const void* k_pages, const void* v_pages,
                                  int kv_dtype, float k_scale, float v_scale,
                                  const int32_t* page_table, const int32_t* kv_lens, int batch,
                                  int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                                  int num_pages, int max_pages_per_seq, int max_kv_len,
                                  int keys_per_split, float softmax_scale, void* workspace,
                                  size_t workspace_bytes, void* out, int out_dtype,
                                  hipStream_t stream) {
    return attn_decode_splitk_ex(q, k_pages, v_pages, kv_dtype, k_scale, v_scale, page_table,
                                 kv_lens, batch, 1, num_q_heads, num_kv_heads, head_dim,
                                 page_size, num_pages, max_pages_per_seq, max_kv_len,
                                 keys_per_split, softmax_scale, nullptr, workspace,
                                 workspace_bytes, out, out_dtype, nullptr, stream);
}
