// Pieces shared by the prefill kernels' translation units: the bf16 /
// widened-FP8 kernel (prefill_hd512.hip) and the block-scaled FP8 MFMA kernel
// (prefill_fp8mma.hip).  Both take one workgroup of 4 waves per 128 packed
// query rows and keep the same online-softmax bookkeeping (a per-row
// reference maximum that is raised, with O and l rescaled, only for the key
// blocks that would overflow against it).  The host validates every
// argument in prefill_launch before a launch.
#pragma once

#include "attn_host.h"
#include "device_common.h"

namespace attn {

constexpr int kRowsPerWg = 128;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
// Page ids of the first kPagesInLds tiles are staged in LDS at the start of
// the workgroup (reading them from the scalar cache inside the loop stalls
// the wave: scalar loads share the LDS wait counter and return out of order).
constexpr int kPagesInLds = 4096;

// Masks one block's raw scores in place: element i is key
// key_base + 8(i/4) + (i%4) (key_base includes 4h); keys >= n_row get -inf,
// and with a window so do keys < lo_row.
template <bool WINDOW>
__device__ __forceinline__ void mask_block(f32x16& s, int key_base, int n_row, int lo_row) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int key = key_base + 8 * (i >> 2) + (i & 3);
        const bool vis = WINDOW ? (key < n_row && key >= lo_row) : key < n_row;
        s[i] = vis ? s[i] : -__builtin_inff();
    }
}

// x *= s for every element of an accumulator held in AGPRs, one element at a
// time through one VGPR (VALU cannot read AGPRs): written as asm so that the
// accumulators stay in AGPRs instead of being copied out whole.
__device__ __forceinline__ void scale_acc(f32x16& acc, float s) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        float x = acc[i];
        float t;
        asm volatile(
            "v_accvgpr_read_b32 %1, %0\n\t"
            "v_mul_f32 %1, %1, %2\n\t"
            "v_accvgpr_write_b32 %0, %1"
            : "+a"(x), "=&v"(t)
            : "v"(s));
        acc[i] = x;
    }
}

// Wait states around scale_acc, tied to every accumulator so that no MFMA
// moves across them: an MFMA's result must be written before v_accvgpr_read
// reads it, and an accumulator written by v_accvgpr_write before an MFMA
// reads it as its C operand.
template <int NDB>
__device__ __forceinline__ void acc_fence(f32x16 (&o)[NDB]) {
    static_assert(NDB == 16 || NDB == 8, "accumulator blocks");
    if constexpr (NDB == 16)
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                     : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]), "+a"(o[4]), "+a"(o[5]),
                       "+a"(o[6]), "+a"(o[7]), "+a"(o[8]), "+a"(o[9]), "+a"(o[10]), "+a"(o[11]),
                       "+a"(o[12]), "+a"(o[13]), "+a"(o[14]), "+a"(o[15]));
    else
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                     : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]), "+a"(o[4]), "+a"(o[5]),
                       "+a"(o[6]), "+a"(o[7]));
}

struct PrefillArgs {
    const __bf16* q;
    const char* k_pages;
    const char* v_pages;
    const int* page_table;
    const int* cu_seqlens_q;
    const int* q_start;
    const int* kv_lens;
    void* out;
    int batch, total_q, hq, hkv, g, max_pages, num_pages;
    int tok_per_wg;     // tokens per workgroup = 128 / g (rounded down)
    int wgs_per_seq;    // ceil(max_q_len / tok_per_wg)
    float scale_log2;   // softmax_scale * log2(e) (* k_scale for an FP8 pool)
    float v_scale;      // FP8 pool: value dequantisation scale, applied to O (1 for bf16)
    const float* sinks; // per query head sink logit (natural-log units), or null
    float* lse;         // [total_q][hq] natural-log log-sum-exp, or null
    // split-K over keys: workgroup split s covers key tiles
    // [s split_tiles, (s + 1) split_tiles) and writes unnormalised partials
    int nsplit, split_tiles;
    float* part_o;      // [nsplit][total_q][hq][512] fp32, O * v_scale
    float* part_ml;     // [nsplit][total_q][hq][2]  (m in log2 units, l)
    int window;         // sliding window in keys (0: none)
    int ring_pages;     // ring cache pages per sequence (0: unbounded cache)
    // fused append: the chunk's new K and V rows, bf16 [total_q][hkv][512]
    const char* k_new;
    const char* v_new;
    // persistent launch: the unit counter (workspace) and the unit count
    int* unit_counter;
    int total_units;
};

// The row a prefill workgroup's lane holds, for prefill_epilogue.
struct RowSlot {
    int q0;        // first query row of the sequence
    int q_row;     // the row's query-row index (q0 + token)
    int head;      // its query head
    int t0, t_last;// the workgroup's first and last token of the sequence
    int kvh;       // the workgroup's KV head
    int split;     // split-K range (0 without split-K)
    bool valid;    // a real row (padding rows shadow the last token)
};

// Epilogue shared by the prefill kernels.  Lane (n = lane % 32, h = lane / 32)
// holds dims 32 db + 8 (i / 4) + 4 h + i % 4 of its row in o[db][i] (O in the
// units of l), its half of the row's sum of p in l_run and the row's
// reference m_ref (log2 units).  SPLIT writes the split-K partial (O *
// v_scale, m, l); otherwise the output is O / l with the sink, and the
// log-sum-exp when asked for.  SCALE_V multiplies by v_scale (FP8 pools).
// STAGE (bf16 output) writes the rows through LDS at `smem` (4 waves x 32
// rows x 2 D bytes, free by then) so that every store covers whole rows.
template <bool OUT_FP32, bool SPLIT, int D, bool STAGE, bool SCALE_V>
__device__ __forceinline__ void prefill_epilogue(const PrefillArgs& a, f32x16 (&o)[D / 32],
                                                 float l_run, float m_ref, bool any_tile,
                                                 const RowSlot& r, ATTN_LDS char* smem, int lane,
                                                 int wave) {
    const int n = lane & 31;
    const int h = lane >> 5;
    float l_tot = l_run + __shfl_xor(l_run, 32);
    if constexpr (SPLIT) {
        // split-K partial: O * v_scale, m (log2 units) and l; a row that saw
        // no key of the split gives (0, -inf, 0) and adds nothing in the merge
        if (r.valid) {
            const size_t slot = ((size_t)r.split * a.total_q + r.q_row) * a.hq + r.head;
            float* dst = a.part_o + slot * D;
            const float vs = a.v_scale;
#pragma unroll
            for (int db = 0; db < (D / 32); ++db) {
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const int d0 = 32 * db + 8 * q4 + 4 * h;
                    *(f32x4*)(dst + d0) = f32x4{o[db][4 * q4], o[db][4 * q4 + 1],
                                                o[db][4 * q4 + 2], o[db][4 * q4 + 3]} * vs;
                }
            }
            if (h == 0) {
                a.part_ml[2 * slot] = l_tot > 0.f ? m_ref : -__builtin_inff();
                a.part_ml[2 * slot + 1] = l_tot;
            }
        }
        return;
    }
    // o = O / l, correctly rounded (not O * (1/l)), as the definition reads:
    // with V = 1 it returns exactly 1.  Every value of the lane shares l, so
    // one IEEE division gives r = RN(1 / l), and per value q = RN(O r) is
    // within an ulp of O / l; the remainder O - q l is exact as one fma, and
    // q + (O - q l) r rounded once is then RN(O / l) (Markstein's correction
    // step for a correctly rounded reciprocal): three VALU operations per
    // value instead of a division's ten.
    const float vs = a.v_scale;   // 1 for a bf16 pool
    // A sink (vLLM flash-attention PR 199, second review, finding F4) adds
    // 2^(sink - m_ref) to the denominator in the units of l (log2 units,
    // relative to the row's reference maximum); 0 without one, so that the
    // division below is then exactly O / l.
    const float sink2 = a.sinks ? a.sinks[r.head] * 1.4426950408889634f : -__builtin_inff();
    float lse2 = -__builtin_inff();   // log2-sum-exp of the row
    if (!any_tile) {  // no tile with a visible key (empty cache): the output is 0
        l_tot = 1.f;
        lse2 = sink2;
#pragma unroll
        for (int db = 0; db < (D / 32); ++db) o[db] = f32x16{};
    } else if (l_tot == 0.f) {  // this row saw no key (its band is past the cache end)
        l_tot = 1.f;            // O is 0
        lse2 = sink2;
    } else {
        const float a2 = m_ref + __builtin_log2f(l_tot);
        const float top = fmaxf(a2, sink2);
        lse2 = top + __builtin_log2f(fast_exp2(a2 - top) + fast_exp2(sink2 - top));
        l_tot += fast_exp2(sink2 - m_ref);
    }
    if (a.lse && r.valid && h == 0)
        a.lse[(size_t)r.q_row * a.hq + r.head] = lse2 * 0.6931471805599453f;
    // bf16 output through LDS: a lane holds 4-dim pieces of its row spread
    // over the row, so storing them directly puts 16-byte pieces of 32 rows
    // in every store instruction.  Each wave instead writes its 32 rows into
    // its own part of the (then free) tile buffers and stores them back one
    // whole row per instruction.  16-byte chunk c of a staged row r sits at
    // chunk c ^ (r & 15), so the 16 rows one write instruction covers fall in
    // distinct bank groups.
    const float r_l = 1.f / l_tot;
    auto quot = [&](float x) {
        const float q = x * r_l;
        return __builtin_fmaf(__builtin_fmaf(-q, l_tot, x), r_l, q);
    };
    constexpr int kOutRowB = D * 2;
    if constexpr (STAGE) {
        wait_vmcnt<0>();     // every wave's refills have landed ...
        race_delay<2>();
        __syncthreads();     // ... and no wave reads the tiles any more
        ATTN_LDS char* stage = smem + wave * 32 * kOutRowB;
#pragma unroll
        for (int db = 0; db < (D / 32); ++db) {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                f32x4 v = {quot(o[db][4 * q4]), quot(o[db][4 * q4 + 1]),
                           quot(o[db][4 * q4 + 2]), quot(o[db][4 * q4 + 3])};
                if constexpr (SCALE_V) v *= vs;
                const bf16x4 w = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
                const int c = 4 * db + q4;   // dims 32 db + 8 q4 .. + 7; this lane's half: 4 h
                *(ATTN_LDS bf16x4*)(stage + n * kOutRowB + ((c ^ (n & 15)) << 4) + 8 * h) = w;
            }
        }
        // lane l moves chunk l % (kOutRowB / 16) of staged row
        // 64 i / (kOutRowB / 16) + l / (kOutRowB / 16)
        constexpr int kChunks = kOutRowB / 16;
        constexpr int kRowsPerStore = 64 / kChunks;
        const int cl = lane % kChunks;
#pragma unroll 4
        for (int i = 0; i < 32 / kRowsPerStore; ++i) {
            const int rr = i * kRowsPerStore + lane / kChunks;   // staged row
            const int pr = wave * 32 + rr;                       // packed row of the workgroup
            const int trr = pr / a.g;
            const bf16x8 x = *(const ATTN_LDS bf16x8*)(stage + rr * kOutRowB + ((cl ^ (rr & 15)) << 4));
            if (trr < a.tok_per_wg && r.t0 + trr <= r.t_last) {
                const size_t ob = ((size_t)(r.q0 + r.t0 + trr) * a.hq + r.kvh * a.g + (pr - trr * a.g)) * D;
                *(bf16x8*)((__bf16*)a.out + ob + 8 * cl) = x;
            }
        }
        return;
    }
    if (r.valid) {
        const size_t obase = ((size_t)r.q_row * a.hq + r.head) * D;
#pragma unroll
        for (int db = 0; db < (D / 32); ++db) {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int d0 = 32 * db + 8 * q4 + 4 * h;
                f32x4 v = {quot(o[db][4 * q4]), quot(o[db][4 * q4 + 1]),
                           quot(o[db][4 * q4 + 2]), quot(o[db][4 * q4 + 3])};
                if constexpr (SCALE_V) v *= vs;
                if constexpr (OUT_FP32) {
                    *(f32x4*)((float*)a.out + obase + d0) = v;
                } else {
                    bf16x4 w = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
                    *(bf16x4*)((__bf16*)a.out + obase + d0) = w;
                }
            }
        }
    }
}

// The FP8-MFMA prefill over `grid` workgroups of 256 threads, with the
// work-unit numbering of the other prefill kernel: one pass per workgroup
// writing out (and lse), or with `split` one key range per workgroup writing
// the split-K partials (a.part_o, a.part_ml) for prefill_merge_kernel.
// Enqueues only (launch errors surface through hipGetLastError).
void launch_prefill_fp8mma(const PrefillArgs& a, bool out_fp32, bool split, unsigned grid,
                           hipStream_t stream);

}  // namespace attn
