// Pieces shared by the prefill kernels' translation units: the bf16 /
// widened-FP8 kernel (prefill_hd512.hip) and the block-scaled FP8 MFMA kernel
// (prefill_fp8mma.hip).  Both take one workgroup of 4 waves per 128 packed
// query rows and keep the same online-softmax bookkeeping (a fixed per-row
// reference maximum with a bounded restart).  The host validates every
// argument in prefill_launch before a launch.
#pragma once

#include "attn_host.h"
#include "device_common.h"

namespace attn {

constexpr int kRowsPerWg = 128;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
// Largest allowed excess (log2 units) of a row's scores over its reference
// maximum: p <= 2^32 and l <= 2^32 * keys stay far inside fp32 and bf16.
constexpr float kRescaleMargin = 32.f;
constexpr float kOverSum = 4294967296.f;   // 2^kRescaleMargin
constexpr float kBlindRaise = 123.f;       // log2(FLT_MAX / 32), rounded down
// Page ids of the first kPagesInLds tiles are staged in LDS at the start of
// the workgroup (reading them from the scalar cache inside the loop stalls
// the wave: scalar loads share the LDS wait counter and return out of order).
constexpr int kPagesInLds = 4096;
// Restarts per workgroup are capped so that non-finite inputs (a caller error)
// cannot loop forever; each genuine restart raises a row's reference by > 32.
constexpr int kMaxRestarts = 8;

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
};

// The FP8-MFMA prefill over `grid` workgroups of 256 threads, with the
// work-unit numbering of the other prefill kernel: one pass per workgroup
// writing out (and lse), or with `split` one key range per workgroup writing
// the split-K partials (a.part_o, a.part_ml) for prefill_merge_kernel.
// Enqueues only (launch errors surface through hipGetLastError).
void launch_prefill_fp8mma(const PrefillArgs& a, bool out_fp32, bool split, unsigned grid,
                           hipStream_t stream);

}  // namespace attn
