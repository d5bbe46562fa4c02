/*
 * attn_hd512 -- head-dim-512 causal GQA/MQA attention over a paged KV cache
 * for AMD MI355X (gfx950).  C ABI of libattn_hd512.so.
 *
 * Two operations, both FlashAttention forwards whose online softmax never
 * writes the [query x attended key] score matrix to device memory (Writing a
 * FlashAttention Prefill Kernel for Gemma 4, intro and "The starting point"):
 *   - attn_prefill_hd512: chunked causal prefill, one call per chunk; a chunk
 *     attends to every key before it in the cache (pegainfer issue 1051,
 *     "Description"); attn_prefill_hd512_e4m3 is the same over an FP8-E4M3
 *     cache;
 *   - attn_decode_splitk: Flash-Decoding for one query token per sequence:
 *     the key range is split across workgroups, each writes an unnormalised
 *     (O, m, l) partial, and a merge kernel combines them (Flash-Decoding for
 *     MQA in CUDA, "One KV head breaks the textbook").
 * Around them: _ex forms with sinks, a log-sum-exp output and multi-token
 * decode; split-K prefill for short chunks over long prefixes; the paged KV
 * append, alone or fused into the prefill launch; sliding-window (local)
 * layers at head dim 256 over ring caches (attn_prefill_swa); a measurement
 * helper (the HBM read probe).
 *
 * Common conventions
 *   Pointers are device pointers unless stated otherwise; the caller owns and
 *   frees every buffer.  Calls only enqueue work on `stream` and never
 *   synchronise; the library allocates nothing and keeps no per-call state.
 *   Shapes, counts and pointers are checked on the host before any launch;
 *   a failed check returns a non-zero attn_status_t and launches nothing.
 *   Device-resident data (page ids, lengths, offsets) is NOT validated,
 *   because that would need a device synchronisation (vLLM flash-attention
 *   PR 199, review finding F2 makes the same choice); it is clamped inside
 *   the kernels so that bad values cannot read outside the buffers, but the
 *   results are then undefined.
 *
 *   head_dim must be 512 (256 is accepted by attn_prefill_swa only) and
 *   page_size 64.  num_q_heads must be a multiple
 *   of num_kv_heads, with group g = num_q_heads / num_kv_heads <= 128; query
 *   head h uses KV head h / g (consecutive grouping, so that [B, 1, Hq*D] and
 *   [B*Hkv, g, D] are one layout: Flash-Decoding for MQA in CUDA, "One KV head
 *   breaks the textbook").
 *
 *   Page pools: [num_pages][num_kv_heads][64][512], row-major.  One (page, KV
 *   head) is one contiguous 64-key tile, the pool being paged at the key-tile
 *   size (pegainfer issue 1051, "Proposed Plan").  Logical key j of sequence b
 *   is slot j % 64 of page page_table[b * max_pages_per_seq + j / 64].  Only
 *   keys j < kv_lens[b] are ever read: page slots and table entries past the
 *   live band may hold anything, NaN included, without affecting results
 *   (pegainfer issue 1051, "Acceptance Criteria"; Flash-Decoding for MQA in
 *   CUDA, "The test that catches what parity misses").  Inside the live band
 *   a NaN key row makes exactly the rows that attend to it NaN; a NaN or
 *   infinite value row does the same and may also reach rows that share its
 *   64-key tile without attending to it (masked keys enter P.V with p = 0,
 *   and 0 x NaN is NaN).
 */
#ifndef ATTN_HD512_H
#define ATTN_HD512_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ATTN_BF16 = 0,      /* bfloat16 */
    ATTN_FP32 = 1,      /* IEEE binary32 */
    ATTN_FP8_E4M3 = 2   /* OCP 8-bit E4M3FN (no infinities, max 448) */
} attn_dtype_t;

typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_NULL = 1,         /* a required pointer is NULL */
    ATTN_ERR_SHAPE = 2,        /* a count or size is out of range or inconsistent */
    ATTN_ERR_UNSUPPORTED = 3,  /* valid request outside the supported set (dtype, head_dim, ...) */
    ATTN_ERR_WORKSPACE = 4,    /* decode workspace missing or too small */
    ATTN_ERR_HIP = 5           /* the HIP runtime reported an error at launch */
} attn_status_t;

/*
 * Chunked causal prefill.
 *
 *   q            bf16 [total_q][num_q_heads][512]; rows cu_seqlens_q[b] ..
 *                cu_seqlens_q[b+1]-1 are sequence b's query rows, in order.
 *   k_pages,
 *   v_pages      bf16 page pools (layout above).
 *   page_table   int32 [batch][max_pages_per_seq].
 *   cu_seqlens_q int32 [batch + 1], cu_seqlens_q[0] = 0, non-decreasing,
 *                cu_seqlens_q[batch] = total_q.
 *   q_start_pos  int32 [batch]: absolute position of sequence b's first
 *                query row (the chunk offset).
 *   kv_lens      int32 [batch]: keys in the cache for sequence b, this chunk
 *                included.  Precondition: q_start_pos[b] + q_len_b <= kv_lens[b]
 *                <= 64 * max_pages_per_seq.
 *   out          [total_q][num_q_heads][512] of out_dtype (ATTN_BF16, rounded
 *                to nearest even, or ATTN_FP32).  Only rows < total_q are
 *                written.
 *
 * Query row i of sequence b sits at position p = q_start_pos[b] + i and sees
 * keys j <= p (bottom-right causal alignment).  Its output is
 * softmax(scale * q K^T) V over those keys, computed with fp32 statistics and
 * accumulators from bf16 products.  max_q_len is an upper bound of the
 * per-sequence query counts and sets the grid; sequences with q_len = 0 are
 * allowed and write nothing.
 */
int attn_prefill_hd512(const void* q, const void* k_pages, const void* v_pages,
                       const int32_t* page_table, const int32_t* cu_seqlens_q,
                       const int32_t* q_start_pos, const int32_t* kv_lens, int batch,
                       int total_q, int max_q_len, int num_q_heads, int num_kv_heads,
                       int head_dim, int page_size, int num_pages, int max_pages_per_seq,
                       float softmax_scale, void* out, int out_dtype, hipStream_t stream);

/*
 * Chunked causal prefill over an FP8-E4M3 KV cache (OCP E4M3, the "fn"
 * variant: max 448, no infinities).  Same arguments and semantics as
 * attn_prefill_hd512, except:
 *
 *   k_pages,
 *   v_pages      E4M3 byte pools [num_pages][num_kv_heads][64][512] whose real
 *                values are byte * k_scale (keys) and byte * v_scale (values).
 *   k_scale,
 *   v_scale      per-tensor fp32 dequantisation scales, both > 0
 *                (ATTN_ERR_SHAPE otherwise).
 *
 * The bytes are widened exactly to bf16 inside the kernel (every E4M3 value
 * is a bf16 value); products and the softmax run as in the bf16 path, k_scale
 * folded into the softmax scale and v_scale applied to the output (vLLM
 * flash-attention PR 199, "Summary": FP8 KV with 16-bit MMA; P accumulated in
 * fp32 per key block as in commit 3 of the first review).
 */
int attn_prefill_hd512_e4m3(const void* q, const void* k_pages, const void* v_pages,
                            float k_scale, float v_scale, const int32_t* page_table,
                            const int32_t* cu_seqlens_q, const int32_t* q_start_pos,
                            const int32_t* kv_lens, int batch, int total_q, int max_q_len,
                            int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                            int num_pages, int max_pages_per_seq, float softmax_scale,
                            void* out, int out_dtype, hipStream_t stream);

/*
 * Chunked causal prefill with every option: a bf16 or FP8-E4M3 pool
 * (kv_dtype ATTN_BF16 or ATTN_FP8_E4M3; the scales are used for FP8 only),
 * attention sinks and a log-sum-exp output.  Other arguments as for
 * attn_prefill_hd512.
 *
 *   sinks        fp32 [num_q_heads] or NULL: one logit per query head, an
 *                extra softmax term with no value row, in the units of
 *                softmax_scale * q.k (natural log).  o = sum_j e^{S_j} V_j /
 *                (e^{sink} + sum_j e^{S_j}).
 *   lse          fp32 [total_q][num_q_heads] or NULL: log(e^{sink} +
 *                sum_j e^{S_j}) (natural log) of every written row.  A row
 *                with no visible key gets the sink logit, or -inf without a
 *                sink (vLLM flash-attention PR 199, second review, finding F4).
 */
int attn_prefill_hd512_ex(const void* q, const void* k_pages, const void* v_pages, int kv_dtype,
                          float k_scale, float v_scale, const int32_t* page_table,
                          const int32_t* cu_seqlens_q, const int32_t* q_start_pos,
                          const int32_t* kv_lens, int batch, int total_q, int max_q_len,
                          int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                          int num_pages, int max_pages_per_seq, float softmax_scale,
                          const float* sinks, void* out, int out_dtype, float* lse,
                          hipStream_t stream);

/*
 * Chunked causal prefill over an FP8-E4M3 KV cache with both products on the
 * gfx950 block-scaled FP8 matrix core (the FP8-MMA form of vLLM
 * flash-attention PR 199, "Summary": FP8 KV and FP8 QK/PV MMA).  Arguments,
 * semantics and results as attn_prefill_hd512_ex with kv_dtype
 * ATTN_FP8_E4M3, up to the rounding of the two operands that are not E4M3
 * already:
 *
 *   Q            each 32 consecutive head dims of a row are scaled by a power
 *                of two (from their largest magnitude) and split into two
 *                E4M3 terms, a high part and a residual x 32 (second review,
 *                commit 4 and finding F1), about 8 significant bits; any
 *                finite bf16 Q is in range (finding F2's |q| <= 448 limit of
 *                a fixed scale does not apply).
 *   P            the softmax weights of each 32-key block of a row are scaled
 *                by a power of two from the block's largest weight and split
 *                the same way; weights below about 2^-21 of that maximum lose
 *                relative precision (finding F1).
 *
 * Products accumulate in fp32 (O over the whole key range).  head_dim 512
 * only; ATTN_ERR_UNSUPPORTED otherwise.  Other errors as for
 * attn_prefill_hd512_e4m3.
 */
int attn_prefill_hd512_e4m3_mma(const void* q, const void* k_pages, const void* v_pages,
                                float k_scale, float v_scale, const int32_t* page_table,
                                const int32_t* cu_seqlens_q, const int32_t* q_start_pos,
                                const int32_t* kv_lens, int batch, int total_q, int max_q_len,
                                int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                                int num_pages, int max_pages_per_seq, float softmax_scale,
                                const float* sinks, void* out, int out_dtype, float* lse,
                                hipStream_t stream);

/*
 * attn_prefill_hd512_ex with persistent, heaviest-first scheduling (A custom
 * attention kernel for Gemma 4 on the RTX PRO 6000, "The kernel in three
 * steps", step 3): one workgroup per compute unit of the stream's device,
 * each taking work units (128 packed query rows of one KV head) from a
 * counter in `workspace`, heaviest units first, until none is left.  Every
 * unit computes exactly what the one-workgroup-per-unit launch of
 * attn_prefill_hd512_ex computes, so the results are bitwise the same.
 *
 *   kv_dtype     ATTN_BF16 or ATTN_FP8_E4M3 (widened to bf16, as in
 *                attn_prefill_hd512_e4m3); other arguments as for
 *                attn_prefill_hd512_ex.
 *   workspace    device buffer of at least
 *                attn_prefill_hd512_persistent_workspace_size() bytes; the
 *                call resets its counter itself (a one-thread kernel ahead of
 *                the prefill on `stream`, no memset), so its contents on
 *                entry are ignored; calls that overlap must not share it.
 *
 * ATTN_ERR_NULL for a missing workspace, ATTN_ERR_WORKSPACE when it is too
 * small, ATTN_ERR_HIP when the device's compute-unit count cannot be read.
 */
size_t attn_prefill_hd512_persistent_workspace_size(void);

int attn_prefill_hd512_persistent(const void* q, const void* k_pages, const void* v_pages,
                                  int kv_dtype, float k_scale, float v_scale,
                                  const int32_t* page_table, const int32_t* cu_seqlens_q,
                                  const int32_t* q_start_pos, const int32_t* kv_lens, int batch,
                                  int total_q, int max_q_len, int num_q_heads, int num_kv_heads,
                                  int head_dim, int page_size, int num_pages,
                                  int max_pages_per_seq, float softmax_scale, const float* sinks,
                                  void* workspace, size_t workspace_bytes, void* out,
                                  int out_dtype, float* lse, hipStream_t stream);

/*
 * Chunked causal prefill of a sliding-window (local) layer over a bf16 pool,
 * at head_dim 256 (the local layers' heads; A custom attention kernel for
 * Gemma 4 on the RTX PRO 6000, "The deployment": local layers attend to the
 * last 1,024 tokens with 256-dimensional heads) or 512.  Arguments as for
 * attn_prefill_hd512, with pools [num_pages][num_kv_heads][64][head_dim] and
 * q / out [total_q][num_q_heads][head_dim], plus:
 *
 *   window       >= 0: a row at absolute position p sees keys
 *                max(0, p - window + 1) <= j <= p (and j < kv_lens[b]); 0 means
 *                no window.
 *   ring_pages   >= 0, <= max_pages_per_seq: 0 for a cache indexed by
 *                position; otherwise (window > 0 required) the sequence's
 *                cache is a ring of
 *                C = 64 ring_pages slots and key j is read from slot j % C,
 *                i.e. page page_table[b][(j % C) / 64] (Flash-Decoding for MQA
 *                in CUDA, "One KV head breaks the textbook": slot = position %
 *                capacity, only the live band is read).  The caller keeps the
 *                band every row needs resident: C >= q_len + window - 1 for a
 *                chunk, C >= window for one token.
 *
 * ATTN_ERR_UNSUPPORTED for head_dim other than 256 or 512 or page_size other
 * than 64; ATTN_ERR_SHAPE for a negative window or ring size, a ring longer
 * than the table, or a ring without a window.  Decode is the case q_len = 1.
 */
int attn_prefill_swa(const void* q, const void* k_pages, const void* v_pages,
                     const int32_t* page_table, const int32_t* cu_seqlens_q,
                     const int32_t* q_start_pos, const int32_t* kv_lens, int batch, int total_q,
                     int max_q_len, int num_q_heads, int num_kv_heads, int head_dim,
                     int page_size, int num_pages, int max_pages_per_seq, int window,
                     int ring_pages, float softmax_scale, void* out, int out_dtype,
                     hipStream_t stream);

/*
 * Bytes of device workspace attn_prefill_hd512_splitk needs for these sizes:
 * fp32 partial outputs plus (m, l) per split, query row and query head.
 * Returns 0 when the plan has a single key range (the call then runs the
 * single-pass kernel and needs no workspace) and for invalid sizes.
 */
size_t attn_prefill_hd512_splitk_workspace_size(int batch, int max_q_len, int total_q,
                                                int num_q_heads, int num_kv_heads,
                                                int max_kv_len, int keys_per_split);

/*
 * Chunked causal prefill with the key range split across workgroups, for
 * short chunks over long prefixes, where one workgroup per block of query
 * rows would leave most compute units idle while each walks the whole
 * prefix (vLLM flash-attention PR 199, second review: vLLM's call shapes
 * include prefix prefill and explicit split counts; the partials combine as
 * in split-K decode).  Arguments as for attn_prefill_hd512_ex, plus:
 *
 *   max_kv_len       host bound on kv_lens[b], 1 <= max_kv_len <=
 *                    max_pages_per_seq * 64; keys past the last split of
 *                    the plan (nsplit * keys_per_split >= max_kv_len) are
 *                    not read.
 *   keys_per_split   keys per range, a positive multiple of 64, or 0 for the
 *                    library default: the range count (at most 64, ranges of
 *                    at least 512 keys) that keeps the 256 compute units
 *                    busiest, each range charged 2% for its partials.
 *   workspace        device buffer of at least
 *                    attn_prefill_hd512_splitk_workspace_size(...) bytes
 *                    (may be NULL when that is 0); contents on entry are
 *                    ignored; not to be shared by concurrent calls.
 *
 * The split kernel writes, for every (query row, query head, range) whose
 * range holds at least one key the row sees, O * v_scale, m and l of that
 * range; the merge kernel combines a row's ranges (the count follows from
 * q_start_pos, kv_lens and the row's position) with the sink, divides, and
 * writes out (and lse).  Results equal attn_prefill_hd512_ex's up to
 * rounding order.
 */
int attn_prefill_hd512_splitk(const void* q, const void* k_pages, const void* v_pages,
                              int kv_dtype, float k_scale, float v_scale,
                              const int32_t* page_table, const int32_t* cu_seqlens_q,
                              const int32_t* q_start_pos, const int32_t* kv_lens, int batch,
                              int total_q, int max_q_len, int num_q_heads, int num_kv_heads,
                              int head_dim, int page_size, int num_pages,
                              int max_pages_per_seq, int max_kv_len, int keys_per_split,
                              float softmax_scale, const float* sinks, void* workspace,
                              size_t workspace_bytes, void* out, int out_dtype, float* lse,
                              hipStream_t stream);

/*
 * attn_prefill_hd512_splitk over an FP8-E4M3 pool with both products on the
 * block-scaled FP8 matrix core: each key range runs the kernel of
 * attn_prefill_hd512_e4m3_mma (same operand rounding), the merge is the same.
 * Arguments as attn_prefill_hd512_splitk without kv_dtype (the pools are
 * E4M3); workspace size from attn_prefill_hd512_splitk_workspace_size.
 */
int attn_prefill_hd512_splitk_e4m3_mma(const void* q, const void* k_pages, const void* v_pages,
                                       float k_scale, float v_scale, const int32_t* page_table,
                                       const int32_t* cu_seqlens_q, const int32_t* q_start_pos,
                                       const int32_t* kv_lens, int batch, int total_q,
                                       int max_q_len, int num_q_heads, int num_kv_heads,
                                       int head_dim, int page_size, int num_pages,
                                       int max_pages_per_seq, int max_kv_len, int keys_per_split,
                                       float softmax_scale, const float* sinks, void* workspace,
                                       size_t workspace_bytes, void* out, int out_dtype,
                                       float* lse, hipStream_t stream);

/*
 * Bytes of device workspace attn_decode_splitk needs for these sizes: fp32
 * partial outputs plus (m, l) for up to 4 partials per split, per query head
 * and sequence (valid for either KV dtype).  keys_per_split = 0 selects the
 * library default: batch * num_kv_heads * max_kv_len keys over about 4096
 * ranges (2048 when a split carries two or three 16-column blocks of a
 * multi-token decode), rounded up to a multiple of 64 and at least 256.
 * Returns 0 for invalid sizes.
 */
size_t attn_decode_splitk_workspace_size(int batch, int num_q_heads, int num_kv_heads,
                                         int max_kv_len, int keys_per_split);

/*
 * Split-K decode: one query token per sequence at position kv_lens[b] - 1.
 *
 *   q            bf16 [batch][num_q_heads][512].
 *   k_pages,
 *   v_pages      page pools of kv_dtype: ATTN_BF16, or ATTN_FP8_E4M3 bytes
 *                whose real values are byte * k_scale (keys) and
 *                byte * v_scale (values), per-tensor fp32 scales.  FP8 values
 *                are widened exactly to bf16 inside the kernel and every
 *                product is accumulated in fp32 per key block (vLLM
 *                flash-attention PR 199, commit 3 of the first review).
 *   page_table, kv_lens   as for prefill; 1 <= kv_lens[b] <= max_kv_len.
 *   keys_per_split        keys per partial, a positive multiple of 64, or 0
 *                for the library default.
 *   workspace    device buffer of at least
 *                attn_decode_splitk_workspace_size(...) bytes; contents on
 *                entry are ignored; it must not be shared by concurrent calls.
 *   out          [batch][num_q_heads][512] of out_dtype (ATTN_BF16 or ATTN_FP32).
 *
 * Two kernels run back to back on `stream`: the split kernel writes the
 * partials of every (sequence, KV head, split) for every query head of the
 * group (one per split for a bf16 pool, one per wave of the split workgroup
 * for an FP8 pool), and the merge kernel combines them.  Splits that start
 * at or past a sequence's kv_len are neither written nor read: the merge
 * derives each sequence's split count from kv_lens.  A partial that saw no
 * key (m = -inf, l = 0, O = 0) contributes nothing.
 */
int attn_decode_splitk(const void* q, const void* k_pages, const void* v_pages, int kv_dtype,
                       float k_scale, float v_scale, const int32_t* page_table,
                       const int32_t* kv_lens, int batch, int num_q_heads, int num_kv_heads,
                       int head_dim, int page_size, int num_pages, int max_pages_per_seq,
                       int max_kv_len, int keys_per_split, float softmax_scale,
                       void* workspace, size_t workspace_bytes, void* out, int out_dtype,
                       hipStream_t stream);

/*
 * Split-K decode with every option: q_len query tokens per sequence
 * (multi-token decode, e.g. verifying q_len - 1 draft tokens; vLLM
 * flash-attention PR 199, second review: "MTP decode"; A custom attention
 * kernel for Gemma 4 on the RTX PRO 6000, "The deployment": a 4-token draft
 * at 32 query heads over 4 KV heads), attention sinks and a log-sum-exp
 * output.  Other arguments as for attn_decode_splitk.
 *
 *   q            bf16 [batch * q_len][num_q_heads][512]: token t of sequence
 *                b is row b * q_len + t, at position kv_lens[b] - q_len + t,
 *                and sees keys j <= that position.  q_len >= 1;
 *                kv_lens[b] >= q_len is a precondition.
 *   sinks, lse   as for attn_prefill_hd512_ex; lse is [batch * q_len][num_q_heads].
 *   out          [batch * q_len][num_q_heads][512].
 *   workspace    at least attn_decode_splitk_ex_workspace_size(...) bytes.
 *
 * Up to 48 (token, query head) columns per KV head (q_len * g <= 48, e.g.
 * 5 tokens at g = 8) run on the decode kernels, in blocks of 16 columns that
 * share each K and V tile read.  Wider calls are the prefill of q_len rows
 * per sequence at positions kv_lens[b] - q_len ..: they run as
 * attn_prefill_hd512_splitk on the same pool (keys_per_split, else the decode
 * default, sets that call's ranges), after a one-workgroup kernel has
 * written its row offsets and chunk starts to the head of the workspace; the
 * workspace size covers both.
 */
size_t attn_decode_splitk_ex_workspace_size(int batch, int q_len, int num_q_heads,
                                            int num_kv_heads, int max_kv_len,
                                            int keys_per_split);

int attn_decode_splitk_ex(const void* q, const void* k_pages, const void* v_pages, int kv_dtype,
                          float k_scale, float v_scale, const int32_t* page_table,
                          const int32_t* kv_lens, int batch, int q_len, int num_q_heads,
                          int num_kv_heads, int head_dim, int page_size, int num_pages,
                          int max_pages_per_seq, int max_kv_len, int keys_per_split,
                          float softmax_scale, const float* sinks, void* workspace,
                          size_t workspace_bytes, void* out, int out_dtype, float* lse,
                          hipStream_t stream);

/*
 * attn_decode_splitk_ex for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  Arguments and results as attn_decode_splitk_ex, without the
 * workspace: the split kernel's partials go to a static device array of the
 * library (64 MiB per GPU, held until the process ends), whose address is
 * looked up once per device on the first call that runs on it (the device
 * of `stream`; the current device for the null stream).  The call allocates
 * nothing and enqueues the same two kernels.
 *
 * ATTN_ERR_WORKSPACE when the plan's partials, batch * q_len * num_q_heads *
 * ceil(max_kv_len / keys_per_split) * 2056 bytes (keys_per_split after the
 * default is applied), exceed 64 MiB; ATTN_ERR_HIP when the address lookup
 * fails.  The scratch needs no clearing (every partial the merge reads is
 * written by the same call), but it is one array per GPU shared by every
 * call: calls that overlap on one GPU (concurrent streams, or threads) race
 * and give undefined results.
 */
int attn_decode_splitk_ex_noalloc(const void* q, const void* k_pages, const void* v_pages,
                                  int kv_dtype, float k_scale, float v_scale,
                                  const int32_t* page_table, const int32_t* kv_lens, int batch,
                                  int q_len, int num_q_heads, int num_kv_heads, int head_dim,
                                  int page_size, int num_pages, int max_pages_per_seq,
                                  int max_kv_len, int keys_per_split, float softmax_scale,
                                  const float* sinks, void* out, int out_dtype, float* lse,
                                  hipStream_t stream);

/*
 * Paged KV append: writes a chunk's new key and value rows into their cache
 * slots (one page per key tile of the attention kernels: pegainfer issue
 * 1051, "Proposed Plan").
 *
 *   k_new, v_new   bf16 [total_q][num_kv_heads][512]; row order as q.
 *   kv_dtype       ATTN_BF16 (rows copied) or ATTN_FP8_E4M3 (each element
 *                  stored as the E4M3FN code of x / scale (fp32 division),
 *                  saturated to +-448, rounded to nearest even; NaN stays NaN).
 *   page_table, cu_seqlens, q_start_pos   as for prefill: token i of sequence
 *                  b goes to position q_start_pos[b] + i, i.e. page
 *                  page_table[b][p / 64], slot p % 64.
 *   k_pages, v_pages   the pools written (layout above).
 *
 * Rows whose position falls outside the table, or whose page id falls
 * outside the pool, are skipped.  Rows must not share a slot (no two tokens
 * at one position of one sequence, no page shared by two sequences'
 * written slots); then the result does not depend on execution order.
 */
int attn_append_kv(const void* k_new, const void* v_new, int kv_dtype, float k_scale,
                   float v_scale, const int32_t* page_table, const int32_t* cu_seqlens,
                   const int32_t* q_start_pos, int batch, int total_q, int num_kv_heads,
                   int head_dim, int page_size, int num_pages, int max_pages_per_seq,
                   void* k_pages, void* v_pages, hipStream_t stream);

/*
 * Chunked causal prefill with the chunk's paged KV append fused into the same
 * launch, over a bf16 pool at head_dim 512: a page holds exactly one key
 * tile, so each tile is a single contiguous copy (pegainfer issue 1051,
 * "Proposed Plan"), and the rows a chunk appends are the keys it attends to
 * last.  Arguments as for attn_prefill_hd512_ex with kv_dtype ATTN_BF16,
 * plus:
 *
 *   k_new, v_new   bf16 [total_q][num_kv_heads][512], row order as q: the
 *                  chunk's new key and value rows, token i of sequence b at
 *                  position q_start_pos[b] + i.
 *   k_pages, v_pages   written as attn_append_kv(ATTN_BF16) writes them,
 *                  and read for the keys before the chunk.
 *
 * Keys at the chunk's own positions are read from k_new / v_new, so the
 * result and the pool afterwards are bitwise those of attn_append_kv followed
 * by attn_prefill_hd512_ex, provided every chunk position maps to a page of
 * the pool (a row whose page id falls outside it is skipped by both writes,
 * but the fused call still attends to its new row), q_start_pos[b] >= 0,
 * and no page slot the call writes is visible to another sequence of the
 * call (the writes are not ordered with the other workgroups' reads).  ATTN_ERR_NULL for a missing k_new or v_new;
 * ATTN_ERR_SHAPE when total_q * num_kv_heads * 1024 exceeds 2^32 - 1 bytes.
 */
int attn_prefill_hd512_append(const void* q, const void* k_new, const void* v_new,
                              void* k_pages, void* v_pages, const int32_t* page_table,
                              const int32_t* cu_seqlens_q, const int32_t* q_start_pos,
                              const int32_t* kv_lens, int batch, int total_q, int max_q_len,
                              int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                              int num_pages, int max_pages_per_seq, float softmax_scale,
                              const float* sinks, void* out, int out_dtype, float* lse,
                              hipStream_t stream);

/*
 * The same call for an FP8-E4M3 pool with both products on the FP8 matrix
 * core: the chunk's new rows are encoded into the pool as attn_append_kv
 * (ATTN_FP8_E4M3) encodes them, and the chunk attends to them as codes
 * (pegainfer issue 1051, "Proposed Plan"; vLLM flash-attention PR 199,
 * "Summary": FP8 paged KV with FP8 MMA).  Arguments as for
 * attn_prefill_hd512_append, plus k_scale and v_scale as for
 * attn_prefill_hd512_e4m3_mma; k_pages and v_pages are E4M3 pools.
 *
 * Runs as two launches on `stream`, the append kernel and then the FP8-MMA
 * prefill, so the output and the pool are bitwise those of attn_append_kv
 * followed by attn_prefill_hd512_e4m3_mma.  (Encoding the chunk's rows
 * inside the prefill would put the conversion on the refill path of a
 * kernel whose VALU issue already sets its pace, and reading them back as
 * codes would wait on other workgroups' writes; on this hardware even the
 * bf16 fused launch does not beat the two launches.)  Every argument of both
 * steps is checked before the first launch: a call that returns an error
 * leaves the pool untouched.  ATTN_ERR_NULL for a missing k_new or v_new.
 */
int attn_prefill_hd512_e4m3_mma_append(const void* q, const void* k_new, const void* v_new,
                                       void* k_pages, void* v_pages, float k_scale,
                                       float v_scale, const int32_t* page_table,
                                       const int32_t* cu_seqlens_q, const int32_t* q_start_pos,
                                       const int32_t* kv_lens, int batch, int total_q,
                                       int max_q_len, int num_q_heads, int num_kv_heads,
                                       int head_dim, int page_size, int num_pages,
                                       int max_pages_per_seq, float softmax_scale,
                                       const float* sinks, void* out, int out_dtype, float* lse,
                                       hipStream_t stream);

/*
 * Measurement helper: streams `bytes` (a multiple of 16) of device memory
 * once with 16-byte loads and writes one word per workgroup to `sink`
 * (at least attn_hbm_probe_sink_words(bytes) uint32 values).  Used to take
 * the same-process HBM read roofline that decode is reported against.
 */
int attn_hbm_read_probe(const void* buf, size_t bytes, void* sink, hipStream_t stream);
size_t attn_hbm_probe_sink_words(size_t bytes);

/*
 * Measurement helper: launches `slots` one-wave workgroups (1 <= slots <=
 * 65536) on `stream`; workgroup i writes three uint64 words to stamps[3 i ..]:
 * where it ran (the XCD id, 0..7, in bits 32..35 and the HW_ID hardware
 * register in bits 0..31: compute unit in bits 8..11, shader array in 12,
 * shader engine in 13..15), the shader-clock cycle counter (s_memtime, which
 * is not synchronised between compute units) and the constant 100 MHz
 * counter (s_memrealtime).  Two launches around a timed region give, for a
 * compute unit that holds a stamp of both, its mean shader clock over the
 * region: delta(cycles) / delta(100 MHz ticks) * 100 MHz.
 */
int attn_clock_stamps(void* stamps, int slots, hipStream_t stream);

/* Static text for a status code. */
const char* attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_HD512_H */
