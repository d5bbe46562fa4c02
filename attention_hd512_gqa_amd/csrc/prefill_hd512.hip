// Chunked causal GQA/MQA prefill at head_dim 512 over a paged bf16 KV cache,
// for gfx950 (MI355X).  One FlashAttention-style pass per workgroup: the score
// tile lives in registers only, with an online softmax in fp32 (Writing a
// FlashAttention Prefill Kernel for Gemma 4, "Head dim 512 breaks the
// textbook" and "The bug that passed every test").
//
// Work unit (one workgroup, 4 waves): 128 packed query rows of one KV head of
// one sequence.  Packed row r is token r / g and query head r % g of the
// group, so every K/V tile brought into LDS serves all g heads of the group
// (A custom attention kernel for Gemma 4 on the RTX PRO 6000, "The kernel in
// three steps", step 1).  Wave w owns packed rows 32w .. 32w+31 with the full
// 512-wide Q row in VGPRs and the full 512-wide O row in accumulators: a
// gfx950 wave has up to 512 registers, so the register ceiling that pushed
// the Ada and Blackwell kernels to split head_dim across warps does not bind
// here, and no score partials need exchanging between waves.
//
// Per 64-key tile (= one page of one KV head):
//   K and V arrive in two separate 64 KB LDS buffers (no time-sharing of one
//   buffer; pegainfer issue 1051, "Description") by direct global->LDS loads,
//   one coalesced 1 KB key row per wave instruction, XOR-swizzled per 16 bytes;
//   S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (fp32 accumulators), so that each
//   lane holds one query row's scores and softmax statistics;
//   masked keys get -inf (only tiles that cross a row's causal limit or the
//   cache length are masked; tiles past the last row's limit are never loaded);
//   softmax statistics in fp32 with exp2, per 64-key tile (Flash-Decoding for
//   MQA in CUDA, "One KV head breaks the textbook": statistics per tile, not
//   per key), against a per-row reference maximum (see the loop below for why
//   O is never rescaled in place);
//   P goes to bf16 and O^T += V^T P^T on the same MFMA, V^T read with the
//   gfx950 transposing LDS load.  O accumulates in fp32 across the whole key
//   range (vLLM flash-attention PR 199, commit 3 of the first review).
// K(j+1) streams in while softmax and P.V of tile j run; V(j+1) while Q.K^T of
// tile j+1 runs.
#include "device_common.h"
#include "attn_host.h"

namespace attn {

namespace {

constexpr int kRowsPerWg = 128;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWaveLoad = kPage / kWaves;  // tile rows each wave moves
// Largest allowed excess (log2 units) of a row's running maximum over its
// reference maximum: p <= 2^24, l <= 2^24 * keys, all well inside fp32/bf16.
constexpr float kRescaleMargin = 24.f;

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
    float scale_log2;   // softmax_scale * log2(e)
};

// Queue the 64 rows of one (page, KV head) tile into an LDS tile buffer.  Each
// wave moves 16 rows with exactly 16 vector-memory operations, which the
// callers' vmcnt arithmetic relies on.  The resource covers only the `valid`
// rows, so rows of keys past the cache length (whose slots may hold anything)
// arrive as zeros.
__device__ __forceinline__ void issue_tile(const char* pool, const int* ptab, int kt,
                                           int num_pages, int hkv, int kvh, int valid,
                                           ATTN_LDS char* buf, int wave, int lane16) {
    int page = load_uniform(ptab, kt);
    page = page < 0 ? 0 : (page >= num_pages ? num_pages - 1 : page);
    const char* src = pool + ((size_t)page * hkv + kvh) * (size_t)kTileBytes;
    const u32x4 rsrc = buffer_rsrc(src, (uint32_t)valid * kRowBytes);
#pragma unroll
    for (int i = 0; i < kRowsPerWaveLoad; ++i) {
        const int r = wave * kRowsPerWaveLoad + i;   // r % 16 == i, so swz(r) == swz(i)
        row_to_lds(rsrc, buf + r * kRowBytes, lane16 ^ (swz(i) << 4), r * kRowBytes);
    }
}

template <bool FIRST>
__device__ __forceinline__ void pv_tile(f32x16 (&o)[16], const bf16x8 (&pf)[4],
                                        const ATTN_LDS char* sV, int lane) {
    const int h = lane >> 5;
    const int grp = lane & 15;
    const int dsub = (lane >> 4) & 1;
    const int krow = 4 * h + (grp >> 2);               // + 16 c (+ 8)
    // 32-dim block db covers chunks 4 db .. 4 db + 3; this lane reads chunk
    // 4 db + cb at byte `within`.  The swizzle permutes chunks within aligned
    // groups of 16, so with db = 4 u + w the offset is voff[w] + 256 u.
    const int cb = 2 * dsub + ((grp & 3) >> 1);
    const int within = 8 * (grp & 1);
    int voffA[4], voffB[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        voffA[w] = krow * kRowBytes + (((4 * w + cb) ^ swz(krow)) << 4) + within;
        voffB[w] = (krow + 8) * kRowBytes + (((4 * w + cb) ^ swz(krow + 8)) << 4) + within;
    }
    auto vread = [&](int step) -> bf16x8 {
        const int c = step >> 4, db = step & 15;
        const int rel = 16 * c * kRowBytes + 256 * (db >> 2);  // swz(16c + k) == swz(k)
        const bf16x4 va = lds_read_tr16(sV + voffA[db & 3] + rel);
        const bf16x4 vb = lds_read_tr16(sV + voffB[db & 3] + rel);
        return __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    constexpr int kPrefetch = 4;
    bf16x8 vbuf[kPrefetch];
#pragma unroll
    for (int j = 0; j < kPrefetch; ++j) vbuf[j] = vread(j);
#pragma unroll
    for (int step = 0; step < 64; ++step) {
        const bf16x8 cur = vbuf[step % kPrefetch];
        if (step + kPrefetch < 64) vbuf[step % kPrefetch] = vread(step + kPrefetch);
        if (FIRST && step < 16)
            o[step] = mfma32x32x16(cur, pf[0], f32x16{});
        else
            o[step & 15] = mfma32x32x16(cur, pf[step >> 4], o[step & 15]);
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <bool OUT_FP32>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void prefill_hd512_kernel(PrefillArgs a) {
    __shared__ __attribute__((aligned(1024))) char smem[2 * kTileBytes];
    __shared__ int sFlag[kWaves];
    ATTN_LDS char* sK = (ATTN_LDS char*)smem;
    ATTN_LDS char* sV = sK + kTileBytes;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    // ---- work unit: heaviest query tiles first; KV head fastest so that
    // consecutive workgroups (spread round-robin over the XCDs) share a KV
    // head per XCD whenever the KV head count divides 8.
    const int per_rank = a.batch * a.hkv;
    const int rank = blockIdx.x / per_rank;
    const int rem = blockIdx.x - rank * per_rank;
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
    L = L < 0 ? 0 : (L > a.max_pages * kPage ? a.max_pages * kPage : L);
    const int qs = a.q_start[b];
    const int n_max = min(qs + t_last + 1, L);   // keys the last row sees
    const int n_min = min(qs + t0 + 1, L);       // keys the first row sees
    const int ntiles = n_max > 0 ? (n_max + kPage - 1) / kPage : 0;

    // ---- this lane's query row: n = column of the MFMA tiles, h = k-half
    const int n = lane & 31;
    const int h = lane >> 5;
    const int r = wave * 32 + n;
    const int tr = r / a.g;
    const bool valid = (tr < a.tok_per_wg) && (t0 + tr <= t_last);
    const int t = valid ? t0 + tr : t_last;      // padding rows shadow the last real token
    const int head = kvh * a.g + (valid ? r - tr * a.g : 0);
    const int n_row = min(qs + t + 1, L);

    // ---- Q^T operand: k-step ks covers head dims 16 ks .. 16 ks + 15; this
    // lane holds dims 16 ks + 8 h .. + 7 of its row.
    bf16x8 qf[32];
    {
        const bf16x8* qp =
            (const bf16x8*)(a.q + ((size_t)(q0 + t) * a.hq + head) * kHeadDim) + h;
#pragma unroll
        for (int ks = 0; ks < 32; ++ks) {
            bf16x8 v = qp[2 * ks];
            qf[ks] = valid ? v : bf16x8{};
        }
    }

    f32x16 o[16];  // written first by tile 0's P.V
    // Online softmax with a fixed per-row reference maximum: p = 2^(x - m_ref)
    // where m_ref is the row's maximum over the first tile.  O and l carry the
    // same factor 2^(m_true - m_ref), which cancels in O / l.  A row whose
    // maximum climbs more than kRescaleMargin above m_ref would push p past
    // 2^kRescaleMargin, so the workgroup then restarts its key loop with every
    // row's reference raised to the maximum seen so far: the rescale of O is
    // replaced by a recompute that typical inputs never trigger.  This keeps
    // the 256 O accumulators (AGPRs, which VALU cannot address) out of all
    // VALU code in the loop.
    float m_ref = -__builtin_inff();
    float m_seen = -__builtin_inff();
    float l_run = 0.f;

    const int* ptab = a.page_table + (size_t)b * a.max_pages;
    const int lane16 = lane * 16;
    int koff[8];
#pragma unroll
    for (int v = 0; v < 8; ++v) koff[v] = n * kRowBytes + (((2 * v + h) ^ swz(n)) << 4);
    if (ntiles > 0) {
        const int v0 = min(L, kPage);
        issue_tile(a.k_pages, ptab, 0, a.num_pages, a.hkv, kvh, v0, sK, wave, lane16);
        issue_tile(a.v_pages, ptab, 0, a.num_pages, a.hkv, kvh, v0, sV, wave, lane16);
    }

    for (int kt = 0; kt < ntiles; ++kt) {
        const bool more = kt + 1 < ntiles;
        const int key0 = kt * kPage;
        // K(kt) has landed when only V(kt)'s 16 loads may still be in flight
        wait_vmcnt<kRowsPerWaveLoad>();
        lds_barrier();

        // ---- S^T[key][row] = K Q^T for the tile's two 32-key blocks.  The K
        // operand of step j is read kPrefetch steps ahead of its MFMA; the
        // scheduling fences keep the compiler from hoisting more reads than that.
        f32x16 s[2];
        {
            // step = 32 kb + ks reads chunk 2 ks + h of key row 32 kb + n; the
            // swizzle permutes chunks within aligned groups of 16, so with
            // ks = 8 u + v the byte offset is koff[v] + 256 u + 32 KiB kb.
            auto kread = [&](int step) -> bf16x8 {
                const int kb = step >> 5, ks = step & 31;
                return *(const ATTN_LDS bf16x8*)(sK + koff[ks & 7] + 256 * (ks >> 3) +
                                                  kb * 32 * kRowBytes);
            };
            constexpr int kPrefetch = 4;
            bf16x8 kbuf[kPrefetch];
#pragma unroll
            for (int j = 0; j < kPrefetch; ++j) kbuf[j] = kread(j);
#pragma unroll
            for (int step = 0; step < 64; ++step) {
                const bf16x8 cur = kbuf[step % kPrefetch];
                if (step + kPrefetch < 64) kbuf[step % kPrefetch] = kread(step + kPrefetch);
                if ((step & 31) == 0)
                    mfma32x32x16_vgpr_first(s[step >> 5], cur, qf[0]);
                else
                    mfma32x32x16_vgpr(s[step >> 5], cur, qf[step & 31]);
                __builtin_amdgcn_sched_barrier(0);
            }
            mfma_vgpr_drain(s[0], s[1]);
        }

        // ---- scores in log2 units, masked; accumulator element i of block kb
        // holds key kb*32 + 8(i/4) + 4h + (i%4) of this tile for this lane's row.
        const bool mask = key0 + kPage > n_min;
        float mt = -__builtin_inff();
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float v = s[kb][i] * a.scale_log2;
                if (mask) {
                    const int key = key0 + kb * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
                    v = key < n_row ? v : -__builtin_inff();
                }
                s[kb][i] = v;
                mt = fmaxf(mt, v);
            }
        }
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        m_seen = fmaxf(m_seen, mt);
        if (kt == 0) m_ref = mt;   // every row sees key 0, so this is finite
        if (lane == 0) sFlag[wave] = __any(mt > m_ref + kRescaleMargin) ? 1 : 0;
        lds_barrier();  // every wave is done with sK; restart flags visible
        if (sFlag[0] | sFlag[1] | sFlag[2] | sFlag[3]) {
            // drain this wave's V(kt) loads before sV is refilled from key 0
            wait_vmcnt<0>();
            lds_barrier();
            m_ref = m_seen;
            l_run = 0.f;   // O restarts too: tile 0's P.V overwrites it
            const int v0 = min(L, kPage);
            issue_tile(a.k_pages, ptab, 0, a.num_pages, a.hkv, kvh, v0, sK, wave, lane16);
            issue_tile(a.v_pages, ptab, 0, a.num_pages, a.hkv, kvh, v0, sV, wave, lane16);
            kt = -1;
            continue;
        }
        if (more) {
            const int vn = min(L - (key0 + kPage), kPage);
            issue_tile(a.k_pages, ptab, kt + 1, a.num_pages, a.hkv, kvh, vn, sK, wave, lane16);
        }

        // ---- P = 2^(x - m_ref) in bf16 for the P.V MFMA; l in fp32
        float psum = 0.f;
        bf16x8 pf[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float p = fast_exp2(s[c >> 1][8 * (c & 1) + j] - m_ref);
                psum += p;
                pf[c][j] = (__bf16)p;
            }
        }
        l_run += psum;

        // V(kt) has landed when only K(kt+1)'s loads may still be in flight
        if (more) wait_vmcnt<kRowsPerWaveLoad>(); else wait_vmcnt<0>();
        lds_barrier();

        // ---- O^T[d][row] += V^T P^T (tile 0 of a pass starts O from zero).
        if (kt == 0)
            pv_tile<true>(o, pf, sV, lane);
        else
            pv_tile<false>(o, pf, sV, lane);
        lds_barrier();  // every wave is done with sV
        if (more) {
            const int vn = min(L - (key0 + kPage), kPage);
            issue_tile(a.v_pages, ptab, kt + 1, a.num_pages, a.hkv, kvh, vn, sV, wave, lane16);
        }
    }

    // ---- epilogue: lane holds d = 32 db + 8 (i/4) + 4 h + (i%4) of its row.
    // o = O / l with an IEEE division (not O * (1/l)), as the definition reads:
    // with V = 1 it returns exactly 1.
    float l_tot = l_run + __shfl_xor(l_run, 32);
    if (ntiles == 0) {  // no visible key (empty cache): the output row is 0
        l_tot = 1.f;
#pragma unroll
        for (int db = 0; db < 16; ++db) o[db] = f32x16{};
    }
    if (valid) {
        const size_t obase = ((size_t)(q0 + t) * a.hq + head) * kHeadDim;
#pragma unroll
        for (int db = 0; db < 16; ++db) {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int d0 = 32 * db + 8 * q4 + 4 * h;
                f32x4 v = {o[db][4 * q4] / l_tot, o[db][4 * q4 + 1] / l_tot,
                           o[db][4 * q4 + 2] / l_tot, o[db][4 * q4 + 3] / l_tot};
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

}  // namespace

}  // namespace attn

extern "C" int attn_prefill_hd512(const void* q, const void* k_pages, const void* v_pages,
                                  const int32_t* page_table, const int32_t* cu_seqlens_q,
                                  const int32_t* q_start_pos, const int32_t* kv_lens, int batch,
                                  int total_q, int max_q_len, int num_q_heads,
                                  int num_kv_heads, int head_dim, int page_size,
                                  int num_pages, int max_pages_per_seq, float softmax_scale,
                                  void* out, int out_dtype, hipStream_t stream) {
    using namespace attn;
    if (!q || !k_pages || !v_pages || !page_table || !cu_seqlens_q || !q_start_pos ||
        !kv_lens || !out)
        return ATTN_ERR_NULL;
    if (batch < 1 || total_q < 0 || max_q_len < 0 || num_q_heads < 1 || num_kv_heads < 1 ||
        num_pages < 1 || max_pages_per_seq < 1 || !(softmax_scale == softmax_scale))
        return ATTN_ERR_SHAPE;
    if (num_q_heads % num_kv_heads) return ATTN_ERR_SHAPE;
    if (head_dim != kHeadDim || page_size != kPage) return ATTN_ERR_UNSUPPORTED;
    const int g = num_q_heads / num_kv_heads;
    if (g > kRowsPerWg) return ATTN_ERR_UNSUPPORTED;
    if (out_dtype != ATTN_BF16 && out_dtype != ATTN_FP32) return ATTN_ERR_UNSUPPORTED;
    if ((long long)max_pages_per_seq * kPage > 0x7fffffffLL) return ATTN_ERR_SHAPE;
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
    a.scale_log2 = softmax_scale * 1.4426950408889634f;
    const long long grid = (long long)a.wgs_per_seq * batch * num_kv_heads;
    if (grid > 0x7fffffffLL) return ATTN_ERR_SHAPE;
    if (out_dtype == ATTN_FP32)
        hipLaunchKernelGGL(prefill_hd512_kernel<true>, dim3((unsigned)grid), dim3(kThreads), 0,
                           stream, a);
    else
        hipLaunchKernelGGL(prefill_hd512_kernel<false>, dim3((unsigned)grid), dim3(kThreads), 0,
                           stream, a);
    return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}
