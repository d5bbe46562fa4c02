// Split-K (Flash-Decoding) decode at head_dim 512 over a paged KV cache, for
// gfx950 (MI355X): one query token per sequence, GQA/MQA.
//
// A single KV head per sequence would give one workgroup per (sequence, KV
// head) and leave most CUs idle, so the key range is cut into splits of
// `keys_per_split` keys, each handled by one workgroup that writes an
// unnormalised partial (O, m, l) for every query head of the group; a merge
// kernel then combines the partials with the online-softmax rule (Flash-
// Decoding for MQA in CUDA, "One KV head breaks the textbook").  Only the live
// band [0, kv_len) is read (same page, "The starting point").
//
// Split workgroup (4 waves), per 64-key tile (= one page of one KV head):
//   K and V land in separate 64 KB LDS buffers, swizzled as in prefill.  The
//   bf16 pool goes global -> LDS directly; an FP8-E4M3 pool is loaded to
//   registers, widened exactly to bf16 and written to the same layout (vLLM
//   flash-attention PR 199, "Summary": FP8 KV with 16-bit MMA), with k_scale
//   folded into the softmax scale and v_scale into the partial output.
//   S^T = K Q^T on v_mfma_f32_16x16x32_bf16: the g query heads of the group
//   are the (zero-padded) 16 columns, wave w takes keys 16w .. 16w+15.  Scores
//   meet in a 4 KB LDS buffer; every wave then runs the softmax for all 64
//   keys (identical in each wave) and O^T += V^T P^T for its own 128 of the
//   512 output dims, in fp32 per key block (vLLM flash-attention PR 199,
//   commit 3 of the first review).
// Decode moves ~2 bytes per flop: HBM bandwidth, not the MFMA rate, bounds
// it; the padded MFMA rows cost issue slots that are free at that ratio.
#include "device_common.h"
#include "attn_host.h"

namespace attn {

namespace {

constexpr int kDecRows = 16;        // query heads of one group, zero-padded
constexpr int kDecWaves = 4;
constexpr int kDecThreads = 64 * kDecWaves;
constexpr int kRowsPerWaveLoad = kPage / kDecWaves;
constexpr int kSxStride = 272;      // bytes per score-exchange row (256 + 16 pad)
constexpr int kDefaultTargetWgs = 4096;

struct DecodeArgs {
    const __bf16* q;
    const char* k_pages;
    const char* v_pages;
    const int* page_table;
    const int* kv_lens;
    float* part_o;      // [batch][hkv][max_splits][g][512]
    float* part_ml;     // [batch][hkv][max_splits][g][2]  (m in log2 units, l)
    int batch, hq, hkv, g, max_pages, num_pages;
    int max_splits, tiles_per_split;
    float scale_log2;   // softmax_scale * log2(e) * k_scale
    float v_scale;
};

__device__ __forceinline__ const char* page_tile(const char* pool, const int* ptab, int tile,
                                                 int num_pages, int hkv, int kvh,
                                                 int tile_bytes) {
    int page = load_uniform(ptab, tile);
    page = page < 0 ? 0 : (page >= num_pages ? num_pages - 1 : page);
    return pool + ((size_t)page * hkv + kvh) * (size_t)tile_bytes;
}

// bf16 pool: 16 rows per wave, global -> LDS, rows past `valid` arrive as zeros.
__device__ __forceinline__ void issue_tile_bf16(const char* src, int valid, ATTN_LDS char* buf,
                                                int wave, int lane16) {
    rows16_to_lds(buffer_rsrc(src, (uint32_t)valid * kRowBytes), buf, wave, lane16);
}

// FP8 pool: a 64-key tile is 64 rows of 512 bytes.  Each wave loads 16 rows,
// two per instruction (lanes 0-31 row r, lanes 32-63 row r+1, 16 bytes each);
// rows past `valid` arrive as zeros.
struct Fp8Stage {
    u32x4 k[8];
    u32x4 v[8];
};

__device__ __forceinline__ void load_fp8(u32x4 (&dst)[8], const char* src, int valid, int wave,
                                         int lane) {
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(src), (short)0, valid * 512, 0x00020000);
    const int voff = (lane >> 5) * 512 + (lane & 31) * 16;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r = wave * kRowsPerWaveLoad + 2 * i;
        dst[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff, r * 512, 0));
    }
}

// Widen 16 E4M3 values (exact in bf16) and store them as two swizzled chunks.
__device__ __forceinline__ void store_fp8_as_bf16(const u32x4 (&src)[8], ATTN_LDS char* buf,
                                                  int wave, int lane) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r = wave * kRowsPerWaveLoad + 2 * i + (lane >> 5);
        const int c0 = 2 * (lane & 31);  // logical 16-byte chunks c0, c0 + 1 of row r
        bf16x8 lo, hi;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const uint32_t word = src[i][w];
            const auto f01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)word, false);
            const auto f23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)word, true);
            bf16x8& dstv = w < 2 ? lo : hi;
            const int base = (w & 1) * 4;
            dstv[base + 0] = (__bf16)f01[0];
            dstv[base + 1] = (__bf16)f01[1];
            dstv[base + 2] = (__bf16)f23[0];
            dstv[base + 3] = (__bf16)f23[1];
        }
        const int sw = swz(r);
        *(ATTN_LDS bf16x8*)(buf + r * kRowBytes + ((c0 ^ sw) << 4)) = lo;
        *(ATTN_LDS bf16x8*)(buf + r * kRowBytes + (((c0 + 1) ^ sw) << 4)) = hi;
    }
}

template <bool FP8>
__global__ __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_split_kernel(DecodeArgs a) {
    __shared__ __attribute__((aligned(1024))) char smem[2 * kTileBytes + kDecRows * kSxStride];
    ATTN_LDS char* sK = (ATTN_LDS char*)smem;
    ATTN_LDS char* sV = sK + kTileBytes;
    ATTN_LDS char* sX = sV + kTileBytes;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int split = blockIdx.x % a.max_splits;
    const int rest = blockIdx.x / a.max_splits;
    const int kvh = rest % a.hkv;
    const int b = rest / a.hkv;

    int L = a.kv_lens[b];
    L = L < 0 ? 0 : (L > a.max_pages * kPage ? a.max_pages * kPage : L);
    const int tile0 = split * a.tiles_per_split;
    const int k_begin = tile0 * kPage;
    if (k_begin >= L) return;  // empty split: the merge never reads it
    const int k_end = min(k_begin + a.tiles_per_split * kPage, L);
    const int ntiles = (k_end - k_begin + kPage - 1) / kPage;

    // lane roles: n = query head of the group (MFMA column), kq = k-group
    const int n = lane & 15;
    const int kq = lane >> 4;
    const bool row_ok = n < a.g;

    // Q^T operand, k-step ks covers dims 32 ks .. 32 ks + 31; lane holds 32 ks + 8 kq .. + 7
    bf16x8 qf[16];
    {
        const bf16x8* qp = (const bf16x8*)(a.q + ((size_t)b * a.hq + kvh * a.g +
                                                  (row_ok ? n : 0)) * kHeadDim) + kq;
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) {
            const bf16x8 v = qp[4 * ks];
            qf[ks] = row_ok ? v : bf16x8{};
        }
    }
    // K operand offsets: row 16 wave + n, chunk 4 ks + kq; with ks = 4 u + v the
    // byte offset is koff[v] + 256 u.
    int koff[4];
#pragma unroll
    for (int v = 0; v < 4; ++v)
        koff[v] = (16 * wave + n) * kRowBytes + (((4 * v + kq) ^ swz(n)) << 4);
    // V^T operand (transposing reads): key row 32 c + 8 kq + (n >> 2) (+4 for the
    // second read), dims 128 wave + 16 db + 4 (n & 3), i.e. logical chunk
    // 16 wave + 2 db + (n & 3) / 2 at byte 8 (n & 1).  Rows of different c
    // share the swizzle (32 c is a multiple of 16).
    int vrow[2], vsw[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        vrow[half] = (8 * kq + (n >> 2) + 4 * half) * kRowBytes + 8 * (n & 1);
        vsw[half] = swz(8 * kq + (n >> 2) + 4 * half);
    }
    const int vchunk0 = 16 * wave + ((n & 3) >> 1);
    f32x4 o[8];
#pragma unroll
    for (int db = 0; db < 8; ++db) o[db] = f32x4{};
    float m_run = -__builtin_inff();
    float l_run = 0.f;

    const int* ptab = a.page_table + (size_t)b * a.max_pages;
    const int lane16 = lane * 16;
    const int tile_bytes = FP8 ? kTileBytes / 2 : kTileBytes;
    Fp8Stage st;
    if constexpr (FP8) {
        const int valid0 = min(L - k_begin, kPage);
        load_fp8(st.k, page_tile(a.k_pages, ptab, tile0, a.num_pages, a.hkv, kvh, tile_bytes),
                 valid0, wave, lane);
        load_fp8(st.v, page_tile(a.v_pages, ptab, tile0, a.num_pages, a.hkv, kvh, tile_bytes),
                 valid0, wave, lane);
    } else {
        const int valid0 = min(L - k_begin, kPage);
        issue_tile_bf16(page_tile(a.k_pages, ptab, tile0, a.num_pages, a.hkv, kvh, tile_bytes),
                        valid0, sK, wave, lane16);
        issue_tile_bf16(page_tile(a.v_pages, ptab, tile0, a.num_pages, a.hkv, kvh, tile_bytes),
                        valid0, sV, wave, lane16);
    }

    for (int t = 0; t < ntiles; ++t) {
        const int key0 = k_begin + t * kPage;
        const bool more = t + 1 < ntiles;
        if constexpr (FP8) {
            // the previous tile's readers passed the barrier at the loop end
            store_fp8_as_bf16(st.k, sK, wave, lane);
            store_fp8_as_bf16(st.v, sV, wave, lane);
            if (more) {
                const int vn = min(L - (key0 + kPage), kPage);
                load_fp8(st.k, page_tile(a.k_pages, ptab, tile0 + t + 1, a.num_pages, a.hkv, kvh,
                                         tile_bytes), vn, wave, lane);
                load_fp8(st.v, page_tile(a.v_pages, ptab, tile0 + t + 1, a.num_pages, a.hkv, kvh,
                                         tile_bytes), vn, wave, lane);
            }
            lds_barrier();
        } else {
            wait_vmcnt<kRowsPerWaveLoad>();   // K(t) in; V(t) may still be in flight
            lds_barrier();
        }

        // ---- S^T[16 keys of this wave][16 heads] over 512 dims
        f32x4 s = f32x4{};
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) {
            const bf16x8 kv = *(const ATTN_LDS bf16x8*)(sK + koff[ks & 3] + 256 * (ks >> 2));
            s = mfma16x16x32(kv, qf[ks], s);
        }
        // accumulator element i is key 16 wave + 4 kq + i of head n
        *(ATTN_LDS f32x4*)(sX + n * kSxStride + (16 * wave + 4 * kq) * 4) = s;
        lds_barrier();  // scores visible; every wave is done with sK
        if constexpr (!FP8) {
            if (more) {
                const int vn = min(L - (key0 + kPage), kPage);
                issue_tile_bf16(page_tile(a.k_pages, ptab, tile0 + t + 1, a.num_pages, a.hkv,
                                          kvh, tile_bytes), vn, sK, wave, lane16);
            }
        }

        // ---- online softmax over the tile; this lane takes keys 32 c + 8 kq + j
        float x[2][8];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const f32x4 lo = *(const ATTN_LDS f32x4*)(sX + n * kSxStride + (32 * c + 8 * kq) * 4);
            const f32x4 hi = *(const ATTN_LDS f32x4*)(sX + n * kSxStride + (32 * c + 8 * kq + 4) * 4);
#pragma unroll
            for (int j = 0; j < 4; ++j) { x[c][j] = lo[j]; x[c][4 + j] = hi[j]; }
        }
        float mt = -__builtin_inff();
#pragma unroll
        for (int c = 0; c < 2; ++c) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int key = key0 + 32 * c + 8 * kq + j;
                const float v = key < k_end ? x[c][j] * a.scale_log2 : -__builtin_inff();
                x[c][j] = v;
                mt = fmaxf(mt, v);
            }
        }
        mt = fmaxf(mt, __shfl_xor(mt, 16));
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const float m_new = fmaxf(m_run, mt);   // finite: every tile has a visible key
        const float alpha = fast_exp2(m_run - m_new);
        bf16x8 pf[2];
        float psum = 0.f;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float p = fast_exp2(x[c][j] - m_new);
                psum += p;
                pf[c][j] = (__bf16)p;
            }
        }
        l_run = l_run * alpha + psum;
        m_run = m_new;
#pragma unroll
        for (int db = 0; db < 8; ++db) o[db] *= alpha;

        if constexpr (!FP8) {
            if (more) wait_vmcnt<kRowsPerWaveLoad>(); else wait_vmcnt<0>();
            lds_barrier();  // V(t) visible
        }

        // ---- O^T[128 dims of this wave][16 heads] += V^T P^T
#pragma unroll
        for (int c = 0; c < 2; ++c) {
#pragma unroll
            for (int db = 0; db < 8; ++db) {
                const int ch = vchunk0 + 2 * db;
                const ATTN_LDS char* base = sV + 32 * c * kRowBytes;
                const bf16x4 va = lds_read_tr16(base + vrow[0] + ((ch ^ vsw[0]) << 4));
                const bf16x4 vb = lds_read_tr16(base + vrow[1] + ((ch ^ vsw[1]) << 4));
                const bf16x8 vt = __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7);
                o[db] = mfma16x16x32(vt, pf[c], o[db]);
            }
        }
        lds_barrier();  // every wave is done with sV and sX
        if constexpr (!FP8) {
            if (more) {
                const int vn = min(L - (key0 + kPage), kPage);
                issue_tile_bf16(page_tile(a.v_pages, ptab, tile0 + t + 1, a.num_pages, a.hkv,
                                          kvh, tile_bytes), vn, sV, wave, lane16);
            }
        }
    }

    // ---- partial: O^T accumulator element i of block db is dim
    // 128 wave + 16 db + 4 kq + i of head n.  l sums over the four k-groups.
    float l_row = l_run + __shfl_xor(l_run, 16);
    l_row += __shfl_xor(l_row, 32);
    if (row_ok) {
        const size_t slot = (((size_t)b * a.hkv + kvh) * a.max_splits + split) * a.g + n;
        float* dst = a.part_o + slot * kHeadDim + 128 * wave + 4 * kq;
#pragma unroll
        for (int db = 0; db < 8; ++db) *(f32x4*)(dst + 16 * db) = o[db] * a.v_scale;
        if (wave == 0 && kq == 0) {
            a.part_ml[2 * slot] = m_run;
            a.part_ml[2 * slot + 1] = l_row;
        }
    }
}

// One workgroup per (sequence, query head): combine the sequence's partials,
// mu = max m_i, o = sum 2^(m_i - mu) O_i / sum 2^(m_i - mu) l_i.
template <bool OUT_FP32>
__global__ __launch_bounds__(128) void decode_merge_kernel(DecodeArgs a, void* out) {
    const int b = blockIdx.x / a.hq;
    const int h = blockIdx.x - b * a.hq;
    const int kvh = h / a.g;
    const int r = h - kvh * a.g;
    int L = a.kv_lens[b];
    L = L < 0 ? 0 : (L > a.max_pages * kPage ? a.max_pages * kPage : L);
    const int split_keys = a.tiles_per_split * kPage;
    int ns = (L + split_keys - 1) / split_keys;
    ns = ns > a.max_splits ? a.max_splits : ns;
    const size_t slot0 = (((size_t)b * a.hkv + kvh) * a.max_splits) * a.g + r;
    float mu = -__builtin_inff();
    for (int i = 0; i < ns; ++i) mu = fmaxf(mu, a.part_ml[2 * (slot0 + (size_t)i * a.g)]);
    f32x4 acc = f32x4{};
    float den = 0.f;
    const int d0 = 4 * threadIdx.x;
    for (int i = 0; i < ns; ++i) {
        const size_t slot = slot0 + (size_t)i * a.g;
        const float w = fast_exp2(a.part_ml[2 * slot] - mu);
        den += w * a.part_ml[2 * slot + 1];
        acc += w * *(const f32x4*)(a.part_o + slot * kHeadDim + d0);
    }
    // IEEE division, as in prefill; no visible key gives 0
    const float dd = den > 0.f ? den : 1.f;
    const size_t obase = ((size_t)b * a.hq + h) * kHeadDim + d0;
    const f32x4 v = {acc[0] / dd, acc[1] / dd, acc[2] / dd, acc[3] / dd};
    if constexpr (OUT_FP32) {
        *(f32x4*)((float*)out + obase) = v;
    } else {
        *(bf16x4*)((__bf16*)out + obase) = bf16x4{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
    }
}

int default_keys_per_split(int batch, int hkv, int max_kv_len) {
    const long long total = (long long)batch * hkv * max_kv_len;
    long long s = (total + kDefaultTargetWgs - 1) / kDefaultTargetWgs;
    s = (s + kPage - 1) / kPage * kPage;
    if (s < 4 * kPage) s = 4 * kPage;
    return (int)s;
}

}  // namespace

}  // namespace attn

extern "C" size_t attn_decode_splitk_workspace_size(int batch, int num_q_heads, int num_kv_heads,
                                                    int max_kv_len, int keys_per_split) {
    using namespace attn;
    if (batch < 1 || num_q_heads < 1 || num_kv_heads < 1 || max_kv_len < 1 ||
        num_q_heads % num_kv_heads || keys_per_split < 0 || keys_per_split % kPage)
        return 0;
    const int kps = keys_per_split ? keys_per_split
                                   : default_keys_per_split(batch, num_kv_heads, max_kv_len);
    const size_t splits = (size_t)(max_kv_len + kps - 1) / kps;
    const size_t slots = (size_t)batch * num_q_heads * splits;  // hkv * g = hq
    return slots * (kHeadDim + 2) * sizeof(float);
}

extern "C" int attn_decode_splitk(const void* q, const void* k_pages, const void* v_pages,
                                  int kv_dtype, float k_scale, float v_scale,
                                  const int32_t* page_table, const int32_t* kv_lens, int batch,
                                  int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                                  int num_pages, int max_pages_per_seq, int max_kv_len,
                                  int keys_per_split, float softmax_scale, void* workspace,
                                  size_t workspace_bytes, void* out, int out_dtype,
                                  hipStream_t stream) {
    using namespace attn;
    if (!q || !k_pages || !v_pages || !page_table || !kv_lens || !out) return ATTN_ERR_NULL;
    if (batch < 1 || num_q_heads < 1 || num_kv_heads < 1 || num_pages < 1 ||
        max_pages_per_seq < 1 || max_kv_len < 1 || keys_per_split < 0 ||
        !(softmax_scale == softmax_scale))
        return ATTN_ERR_SHAPE;
    if (num_q_heads % num_kv_heads || keys_per_split % kPage) return ATTN_ERR_SHAPE;
    if ((long long)max_kv_len > (long long)max_pages_per_seq * kPage) return ATTN_ERR_SHAPE;
    if (head_dim != kHeadDim || page_size != kPage) return ATTN_ERR_UNSUPPORTED;
    const int g = num_q_heads / num_kv_heads;
    if (g > kDecRows) return ATTN_ERR_UNSUPPORTED;
    if (kv_dtype != ATTN_BF16 && kv_dtype != ATTN_FP8_E4M3) return ATTN_ERR_UNSUPPORTED;
    if (out_dtype != ATTN_BF16 && out_dtype != ATTN_FP32) return ATTN_ERR_UNSUPPORTED;
    if (kv_dtype == ATTN_FP8_E4M3 && (!(k_scale > 0.f) || !(v_scale > 0.f))) return ATTN_ERR_SHAPE;
    const size_t need = attn_decode_splitk_workspace_size(batch, num_q_heads, num_kv_heads,
                                                          max_kv_len, keys_per_split);
    if (!workspace || workspace_bytes < need || need == 0) return ATTN_ERR_WORKSPACE;

    const int kps = keys_per_split ? keys_per_split
                                   : default_keys_per_split(batch, num_kv_heads, max_kv_len);
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
    a.max_pages = max_pages_per_seq;
    a.num_pages = num_pages;
    a.max_splits = (max_kv_len + kps - 1) / kps;
    a.tiles_per_split = kps / kPage;
    const size_t slots = (size_t)batch * num_q_heads * a.max_splits;
    a.part_o = (float*)workspace;
    a.part_ml = (float*)workspace + slots * kHeadDim;
    const bool fp8 = kv_dtype == ATTN_FP8_E4M3;
    a.scale_log2 = softmax_scale * 1.4426950408889634f * (fp8 ? k_scale : 1.f);
    a.v_scale = fp8 ? v_scale : 1.f;
    const long long grid = (long long)batch * num_kv_heads * a.max_splits;
    if (grid > 0x7fffffffLL || (long long)batch * num_q_heads > 0x7fffffffLL) return ATTN_ERR_SHAPE;
    if (fp8)
        hipLaunchKernelGGL(decode_split_kernel<true>, dim3((unsigned)grid), dim3(kDecThreads), 0,
                           stream, a);
    else
        hipLaunchKernelGGL(decode_split_kernel<false>, dim3((unsigned)grid), dim3(kDecThreads), 0,
                           stream, a);
    if (hipGetLastError() != hipSuccess) return ATTN_ERR_HIP;
    if (out_dtype == ATTN_FP32)
        hipLaunchKernelGGL(decode_merge_kernel<true>, dim3((unsigned)(batch * num_q_heads)),
                           dim3(128), 0, stream, a, out);
    else
        hipLaunchKernelGGL(decode_merge_kernel<false>, dim3((unsigned)(batch * num_q_heads)),
                           dim3(128), 0, stream, a, out);
    return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}
