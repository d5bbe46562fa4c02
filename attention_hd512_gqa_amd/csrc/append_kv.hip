// Paged KV append for gfx950: writes the key and value rows of a chunk's new
// tokens into their cache slots, one page of one KV head holding 64
// consecutive key rows of 512, so that one page is exactly one key tile of
// the attention kernels (pegainfer issue 1051, "Proposed Plan").
//
// Token i of sequence b sits at position p = q_start_pos[b] + i; its rows go
// to page page_table[b][p / 64], slot p % 64, for every KV head.  An FP8-E4M3
// pool stores round-to-nearest-even(x / scale) saturated to +-448 (the OCP
// E4M3FN range), the encoding the attention kernels widen back exactly.
//
// Pure data movement: each thread moves 8 elements (16 bytes of bf16 in,
// 16 or 8 bytes out) of one row, so every wave reads and writes whole 1 KB
// rows; HBM bandwidth bounds it.
#include "device_common.h"
#include "attn_host.h"

namespace attn {
namespace {

constexpr int kAppendThreads = 256;
constexpr int kChunksPerRow = kHeadDim / 8;

struct AppendArgs {
    const __bf16* k_new;
    const __bf16* v_new;
    char* k_pages;
    char* v_pages;
    const int* page_table;
    const int* cu_seqlens;
    const int* q_start;
    int batch, total_q, hkv, max_pages, num_pages;
    float k_scale, v_scale;   // FP8 only
};

// x / scale (IEEE division) clamped to [-448, 448]; NaN stays NaN.
__device__ __forceinline__ float e4m3_prescale(float x, float scale) {
    float y = x / scale;
    y = y > 448.f ? 448.f : y;
    y = y < -448.f ? -448.f : y;
    return y;
}

template <bool FP8>
__global__ __launch_bounds__(kAppendThreads) void append_kv_kernel(AppendArgs a) {
    const long long total = (long long)a.total_q * a.hkv * kChunksPerRow;
    for (long long idx = (long long)blockIdx.x * kAppendThreads + threadIdx.x; idx < total;
         idx += (long long)gridDim.x * kAppendThreads) {
        const int chunk = (int)(idx % kChunksPerRow);
        const long long rowi = idx / kChunksPerRow;       // token * hkv + kvh
        const int kvh = (int)(rowi % a.hkv);
        const int tok = (int)(rowi / a.hkv);
        // sequence of the token: last b with cu_seqlens[b] <= tok
        int lo = 0, hi = a.batch - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (a.cu_seqlens[mid] <= tok) lo = mid; else hi = mid - 1;
        }
        const int pos = a.q_start[lo] + (tok - a.cu_seqlens[lo]);
        if (pos < 0 || pos / kPage >= a.max_pages) continue;            // outside the table
        const int page = a.page_table[(size_t)lo * a.max_pages + pos / kPage];
        if (page < 0 || page >= a.num_pages) continue;                  // outside the pool
        const size_t src = (size_t)rowi * kHeadDim + 8 * chunk;
        const size_t dst_row = ((size_t)page * a.hkv + kvh) * kPage + pos % kPage;
        const bf16x8 kv = *(const bf16x8*)(a.k_new + src);
        const bf16x8 vv = *(const bf16x8*)(a.v_new + src);
        if constexpr (FP8) {
            uint32_t kw[2], vw[2];
#pragma unroll
            for (int w = 0; w < 2; ++w) {
                int k2 = 0, v2 = 0;
                k2 = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_prescale((float)kv[4 * w], a.k_scale),
                                                     e4m3_prescale((float)kv[4 * w + 1], a.k_scale), k2, false);
                k2 = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_prescale((float)kv[4 * w + 2], a.k_scale),
                                                     e4m3_prescale((float)kv[4 * w + 3], a.k_scale), k2, true);
                v2 = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_prescale((float)vv[4 * w], a.v_scale),
                                                     e4m3_prescale((float)vv[4 * w + 1], a.v_scale), v2, false);
                v2 = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_prescale((float)vv[4 * w + 2], a.v_scale),
                                                     e4m3_prescale((float)vv[4 * w + 3], a.v_scale), v2, true);
                kw[w] = (uint32_t)k2;
                vw[w] = (uint32_t)v2;
            }
            const size_t d = dst_row * kHeadDim + 8 * chunk;
            *(uint2*)(a.k_pages + d) = make_uint2(kw[0], kw[1]);
            *(uint2*)(a.v_pages + d) = make_uint2(vw[0], vw[1]);
        } else {
            const size_t d = (dst_row * kHeadDim + 8 * chunk) * 2;
            *(bf16x8*)(a.k_pages + d) = kv;
            *(bf16x8*)(a.v_pages + d) = vv;
        }
    }
}

}  // namespace
}  // namespace attn

extern "C" int attn_append_kv(const void* k_new, const void* v_new, int kv_dtype, float k_scale,
                              float v_scale, const int32_t* page_table,
                              const int32_t* cu_seqlens, const int32_t* q_start_pos, int batch,
                              int total_q, int num_kv_heads, int head_dim, int page_size,
                              int num_pages, int max_pages_per_seq, void* k_pages,
                              void* v_pages, hipStream_t stream) {
    using namespace attn;
    if (!k_new || !v_new || !page_table || !cu_seqlens || !q_start_pos || !k_pages || !v_pages)
        return ATTN_ERR_NULL;
    if (batch < 1 || total_q < 0 || num_kv_heads < 1 || num_pages < 1 || max_pages_per_seq < 1)
        return ATTN_ERR_SHAPE;
    if (head_dim != kHeadDim || page_size != kPage) return ATTN_ERR_UNSUPPORTED;
    if (kv_dtype != ATTN_BF16 && kv_dtype != ATTN_FP8_E4M3) return ATTN_ERR_UNSUPPORTED;
    const bool fp8 = kv_dtype == ATTN_FP8_E4M3;
    if (fp8 && (!(k_scale > 0.f) || !(v_scale > 0.f))) return ATTN_ERR_SHAPE;
    if (total_q == 0) return ATTN_OK;
    AppendArgs a;
    a.k_new = (const __bf16*)k_new;
    a.v_new = (const __bf16*)v_new;
    a.k_pages = (char*)k_pages;
    a.v_pages = (char*)v_pages;
    a.page_table = page_table;
    a.cu_seqlens = cu_seqlens;
    a.q_start = q_start_pos;
    a.batch = batch;
    a.total_q = total_q;
    a.hkv = num_kv_heads;
    a.max_pages = max_pages_per_seq;
    a.num_pages = num_pages;
    a.k_scale = fp8 ? k_scale : 1.f;
    a.v_scale = fp8 ? v_scale : 1.f;
    const long long total = (long long)total_q * num_kv_heads * kChunksPerRow;
    long long grid = (total + kAppendThreads - 1) / kAppendThreads;
    if (grid > 65536) grid = 65536;   // grid-stride beyond that
    if (fp8)
        hipLaunchKernelGGL(append_kv_kernel<true>, dim3((unsigned)grid), dim3(kAppendThreads), 0,
                           stream, a);
    else
        hipLaunchKernelGGL(append_kv_kernel<false>, dim3((unsigned)grid), dim3(kAppendThreads), 0,
                           stream, a);
    return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}
