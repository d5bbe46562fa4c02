// Measurement helpers.
//
// Same-process HBM read roofline: stream a buffer once with 16-byte loads.
// The buffer should be well beyond the 256 MB Infinity Cache so the rate is
// the HBM rate.  Each workgroup folds what it read into one word of `sink`
// so the loads cannot be dropped.
//
// Clock stamps: each workgroup's first lane records where it runs (XCD and
// hardware id) and two counters, s_memtime (counts shader-clock cycles, so
// its rate follows the clock; not synchronised between compute units) and
// s_memrealtime (a constant 100 MHz).  Two stamp launches around a timed
// region give, for every compute unit that holds a stamp of both, its mean
// shader clock over the region.
#include "device_common.h"
#include "attn_host.h"

namespace attn {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;          // 16-byte loads in flight per thread
constexpr size_t kBytesPerWg = (size_t)kProbeThreads * 16 * kProbeUnroll;

__global__ __launch_bounds__(kProbeThreads) void hbm_read_kernel(const u32x4* buf, size_t n16,
                                                                 uint32_t* sink) {
    u32x4 acc = u32x4{0u, 0u, 0u, 0u};
    const size_t base = (size_t)blockIdx.x * kProbeThreads * kProbeUnroll + threadIdx.x;
    u32x4 v[kProbeUnroll];
#pragma unroll
    for (int i = 0; i < kProbeUnroll; ++i) {
        const size_t idx = base + (size_t)i * kProbeThreads;
        v[i] = idx < n16 ? __builtin_nontemporal_load(buf + idx) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < kProbeUnroll; ++i) acc ^= v[i];
    uint32_t w = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    for (int off = 32; off > 0; off >>= 1) w ^= __shfl_xor(w, off);
    if (threadIdx.x == 0) sink[blockIdx.x] = w;
}

// One 64-lane workgroup per slot: lane 0 writes {XCD id << 32 | HW_ID,
// s_memtime, s_memrealtime} (three 64-bit words) to slot blockIdx.x.
__global__ __launch_bounds__(64) void clock_stamp_kernel(unsigned long long* out) {
    // HW_REG_XCC_ID (hardware register 20), bits 0..3: the XCD this wave runs
    // on; HW_REG_HW_ID (4): its compute unit (bits 8..11), shader array (12)
    // and shader engine (13..15), among other fields
    const unsigned xcc = __builtin_amdgcn_s_getreg((3 << 11) | 20);
    const unsigned hw = __builtin_amdgcn_s_getreg((31 << 11) | 4);
    const unsigned long long t = __builtin_amdgcn_s_memtime();
    const unsigned long long rt = __builtin_amdgcn_s_memrealtime();
    if (threadIdx.x == 0) {
        out[3 * blockIdx.x] = ((unsigned long long)(xcc & 15) << 32) | hw;
        out[3 * blockIdx.x + 1] = t;
        out[3 * blockIdx.x + 2] = rt;
    }
}

}  // namespace
}  // namespace attn

extern "C" int attn_clock_stamps(void* stamps, int slots, hipStream_t stream) {
    using namespace attn;
    if (!stamps) return ATTN_ERR_NULL;
    if (slots < 1 || slots > 65536) return ATTN_ERR_SHAPE;
    hipLaunchKernelGGL(clock_stamp_kernel, dim3((unsigned)slots), dim3(64), 0, stream,
                       (unsigned long long*)stamps);
    return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

extern "C" size_t attn_hbm_probe_sink_words(size_t bytes) {
    return (bytes + attn::kBytesPerWg - 1) / attn::kBytesPerWg;
}

extern "C" int attn_hbm_read_probe(const void* buf, size_t bytes, void* sink, hipStream_t stream) {
    using namespace attn;
    if (!buf || !sink) return ATTN_ERR_NULL;
    if (bytes == 0 || bytes % 16) return ATTN_ERR_SHAPE;
    const size_t grid = attn_hbm_probe_sink_words(bytes);
    if (grid > 0x7fffffffULL) return ATTN_ERR_SHAPE;
    hipLaunchKernelGGL(hbm_read_kernel, dim3((unsigned)grid), dim3(kProbeThreads), 0, stream,
                       (const u32x4*)buf, bytes / 16, (uint32_t*)sink);
    return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}
