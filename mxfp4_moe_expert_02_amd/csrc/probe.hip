// probe.hip -- streaming-read and copy kernels that calibrate the HBM
// roofline and the traffic counters (include/moe_mxfp4_probe.h).
#include "../../include/moe_mxfp4.h"
#include "../../include/moe_mxfp4_probe.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeBlocks = 256 * 8;   // 8 workgroups per CU on 256 CUs
constexpr int kProbeUnroll = 8;         // 128-bit loads in flight per thread

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(kProbeThreads)
stream_read_kernel(const u32x4_t* __restrict__ src, int64_t n16, uint32_t* __restrict__ sink) {
    const int64_t tid = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
    uint32_t acc = 0;
    int64_t i = tid;
    for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
        u32x4_t v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; u++) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < kProbeUnroll; u++) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {
        u32x4_t v = __builtin_nontemporal_load(src + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    sink[tid] = acc;
}

__global__ void __launch_bounds__(kProbeThreads)
copy_kernel(const u32x4_t* __restrict__ src, u32x4_t* __restrict__ dst, int64_t n16) {
    const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
    for (int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x; i < n16; i += stride)
        dst[i] = src[i];
}

}  // namespace
}  // namespace moe

extern "C" {

int64_t moe_probe_sink_words(void) { return (int64_t)moe::kProbeBlocks * moe::kProbeThreads; }

int moe_probe_stream_read(const void* src, int64_t bytes, uint32_t* sink, void* stream) {
    if (!src || !sink) return MOE_E_NULL;
    if (bytes < 0 || bytes % 16) return MOE_E_SHAPE;
    if (((uintptr_t)src & 15u) || ((uintptr_t)sink & 3u)) return MOE_E_ALIGN;
    moe::stream_read_kernel<<<moe::kProbeBlocks, moe::kProbeThreads, 0, (hipStream_t)stream>>>(
        (const moe::u32x4_t*)src, bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_E_HIP;
}

int moe_probe_copy(const void* src, void* dst, int64_t bytes, void* stream) {
    if (!src || !dst) return MOE_E_NULL;
    if (bytes < 0 || bytes % 16) return MOE_E_SHAPE;
    if (((uintptr_t)src & 15u) || ((uintptr_t)dst & 15u)) return MOE_E_ALIGN;
    moe::copy_kernel<<<moe::kProbeBlocks, moe::kProbeThreads, 0, (hipStream_t)stream>>>(
        (const moe::u32x4_t*)src, (moe::u32x4_t*)dst, bytes / 16);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_E_HIP;
}

}  // extern "C"
