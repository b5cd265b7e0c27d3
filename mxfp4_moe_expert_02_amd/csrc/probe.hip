// probe.hip -- streaming-read and copy kernels that calibrate the HBM
// roofline and the traffic counters (include/moe_mxfp4_probe.h).
#include "../../include/moe_mxfp4.h"
#include "../../include/moe_mxfp4_probe.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeBlocks = 256 * 4;    // 4 workgroups per CU on 256 CUs
constexpr int kProbeUnroll = 8;          // 128-bit loads in flight per thread
constexpr int kProbeChunkWords = 16384;  // 256 KB: the contiguous range a workgroup reads at a time

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Each workgroup reads whole 256 KB chunks (chunk blockIdx.x, then every
// gridDim.x-th), its 256 threads covering 32 KB contiguous per step with 8
// loads each; the words past the last whole chunk go grid-stride.  This is
// the expert GEMMs' pattern (a workgroup streams its quads' tiles, a few
// hundred KB, from start to end), and it reads faster than one grid-wide
// stride: 7.05 against 6.29 TB/s on 4 GiB, above every expert kernel.
// NT: nontemporal loads (the roofline probe, like the weight loads);
// otherwise ordinary loads, which allocate in L2 and the Infinity Cache
// (the eviction read before a cold step).
template <bool NT>
__global__ void __launch_bounds__(kProbeThreads)
stream_read_kernel(const u32x4_t* __restrict__ src, int64_t n16, uint32_t* __restrict__ sink) {
    uint32_t acc = 0;
    const int64_t n_chunks = n16 / kProbeChunkWords;
    for (int64_t ch = blockIdx.x; ch < n_chunks; ch += gridDim.x) {
        const u32x4_t* p = src + ch * kProbeChunkWords + threadIdx.x;
        for (int s = 0; s < kProbeChunkWords; s += kProbeThreads * kProbeUnroll) {
            u32x4_t v[kProbeUnroll];
#pragma unroll
            for (int u = 0; u < kProbeUnroll; u++)
                v[u] = NT ? __builtin_nontemporal_load(p + s + u * kProbeThreads) : p[s + u * kProbeThreads];
#pragma unroll
            for (int u = 0; u < kProbeUnroll; u++) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
        }
    }
    const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
    for (int64_t i = n_chunks * kProbeChunkWords + (int64_t)blockIdx.x * kProbeThreads + threadIdx.x; i < n16;
         i += stride) {
        const u32x4_t v = src[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    sink[(int64_t)blockIdx.x * kProbeThreads + threadIdx.x] = acc;
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

static int probe_read(const void* src, int64_t bytes, uint32_t* sink, void* stream, bool nontemporal) {
    if (!src || !sink) return MOE_E_NULL;
    if (bytes < 0 || bytes % 16) return MOE_E_SHAPE;
    if (((uintptr_t)src & 15u) || ((uintptr_t)sink & 3u)) return MOE_E_ALIGN;
    if (nontemporal)
        moe::stream_read_kernel<true><<<moe::kProbeBlocks, moe::kProbeThreads, 0, (hipStream_t)stream>>>(
            (const moe::u32x4_t*)src, bytes / 16, sink);
    else
        moe::stream_read_kernel<false><<<moe::kProbeBlocks, moe::kProbeThreads, 0, (hipStream_t)stream>>>(
            (const moe::u32x4_t*)src, bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_E_HIP;
}

int moe_probe_stream_read(const void* src, int64_t bytes, uint32_t* sink, void* stream) {
    return probe_read(src, bytes, sink, stream, true);
}

int moe_probe_read_cached(const void* src, int64_t bytes, uint32_t* sink, void* stream) {
    return probe_read(src, bytes, sink, stream, false);
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
