// combine.hip -- the weighted combine of the expert outputs, as its own
// kernel after the down projection (the split launch of the bf16 matrix-core
// path):
//
//   out[t, n] = sum_{j = 0 .. k-1} w[t, j] * y[pos[t, j], n]  (+ y[sh_row0 + t, n]),
//   fp32 in slot order j, the shared expert's row (if any) added last,
//   rounded to bf16 (nearest even)
//
// (pos null: the self-routed layer, whose y rows are the slots t*k + j)
//
// (the routing weights renormalised over the token's top-k experts, the
// standard MoE combine the layer's problem statement names).  The same fmaf
// chain as the last-finisher combine of the single-launch layer, so both
// give the same bits.  Reads y once (T*k rows of H fp32) and writes out
// once; the kernel boundary before it makes every y row written by the down
// kernel visible, whatever XCD wrote it.
#include "device_common.h"

namespace moe {
namespace {

constexpr int kCombineThreads = 256;

// Slots [j0, j0 + n) of token t (n <= 8) added to v in slot order: their
// indices and weights first, then the n y rows, then the fmaf chain, so a
// batch costs two memory latencies instead of two per slot.
template <int N>
__device__ inline void combine_batch(const GemmArgs& a, int64_t base, int j0, int c4, float4& v) {
    int p[N];
    float w[N];
    float4 y[N];
#pragma unroll
    for (int u = 0; u < N; u++) {
        p[u] = a.pos ? a.pos[base + j0 + u] : (int)(base + j0 + u);
        w[u] = a.wts[base + j0 + u];
    }
#pragma unroll
    for (int u = 0; u < N; u++)
        y[u] = *reinterpret_cast<const float4*>(a.y + (int64_t)p[u] * a.H + 4 * c4);
#pragma unroll
    for (int u = 0; u < N; u++) {
        v.x = fmaf(w[u], y[u].x, v.x);
        v.y = fmaf(w[u], y[u].y, v.y);
        v.z = fmaf(w[u], y[u].z, v.z);
        v.w = fmaf(w[u], y[u].w, v.w);
    }
}

// blockIdx.x = token * blocks_per_token + column block; each thread owns
// four consecutive columns (one 16-byte load per slot).
__global__ void __launch_bounds__(kCombineThreads) combine_kernel(GemmArgs a) {
    const int per_token = (a.H / 4 + kCombineThreads - 1) / kCombineThreads;
    const int t = blockIdx.x / per_token;
    const int c4 = (blockIdx.x % per_token) * kCombineThreads + threadIdx.x;
    if (c4 * 4 >= a.H) return;
    const int64_t base = (int64_t)t * a.k;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    int j0 = 0;
    for (; j0 + 8 <= a.k; j0 += 8) combine_batch<8>(a, base, j0, c4, v);
    switch (a.k - j0) {  // the last partial batch
        case 1: combine_batch<1>(a, base, j0, c4, v); break;
        case 2: combine_batch<2>(a, base, j0, c4, v); break;
        case 3: combine_batch<3>(a, base, j0, c4, v); break;
        case 4: combine_batch<4>(a, base, j0, c4, v); break;
        case 5: combine_batch<5>(a, base, j0, c4, v); break;
        case 6: combine_batch<6>(a, base, j0, c4, v); break;
        case 7: combine_batch<7>(a, base, j0, c4, v); break;
        default: break;
    }
    if (a.sh_wgu) {
        const float4 s = *reinterpret_cast<const float4*>(a.y + (int64_t)(a.sh_row0 + t) * a.H + 4 * c4);
        v.x += s.x;
        v.y += s.y;
        v.z += s.z;
        v.w += s.w;
    }
    ushort4 o;
    o.x = f32_to_bf16_rne(v.x);
    o.y = f32_to_bf16_rne(v.y);
    o.z = f32_to_bf16_rne(v.z);
    o.w = f32_to_bf16_rne(v.w);
    *reinterpret_cast<ushort4*>(a.out + (int64_t)t * a.H + 4 * c4) = o;
}

}  // namespace

hipError_t launch_combine(const GemmArgs& a, hipStream_t stream) {
    const int per_token = (a.H / 4 + kCombineThreads - 1) / kCombineThreads;
    combine_kernel<<<a.T * per_token, kCombineThreads, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace moe
