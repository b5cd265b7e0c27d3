// router.hip -- the router linear layer upstream of top-k, on the bf16
// matrix cores: logits [T, E] = x [T, H] . W_router [E, H]^T, bf16 inputs,
// fp32 accumulation.
//
// The pages quantise only the experts to 4 bits and keep routing at the
// model's original precision (sandbot 1000-TPS post, technical-breakdown
// section), and give top-k selection and routing a stage of their own
// ahead of the heavy work (HyperAI transcript, the heterogeneous-worker
// example).  Here the router product runs as one kernel ahead of the
// routing, so the layer can take x and the router weight instead of
// precomputed logits.
//
// A workgroup of four waves owns one tile of 16 tokens x ET 16-expert tiles
// (ET = 4 when each workgroup takes the whole K, else 1) and a K range; each wave takes a quarter of it,
// v_mfma_f32_16x16x32_bf16 per expert tile: A = router rows e0..e0+15
// (lane (r, g): 8 bf16 at k + 8g of row e0 + r), B = token rows t0..t0+15
// (lane (c, g): 8 bf16 at k + 8g of token t0 + c), loaded once for the
// ET expert tiles; D: lane (c, g) holds experts e0 + 4g .. +3 of token
// t0 + c.  Rows past E or T read the last row (valid memory) and are never
// stored.  A wave issues the loads of four steps (128 k) before their
// MFMAs; the four waves' sums meet in LDS in wave order.  Layers with many
// tiles give a workgroup the whole K.  Few tiles (verify steps) split K
// over nsplit workgroups of one load batch per wave, so that enough waves
// stream the weight: each stores its partial tile through agent-coherent
// stores, waits for them to complete and counts itself done (no fence: an
// agent-scope release would write back the whole L2); the last of a tile
// reads the partials agent-coherently, adds them in split order (the same
// sum whichever finishes last) and resets the counter.
#include "device_common.h"

namespace moe {
namespace {

constexpr int kRouterThreads = 256;
constexpr int kRouterBatch = 4;  // 32-k steps per load batch

template <int ET>
__global__ void __launch_bounds__(kRouterThreads)
router_gemm_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, int T, int E,
                   int H, int nsplit, int wave_steps, float* __restrict__ partial,
                   int32_t* __restrict__ tile_cnt, float* __restrict__ logits) {
    __shared__ f32x4_t red[3][ET][kWave];
    const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave, c = lane % 16, g = lane / 16;
    const int egroups = (E + 16 * ET - 1) / (16 * ET);
    const int tile = blockIdx.x / nsplit, sp = blockIdx.x % nsplit;
    const int e0 = 16 * ET * (tile % egroups), t0 = 16 * (tile / egroups);
    const uint16_t* arow[ET];
#pragma unroll
    for (int j = 0; j < ET; j++) arow[j] = wr + (int64_t)min(e0 + 16 * j + c, E - 1) * H + 8 * g;
    const uint16_t* brow = x + (int64_t)min(t0 + c, T - 1) * H + 8 * g;
    const int s0 = (sp * 4 + w) * wave_steps, s1 = min(H / 32, s0 + wave_steps);
    f32x4_t acc[ET];
#pragma unroll
    for (int j = 0; j < ET; j++) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int s = s0; s < s1; s += kRouterBatch) {
        u32x4_t A[kRouterBatch][ET], B[kRouterBatch];
#pragma unroll
        for (int i = 0; i < kRouterBatch; i++) {
            const int si = min(s + i, s1 - 1);
            B[i] = *reinterpret_cast<const u32x4_t*>(brow + 32 * si);
#pragma unroll
            for (int j = 0; j < ET; j++)
                A[i][j] = *reinterpret_cast<const u32x4_t*>(arow[j] + 32 * si);
        }
#pragma unroll
        for (int i = 0; i < kRouterBatch; i++)
            if (s + i < s1)
#pragma unroll
                for (int j = 0; j < ET; j++)
                    acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8_t, A[i][j]), __builtin_bit_cast(bf16x8_t, B[i]),
                        acc[j], 0, 0, 0);
    }
    if (w > 0)
#pragma unroll
        for (int j = 0; j < ET; j++) red[w - 1][j][lane] = acc[j];
    __syncthreads();
    if (w > 0) return;
#pragma unroll
    for (int v = 0; v < 3; v++)
#pragma unroll
        for (int j = 0; j < ET; j++) acc[j] += red[v][j][lane];
    const int t = t0 + c;
    if (nsplit == 1) {
#pragma unroll
        for (int j = 0; j < ET; j++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int e = e0 + 16 * j + 4 * g + i;
                if (t < T && e < E) logits[(int64_t)t * E + e] = acc[j][i];
            }
        return;
    }
#pragma unroll
    for (int j = 0; j < ET; j++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int e = e0 + 16 * j + 4 * g + i;
            if (t < T && e < E)
                __hip_atomic_store(partial + ((int64_t)sp * T + t) * E + e, acc[j][i],
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the partial tile is stored
    int old = 0;
    if (lane == 0) old = atomicAdd(&tile_cnt[tile], 1);
    old = __shfl(old, 0);
    if (old != nsplit - 1) return;
    const int tt = min(t, T - 1);
#pragma unroll
    for (int j = 0; j < ET; j++) {
        float p[4][kRouterMaxSplit];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int e = min(e0 + 16 * j + 4 * g + i, E - 1);
#pragma unroll
            for (int k = 0; k < kRouterMaxSplit; k++)
                p[i][k] = k < nsplit ? __hip_atomic_load(partial + ((int64_t)k * T + tt) * E + e,
                                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                     : 0.f;
        }
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int e = e0 + 16 * j + 4 * g + i;
            float v = 0.f;
#pragma unroll
            for (int k = 0; k < kRouterMaxSplit; k++)
                if (k < nsplit) v += p[i][k];
            if (t < T && e < E) logits[(int64_t)t * E + e] = v;
        }
    }
    if (lane == 0) __hip_atomic_store(&tile_cnt[tile], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

hipError_t launch_router_gemm(const uint16_t* x, const uint16_t* wr, int T, int E, int H,
                              const Workspace& ws, float* logits, hipStream_t stream) {
    const int steps = H / 32;
    const int ttiles = (T + 15) / 16;
    const int wide_tiles = ((E + 63) / 64) * ttiles;  // 16 tokens x 64 experts
    if (wide_tiles >= kRouterWaves / 2) {            // whole K per workgroup
        router_gemm_kernel<4><<<wide_tiles, kRouterThreads, 0, stream>>>(
            x, wr, T, E, H, 1, (steps + 3) / 4, ws.router_partial, ws.router_cnt, logits);
        return hipGetLastError();
    }
    // 16 tokens x 16 experts per workgroup, K split: one load batch per
    // wave, at most kRouterMaxSplit workgroups per tile
    const int tiles = ((E + 15) / 16) * ttiles;
    int nsplit = (steps + 4 * kRouterBatch - 1) / (4 * kRouterBatch);
    nsplit = nsplit > kRouterMaxSplit ? kRouterMaxSplit : nsplit;
    int wave_steps = (steps + 4 * nsplit - 1) / (4 * nsplit);
    wave_steps = (wave_steps + kRouterBatch - 1) / kRouterBatch * kRouterBatch;
    nsplit = (steps + 4 * wave_steps - 1) / (4 * wave_steps);
    router_gemm_kernel<1><<<tiles * nsplit, kRouterThreads, 0, stream>>>(
        x, wr, T, E, H, nsplit, wave_steps, ws.router_partial, ws.router_cnt, logits);
    return hipGetLastError();
}

}  // namespace moe
