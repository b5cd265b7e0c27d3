// route.hip -- token routing for the MoE expert layer on gfx950.
//
// The pages say each expert is active on only a small fraction of the
// tokens and that MoE routing makes the work dynamic at run time
// (bjdmk.com.cn news page, co-design section; HyperAI transcript, section on
// maximum speed).  Routing here is top-k over fp32 router logits with a
// renormalised softmax, followed by a stable counting sort of the
// (token, slot) assignments by expert, so that each expert's tokens are
// contiguous and every expert that got no token produces no work at all.
//
// Two kernels:
//   route_topk_kernel  one wave per token: k rounds of a wave-wide arg-max
//                      over (logit desc, index asc), then the weights.
//   route_sort_kernel  one workgroup: per-range histograms in LDS, a scan
//                      over ranges and experts, a stable scatter, and the
//                      lists of active experts (heaviest first) per path.
// All of it is integer or compare-only except the weights, so ids, counts,
// offsets and the sorted order are bit-exact and deterministic.
#include <float.h>
#include <limits.h>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kTopkWavesPerBlock = 4;
constexpr int kMaxPerLane = kMaxExperts / kWave;  // 16 logits per lane

struct Cand {
    float v;
    int i;
};

// a beats b: larger logit, or equal logit and lower expert index
__device__ inline bool beats(float av, int ai, float bv, int bi) {
    return av > bv || (av == bv && ai < bi);
}

__global__ void __launch_bounds__(kTopkWavesPerBlock * kWave)
route_topk_kernel(const float* __restrict__ logits, int T, int E, int k,
                  int32_t* __restrict__ ids, float* __restrict__ wts) {
    const int lane = threadIdx.x % kWave;
    const int t = blockIdx.x * kTopkWavesPerBlock + threadIdx.x / kWave;
    if (t >= T) return;
    const float* row = logits + (int64_t)t * E;

    float v[kMaxPerLane];
    uint32_t taken = 0;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; i++) {
        int e = lane + i * kWave;
        v[i] = (e < E) ? row[e] : -INFINITY;
        if (e >= E) taken |= 1u << i;
    }
    float my_logit = -INFINITY;
    int my_id = 0;
    float top = 0.f;
    for (int r = 0; r < k; r++) {
        // best untaken candidate of this lane
        float bv = -INFINITY;
        int bi = INT_MAX;
#pragma unroll
        for (int i = 0; i < kMaxPerLane; i++) {
            int e = lane + i * kWave;
            if (!(taken & (1u << i)) && beats(v[i], e, bv, bi)) {
                bv = v[i];
                bi = e;
            }
        }
        // wave-wide arg-max by butterfly; every lane ends with the winner
#pragma unroll
        for (int m = 1; m < kWave; m <<= 1) {
            float ov = __shfl_xor(bv, m, kWave);
            int oi = __shfl_xor(bi, m, kWave);
            if (beats(ov, oi, bv, bi)) {
                bv = ov;
                bi = oi;
            }
        }
        if (r == 0) top = bv;
        // the owner marks it taken
        if (bi % kWave == lane) taken |= 1u << (bi / kWave);
        if (lane == r) {
            my_logit = bv;
            my_id = bi;
        }
    }
    // renormalised softmax over the k chosen logits
    float p = (lane < k) ? __expf(my_logit - top) : 0.f;
    float s = p;
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) s += __shfl_xor(s, m, kWave);
    if (lane < k) {
        ids[(int64_t)t * k + lane] = my_id;
        wts[(int64_t)t * k + lane] = p / s;
    }
}

constexpr int kSortThreads = 1024;
constexpr int kSortLdsInts = 16384;  // 64 KiB of per-range histograms

__global__ void __launch_bounds__(kSortThreads)
route_sort_kernel(const int32_t* __restrict__ ids, int S, int E, int32_t* __restrict__ counts,
                  int32_t* __restrict__ offsets, int32_t* __restrict__ sorted,
                  int32_t* __restrict__ pos, int32_t* __restrict__ gemv_list,
                  int32_t* __restrict__ mfma_list, int32_t* __restrict__ meta,
                  int gemv_max_tokens, int path) {
    __shared__ int32_t hist[kSortLdsInts];
    __shared__ int32_t s_cnt[kMaxExperts];
    __shared__ int32_t s_off[kMaxExperts + 1];
    __shared__ int32_t s_ngemv, s_nmfma;
    const int tid = threadIdx.x;

    // number of ranges R (power of two): R*E ints fit in LDS, R <= threads, R <= S
    int R = 1;
    while (R * 2 <= kSortThreads && R * 2 * E <= kSortLdsInts && R * 2 <= S) R *= 2;
    const int L = (S + R - 1) / R;  // slots per range

    for (int i = tid; i < R * E; i += kSortThreads) hist[i] = 0;
    if (tid == 0) {
        s_ngemv = 0;
        s_nmfma = 0;
    }
    __syncthreads();
    // 1. per-range histogram (each range owned by one thread: no atomics)
    if (tid < R) {
        int s0 = tid * L, s1 = min(S, s0 + L);
        for (int s = s0; s < s1; s++) hist[tid * E + ids[s]]++;
    }
    __syncthreads();
    // 2. per expert: exclusive scan over ranges
    for (int e = tid; e < E; e += kSortThreads) {
        int run = 0;
        for (int r = 0; r < R; r++) {
            int c = hist[r * E + e];
            hist[r * E + e] = run;
            run += c;
        }
        s_cnt[e] = run;
        counts[e] = run;
    }
    __syncthreads();
    // 3. exclusive scan over experts (E <= 1024: one wave, chunks of 64)
    if (tid < kWave) {
        int carry = 0;
        for (int base = 0; base < E; base += kWave) {
            int e = base + tid;
            int c = (e < E) ? s_cnt[e] : 0;
            int incl = c;
#pragma unroll
            for (int d = 1; d < kWave; d <<= 1) {
                int o = __shfl_up(incl, d, kWave);
                if (tid >= d) incl += o;
            }
            if (e < E) s_off[e] = carry + incl - c;
            carry += __shfl(incl, kWave - 1, kWave);
        }
        if (tid == 0) s_off[E] = carry;
    }
    __syncthreads();
    for (int e = tid; e <= E; e += kSortThreads) offsets[e] = s_off[e];
    // 4. stable scatter: each range walks its slots in order
    if (tid < R) {
        int s0 = tid * L, s1 = min(S, s0 + L);
        for (int s = s0; s < s1; s++) {
            int e = ids[s];
            int p = s_off[e] + hist[tid * E + e]++;
            sorted[p] = s;
            pos[s] = p;
        }
    }
    // 5. active experts, heaviest first (ties: lower index first), split by path
    for (int e = tid; e < E; e += kSortThreads) {
        int c = s_cnt[e];
        if (c == 0) continue;
        bool to_gemv = (path == 1) || (path == 0 && c <= gemv_max_tokens);
        int rank = 0;
        for (int f = 0; f < E; f++) {
            int cf = s_cnt[f];
            if (cf == 0) continue;
            bool f_gemv = (path == 1) || (path == 0 && cf <= gemv_max_tokens);
            if (f_gemv != to_gemv) continue;
            if (cf > c || (cf == c && f < e)) rank++;
        }
        if (to_gemv) {
            gemv_list[rank] = e;
            atomicAdd(&s_ngemv, 1);
        } else {
            mfma_list[rank] = e;
            atomicAdd(&s_nmfma, 1);
        }
    }
    __syncthreads();
    if (tid == 0) {
        meta[kMetaNumGemv] = s_ngemv;
        meta[kMetaNumMfma] = s_nmfma;
    }
}

}  // namespace

hipError_t launch_route(const float* logits, int T, int E, int k, const Workspace& ws,
                        int gemv_max_tokens, int path, hipStream_t stream) {
    int blocks = (T + kTopkWavesPerBlock - 1) / kTopkWavesPerBlock;
    route_topk_kernel<<<blocks, kTopkWavesPerBlock * kWave, 0, stream>>>(logits, T, E, k, ws.ids,
                                                                          ws.wts);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    route_sort_kernel<<<1, kSortThreads, 0, stream>>>(ws.ids, T * k, E, ws.counts, ws.offsets,
                                                      ws.sorted, ws.pos, ws.gemv_list,
                                                      ws.mfma_list, ws.meta, gemv_max_tokens,
                                                      path);
    return hipGetLastError();
}

}  // namespace moe
