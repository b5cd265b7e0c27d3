// route_rank.h -- top-k by rank counting, shared by the routing kernels and
// the self-routed expert GEMMs.
//
// Routing is top-k over fp32 router logits with a softmax renormalised over
// the chosen experts (the problem statement of the layer: route each token
// to its top-k experts, then combine their outputs with those weights).
// The rank of expert e for token t is the number of experts that beat it
// (larger logit, or equal logit and lower index); ranks 0..k-1 are the
// chosen slots, in slot order.  For finite logits the ranks of one token are
// a permutation of 0..E-1, so every slot gets exactly one expert.  Ranks
// are compare-only, hence the same bits wherever they are computed.
#pragma once

#include <math.h>

#include "moe_internal.h"

namespace moe {

// a beats b: larger logit, or equal logit and lower expert index
__device__ inline bool beats(float av, int ai, float bv, int bi) {
    return av > bv || (av == bv && ai < bi);
}

// Rank-count top-k of the tokens [t0, t0+nt) whose logits sit in LDS
// (lg[i*E + e] for token t0+i).  sel_id/sel_l [nt*k] are LDS scratch.
// Writes ids and weights of those tokens: w[t, j] = exp(l_j - l_0) / sum_q
// exp(l_q - l_0) over the chosen logits l_0 >= l_1 >= ..., summed in slot
// order.  Uses every thread of the block.  PUBLISH: agent-coherent stores,
// for readers on other XCDs in the same launch.
template <bool PUBLISH = false>
__device__ inline void topk_tokens(const float* lg, int nt, int t0, int E, int k, int* sel_id,
                                   float* sel_l, int32_t* ids, float* wts) {
    const int tid = threadIdx.x, nthr = blockDim.x;
    for (int i = tid; i < nt * k; i += nthr) {
        sel_id[i] = i % k;  // defined even if NaN logits leave a rank unfilled
        sel_l[i] = -INFINITY;
    }
    __syncthreads();
    for (int p = tid; p < nt * E; p += nthr) {
        const int i = p / E, e = p % E;
        const float* row = lg + i * E;
        const float v = row[e];
        int rank = 0;
        for (int f = 0; f < E; f++) rank += beats(row[f], f, v, e) ? 1 : 0;
        if (rank < k) {
            sel_id[i * k + rank] = e;
            sel_l[i * k + rank] = v;
        }
    }
    __syncthreads();
    for (int p = tid; p < nt * k; p += nthr) {
        const int i = p / k, j = p % k;
        const float top = sel_l[i * k];
        float s = 0.f;
        for (int q = 0; q < k; q++) s += __expf(sel_l[i * k + q] - top);
        const int64_t o = (int64_t)(t0 + i) * k + j;
        const float wv = __expf(sel_l[p] - top) / s;
        if constexpr (PUBLISH) {
            __hip_atomic_store(&ids[o], sel_id[p], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&wts[o], wv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            ids[o] = sel_id[p];
            wts[o] = wv;
        }
    }
}

// The tokens of a layer of T <= 16 tokens that choose expert e, computed
// by one wave on its own from the router logits [T, E] (no routing pass).
// The (token, 64-expert chunk) pairs are taken 16 at a time: lane l loads
// expert 64*chunk + l of the token's row (one coalesced load per pair) and
// e's own logit, and a ballot counts the experts that beat e; the count
// goes to lane t, which ends with the rank of e for token t.  Returns the
// number m of tokens with rank < k; lane c (c = lane % 16) gets in *slot
// the slot t*k + rank of the c-th of them in ascending token order (lanes
// c >= m: the last one's).  Every wave gets the same result.
__device__ inline int expert_slots(const float* __restrict__ logits, int T, int E, int k, int e,
                                   int* slot) {
    const int lane = threadIdx.x % kWave;
    const int nch = (E + kWave - 1) / kWave, npairs = T * nch;
    int my_rank = 0;  // lane t < T: rank of e for token t
    for (int p0 = 0; p0 < npairs; p0 += 16) {
        float v[16], ve[16];
        int t = p0 / nch, ch = p0 % nch;
#pragma unroll
        for (int i = 0; i < 16; i++) {  // loads first: one latency per batch
            const bool ok = p0 + i < npairs;
            const int f = ch * kWave + lane;
            v[i] = ok && f < E ? logits[(int64_t)t * E + f] : 0.f;
            ve[i] = ok ? logits[(int64_t)t * E + e] : 0.f;
            if (++ch == nch) {
                ch = 0;
                t++;
            }
        }
        t = p0 / nch;
        ch = p0 % nch;
#pragma unroll
        for (int i = 0; i < 16; i++) {
            if (p0 + i >= npairs) break;
            const int f = ch * kWave + lane;
            const int n = __popcll(__ballot(f < E && beats(v[i], f, ve[i], e)));
            my_rank += lane == t ? n : 0;
            if (++ch == nch) {
                ch = 0;
                t++;
            }
        }
    }
    const uint64_t chosen = __ballot(lane < T && my_rank < k);  // bit t: token t
    const int m = __popcll(chosen);
    // lane c: the c-th chosen token (the lowest set bit after dropping c);
    // lanes c >= m take the last one, so every lane holds a real slot
    uint64_t rest = chosen;
    for (int i = 0; i < min(lane % 16, m - 1); i++) rest &= rest - 1;
    const int src = rest ? __builtin_ctzll(rest) : 0;
    const int rank = __builtin_amdgcn_ds_bpermute(src * 4, my_rank);
    *slot = src * k + rank;
    return m;
}

}  // namespace moe
