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
// Top-k is computed by rank counting: the rank of expert e for token t is
// the number of experts that beat it (larger logit, or equal logit and lower
// index); ranks 0..k-1 are the chosen slots.  Every (t, e) pair is ranked
// independently, so there is no serial reduction chain.  The sort builds
// per-range histograms in LDS, scans them, and scatters each range in slot
// order, which makes the order inside an expert ascending and the whole
// result deterministic.  Selection, counts, offsets and order are integer or
// compare-only, hence bit-exact; only the weights use exp.
//
// Small layers (T*E <= kFusedMaxPairs) route in one workgroup (one
// launch); larger ones use a grid for top-k and a multi-block counting sort
// (per-block histograms, one scan, per-block stable scatter).  Both also
// reset the per-(token, column tile) combine counters and the unit queue
// of the single-launch expert layer.
#include <float.h>
#include <limits.h>

#include "route_rank.h"

namespace moe {
namespace {

constexpr int kRouteThreads = 1024;
constexpr int kFusedPairs = 12288;    // logits held in LDS by the single-workgroup kernel
constexpr int kFusedMaxPairs = 4096;  // T*E routed by the single-workgroup kernel
static_assert(kFusedMaxPairs <= kFusedPairs, "the single-workgroup route holds T*E logits in LDS");
constexpr int kSlotBlock = kRouteSlotBlock;
constexpr int kTopkThreads = 256;
constexpr int kSortLdsInts = 12288;   // per-range histograms

// Inclusive prefix sum over a wave64 with DPP row shifts and row broadcasts.
__device__ inline int wave_incl_scan(int v) {
    const int lane = threadIdx.x % kWave;
    int t;
    t = __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
    v += t;
    t = __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
    v += t;
    t = __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
    v += t;
    t = __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
    v += t;
    t = __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
    v += t;
    t = __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
    v += t;
    (void)lane;
    return v;
}

// s_off[e] = exclusive prefix sum of s_cnt over experts, s_off[E] = total
// (LDS arrays); one wave, 64 experts at a time.
__device__ inline void scan_experts(int E, const int* s_cnt, int* s_off) {
    const int tid = threadIdx.x;
    if (tid < kWave) {
        int carry = 0;
        for (int base = 0; base < E; base += kWave) {
            const int e = base + tid;
            const int c = (e < E) ? s_cnt[e] : 0;
            const int incl = wave_incl_scan(c);
            if (e < E) s_off[e] = carry + incl - c;
            carry += __builtin_amdgcn_readlane(incl, kWave - 1);
        }
        if (tid == 0) s_off[E] = carry;
    }
}

// Active-expert lists in ascending expert index, compacted with wave
// scans: the GEMV list and the MFMA list; and the MFMA path's items
// (expert, first row in sorted order, tokens), ceil(c / item_tok) per expert
// of equal numbers of 16-token tiles (+-1): item q of an expert with `tiles`
// tiles over `groups` items has per + (q < extra) tiles from tile q*per +
// min(q, extra) (per = tiles / groups, extra = tiles % groups).
//
// Items are ordered by expert, heaviest expert (most tiles) first, ties by
// expert index, and an expert's items stay adjacent: the heaviest work is
// dispatched first instead of landing in the tail of the grid, and the
// workgroups that stream the same expert's weights for its several items
// run at about the same time (their re-reads then hit in cache).  The order
// of items changes no result: each output element is computed by one item,
// and the combine sums in slot order.  s_cnt/s_off: the per-expert counts
// and exclusive offsets, in LDS.  Writes the list lengths to meta.  Called
// by every thread of one block.
__device__ void build_lists(int E, const Workspace& ws, int gemv_max_tokens, int path, int item_tok,
                            const int* s_cnt, const int* s_off) {
    __shared__ int s_n[3];
    __shared__ int s_key[kMaxExperts];   // tiles of an MFMA-path expert, -1 otherwise
    __shared__ int s_rank[kMaxExperts];  // position of the expert in item order
    __shared__ int s_base[kMaxExperts];  // by rank: the expert's items, then their first index
    const int tid = threadIdx.x, nthr = blockDim.x;
    auto on_gemv = [&](int c) { return c > 0 && ((path == 1) || (path == 0 && c <= gemv_max_tokens)); };
    for (int e = tid; e < E; e += nthr) {
        const int c = s_cnt[e];
        s_key[e] = (c > 0 && !on_gemv(c)) ? (c + 15) / 16 : -1;
    }
    __syncthreads();
    // rank among the MFMA-path experts: (tiles desc, index asc)
    for (int e = tid; e < E; e += nthr) {
        const int ke = s_key[e];
        if (ke < 0) continue;
        int r = 0;
        for (int f = 0; f < E; f++) {
            const int kf = s_key[f];
            r += (kf > ke || (kf == ke && f < e)) ? 1 : 0;
        }
        s_rank[e] = r;
        s_base[r] = (s_cnt[e] + item_tok - 1) / item_tok;  // the expert's items
    }
    __syncthreads();
    if (tid < kWave) {
        // the lists, and the exclusive scan of items over ranks
        int n_g = 0, n_m = 0, n_items = 0;
        for (int base = 0; base < E; base += kWave) {
            const int e = base + tid;
            const int c = (e < E) ? s_cnt[e] : 0;
            const bool g = on_gemv(c);
            const bool m = c > 0 && !g;
            const int ig = wave_incl_scan(g ? 1 : 0);
            const int im = wave_incl_scan(m ? 1 : 0);
            if (g) ws.gemv_list[n_g + ig - 1] = e;
            if (m) ws.mfma_list[n_m + im - 1] = e;
            n_g += __builtin_amdgcn_readlane(ig, kWave - 1);
            n_m += __builtin_amdgcn_readlane(im, kWave - 1);
        }
        for (int base = 0; base < n_m; base += kWave) {
            const int r = base + tid;
            const int n = r < n_m ? s_base[r] : 0;
            const int incl = wave_incl_scan(n);
            if (r < n_m) s_base[r] = n_items + incl - n;
            n_items += __builtin_amdgcn_readlane(incl, kWave - 1);
        }
        if (tid == 0) {
            s_n[0] = n_g;
            s_n[1] = n_m;
            s_n[2] = n_items;
        }
    }
    __syncthreads();
    // each MFMA-path expert writes its items from its first index
    for (int e = tid; e < E; e += nthr) {
        if (s_key[e] < 0) continue;
        const int c = s_cnt[e];
        const int groups = (c + item_tok - 1) / item_tok;
        const int tiles = (c + 15) / 16, per = tiles / groups, extra = tiles % groups;
        int slot = s_base[s_rank[e]];
        for (int q = 0; q < groups; q++) {
            const int t0 = q * per + min(q, extra);
            const int nt = per + (q < extra ? 1 : 0);
            ws.mfma_items[slot++] = make_int4(e, s_off[e] + 16 * t0, min(16 * nt, c - 16 * t0), 0);
        }
    }
    if (tid == 0) {
        ws.meta[kMetaNumGemv] = s_n[0];
        ws.meta[kMetaNumMfma] = s_n[1];
        ws.meta[kMetaNumMfmaItems] = s_n[2];
    }
}

// Stable counting sort of the S slots by expert (ids[s] = expert of slot
// s, in LDS or global memory), the active-expert lists, and the reset of
// the combine counters.  One workgroup.
__device__ void sort_slots(const int32_t* ids, int S, int E, int T, const Workspace& ws,
                           int gemv_max_tokens, int path, int item_tok, int* hist, int* s_cnt,
                           int* s_off) {
    const int tid = threadIdx.x, nthr = blockDim.x;
    // R ranges (power of two) of L consecutive slots: R ~ sqrt(S), R*E fits in LDS
    int R = 1;
    while (R * 2 <= nthr && R * 2 * E <= kSortLdsInts && R * R * 4 <= S) R *= 2;
    const int L = (S + R - 1) / R;

    for (int i = tid; i < R * E; i += nthr) hist[i] = 0;
    // reset the combine counters of the down kernels (sized for the finest tile)
    for (int i = tid; i < T * (int)(ws.H / kMfmaDownRows); i += nthr) ws.tile_done[i] = 0;
    // and the unit queue and per-item gate_up counts of the single-launch layer
    for (int i = tid; i < kQueueHead; i += nthr) ws.queue[i] = 0;
    for (int i = tid; i < kGoLines; i += nthr) ws.queue[kQueueGo + i * kGoStride] = 0;
    for (int i = tid; i < ws.max_items; i += nthr) ws.gu_done[(int64_t)i * kLineInts] = 0;
    __syncthreads();
    if (tid < R) {  // 1. per-range histogram
        const int s0 = tid * L, s1 = min(S, s0 + L);
        for (int s = s0; s < s1; s++) hist[tid * E + ids[s]]++;
    }
    __syncthreads();
    for (int e = tid; e < E; e += nthr) {  // 2. per expert: exclusive scan over ranges
        int run = 0;
        for (int r = 0; r < R; r++) {
            const int c = hist[r * E + e];
            hist[r * E + e] = run;
            run += c;
        }
        s_cnt[e] = run;
        ws.counts[e] = run;
    }
    __syncthreads();
    scan_experts(E, s_cnt, s_off);  // 3. exclusive scan over experts
    __syncthreads();
    for (int e = tid; e <= E; e += nthr) ws.offsets[e] = s_off[e];
    if (tid < R) {  // 4. stable scatter: each range walks its slots in order
        const int s0 = tid * L, s1 = min(S, s0 + L);
        for (int s = s0; s < s1; s++) {
            const int e = ids[s];
            const int p = s_off[e] + hist[tid * E + e]++;
            ws.sorted[p] = s;
            ws.pos[s] = p;
        }
    }
    build_lists(E, ws, gemv_max_tokens, path, item_tok, s_cnt, s_off);
}

__global__ void __launch_bounds__(kRouteThreads)
route_fused_kernel(const float* __restrict__ logits, int T, int E, int k, Workspace ws,
                   int gemv_max_tokens, int path, int item_tok) {
    __shared__ float lg[kFusedPairs];
    __shared__ int sel_id[kRouteThreads];
    __shared__ float sel_l[kRouteThreads];
    __shared__ int hist[kSortLdsInts];
    __shared__ int s_cnt[kMaxExperts];
    __shared__ int s_off[kMaxExperts + 1];
    for (int i = threadIdx.x; i < T * E; i += blockDim.x) lg[i] = logits[i];
    __syncthreads();
    topk_tokens(lg, T, 0, E, k, sel_id, sel_l, ws.ids, ws.wts);
    __syncthreads();
    // the ids of all T*k slots are still in LDS (sel_id), read them there
    sort_slots(sel_id, T * k, E, T, ws, gemv_max_tokens, path, item_tok, hist, s_cnt, s_off);
}

// ---- larger layers: top-k over a grid, then a stable counting sort over
// blocks of kSlotBlock slots (per-block histograms, one scan, per-block
// scatter), four launches whose work all scales out.

// grid over token groups: each block ranks tokens [t0, t0 + nt) and resets
// their combine counters
__global__ void __launch_bounds__(kTopkThreads)
route_topk_kernel(const float* __restrict__ logits, int T, int E, int k, int tokens_per_block,
                  int32_t* __restrict__ ids, float* __restrict__ wts, int32_t* __restrict__ tile_done,
                  int done_per_token) {
    extern __shared__ float dyn[];
    const int t0 = blockIdx.x * tokens_per_block;
    const int nt = min(tokens_per_block, T - t0);
    float* lg = dyn;
    int* sel_id = reinterpret_cast<int*>(dyn + tokens_per_block * E);
    float* sel_l = dyn + tokens_per_block * E + tokens_per_block * k;
    for (int i = threadIdx.x; i < nt * done_per_token; i += blockDim.x)
        tile_done[(int64_t)t0 * done_per_token + i] = 0;
    for (int i = threadIdx.x; i < nt * E; i += blockDim.x) lg[i] = logits[(int64_t)t0 * E + i];
    __syncthreads();
    topk_tokens(lg, nt, t0, E, k, sel_id, sel_l, ids, wts);
}

// bhist[b][e] = slots of block b (slots [b*kSlotBlock, ...)) routed to e
__global__ void __launch_bounds__(kSlotBlock)
route_hist_kernel(const int32_t* __restrict__ ids, int S, int E, int32_t* __restrict__ bhist) {
    __shared__ int h[kMaxExperts];
    for (int e = threadIdx.x; e < E; e += kSlotBlock) h[e] = 0;
    __syncthreads();
    const int s = blockIdx.x * kSlotBlock + threadIdx.x;
    if (s < S) atomicAdd(&h[ids[s]], 1);  // counts only: order-free
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kSlotBlock) bhist[(int64_t)blockIdx.x * E + e] = h[e];
}

// One block: counts, offsets, the first sorted position of every (block,
// expert) pair (bhist rewritten in place), and the lists and items.
__global__ void __launch_bounds__(kRouteThreads)
route_scan_kernel(int nblk, int E, Workspace ws, int32_t* __restrict__ bhist, int gemv_max_tokens,
                  int path, int item_tok) {
    __shared__ int s_cnt[kMaxExperts];
    __shared__ int s_off[kMaxExperts + 1];
    const int tid = threadIdx.x, nthr = blockDim.x;
    for (int e = tid; e < E; e += nthr) {  // per expert: exclusive scan over blocks
        // 16 blocks' counts at a time, loaded before any is rewritten: one
        // memory latency per 16 blocks instead of one per block
        int run = 0;
        for (int b0 = 0; b0 < nblk; b0 += 16) {
            int c[16];
#pragma unroll
            for (int i = 0; i < 16; i++) c[i] = b0 + i < nblk ? bhist[(int64_t)(b0 + i) * E + e] : 0;
#pragma unroll
            for (int i = 0; i < 16; i++) {
                if (b0 + i < nblk) bhist[(int64_t)(b0 + i) * E + e] = run;
                run += c[i];
            }
        }
        s_cnt[e] = run;
        ws.counts[e] = run;
    }
    for (int i = tid; i < kQueueHead; i += nthr) ws.queue[i] = 0;
    for (int i = tid; i < kGoLines; i += nthr) ws.queue[kQueueGo + i * kGoStride] = 0;
    for (int i = tid; i < ws.max_items; i += nthr) ws.gu_done[(int64_t)i * kLineInts] = 0;
    __syncthreads();
    scan_experts(E, s_cnt, s_off);
    __syncthreads();
    for (int e = tid; e <= E; e += nthr) ws.offsets[e] = s_off[e];
    for (int i = tid; i < nblk * E; i += nthr) bhist[i] += s_off[i % E];
    build_lists(E, ws, gemv_max_tokens, path, item_tok, s_cnt, s_off);
}

// Stable scatter: slot s goes to bhist[b][e] + (slots before it in its
// block routed to the same expert).
__global__ void __launch_bounds__(kSlotBlock)
route_scatter_kernel(const int32_t* __restrict__ ids, int S, int E,
                     const int32_t* __restrict__ bhist, int32_t* __restrict__ sorted,
                     int32_t* __restrict__ pos) {
    __shared__ int sid[kSlotBlock];
    const int s = blockIdx.x * kSlotBlock + threadIdx.x;
    const int e = s < S ? ids[s] : -1;
    sid[threadIdx.x] = e;
    __syncthreads();
    if (s < S) {
        int rank = 0;
        for (int i = 0; i < (int)threadIdx.x; i++) rank += sid[i] == e ? 1 : 0;
        const int p = bhist[(int64_t)blockIdx.x * E + e] + rank;
        sorted[p] = s;
        pos[s] = p;
    }
}

// Slot lists of the self-routed layer: wave w of block b ranks expert
// e = 4b + w for every token (expert_slots) and writes m and the slots.
__global__ void __launch_bounds__(kWave * 4)
slot_lists_kernel(const float* __restrict__ logits, int T, int E, int k,
                  int32_t* __restrict__ lists) {
    const int e = blockIdx.x * 4 + threadIdx.x / kWave, lane = threadIdx.x % kWave;
    if (e >= E) return;
    int slot;
    const int m = expert_slots(logits, T, E, k, e, &slot);
    int32_t* list = lists + e * kSlotListInts;
    if (lane < m) list[1 + lane] = slot;
    if (lane == 0) list[0] = m;
}

}  // namespace

hipError_t launch_slot_lists(const GemmArgs& a, hipStream_t stream) {
    slot_lists_kernel<<<(a.E + 3) / 4, kWave * 4, 0, stream>>>(a.logits, a.T, a.E, a.k, a.slot_lists);
    return hipGetLastError();
}

hipError_t launch_route(const float* logits, int T, int E, int k, const Workspace& ws,
                        int gemv_max_tokens, int path, int item_tok, hipStream_t stream) {
    if ((int64_t)T * E <= kFusedMaxPairs && T * k <= kRouteThreads) {
        route_fused_kernel<<<1, kRouteThreads, 0, stream>>>(logits, T, E, k, ws,
                                                            gemv_max_tokens, path, item_tok);
        return hipGetLastError();
    }
    const int S = T * k;
    const int tpb = E >= kTopkThreads ? 1 : kTopkThreads / E;
    const int blocks = (T + tpb - 1) / tpb;
    const size_t lds = (size_t)tpb * (E + 2 * k) * 4;
    route_topk_kernel<<<blocks, kTopkThreads, lds, stream>>>(logits, T, E, k, tpb, ws.ids, ws.wts,
                                                             ws.tile_done,
                                                             (int)(ws.H / kMfmaDownRows));
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int nblk = (S + kSlotBlock - 1) / kSlotBlock;
    route_hist_kernel<<<nblk, kSlotBlock, 0, stream>>>(ws.ids, S, E, ws.bhist);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    route_scan_kernel<<<1, kRouteThreads, 0, stream>>>(nblk, E, ws, ws.bhist, gemv_max_tokens, path,
                                                       item_tok);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    route_scatter_kernel<<<nblk, kSlotBlock, 0, stream>>>(ws.ids, S, E, ws.bhist, ws.sorted, ws.pos);
    return hipGetLastError();
}

}  // namespace moe
