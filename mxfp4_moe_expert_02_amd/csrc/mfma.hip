// mfma.hip -- MXFP4 expert GEMMs on the bf16 matrix cores of gfx950, over
// weights prepacked into the MFMA tile layout.
//
// The weight bytes are the cost of this layer (the pages quantise the MoE
// experts to 4 bits because the decode of a 1T model is bound by weight
// I/O: bjdmk.com.cn news page, co-design section; yifor-blog digest,
// memory-bandwidth section).  The VALU path (gemv.hip) spends about two
// VALU instructions per weight element on decode and dot products; here the
// products and the K reduction go to v_mfma_f32_16x16x32_bf16 and the VALU
// only decodes: one v_cvt_scalef32_pk_bf16_fp4 per two elements, with the
// E8M0 block scale applied by the same instruction (E2M1 * 2^k is exact in
// bf16 for every scale code 1..254).  Activations stay bf16 and
// accumulation fp32, as in the VALU path.
//
// Tile layout (built once by moe_mxfp4_prepack, see prepack.hip): a matrix
// is cut into 64-row quads (four 16-row groups) and 128-column chunks (four
// MX blocks).  For one (quad, chunk) the 4 KB of packed codes are stored as
// [group rg][lane l][16 bytes], lane l = r + 16 g holding block g of row r
// of group rg, and the 256 scale bytes as [lane l][group rg].  One 16-byte
// load per lane per group is then a contiguous 1 KB wave load already in
// MFMA operand order, and one dword load per lane brings the lane's four
// scales.  gate_up quads pair rows: groups 0,1 are gate rows 32q..32q+31 and
// groups 2,3 the up rows I+32q..I+32q+31, so SiLU(gate)*up needs no data
// exchange.
//
// One 16x16x32 MFMA: A = 16 weight rows x 32 k (lane (r, g) supplies word q
// = elements 8q..8q+7 of its block), B = 32 k x 16 tokens (lane (c, g)
// supplies the same 8 k of token c, loaded from global memory: every tile of
// the expert reads the same token rows, so these are L1/L2 hits), D = 16
// rows x 16 tokens (lane (c, g) holds rows 4g..4g+3 of token c).  The 4
// waves of a workgroup split the chunks in four ranges and add their
// accumulators through LDS at the end.  Items come from the route: (expert,
// first row in sorted order, tokens) with up to 16 tokens each (wider items
// go to mfma_wide.hip).  The quad routine is written for NT column tiles;
// these kernels use NT = 1.
#include "mfma_items.h"
#include "route_rank.h"

namespace moe {
namespace {

// The shared expert as launches of its own (the VALU path and the
// single-launch layer, whose kernels do not take its blocks; bf16
// activations): 64-token tiles once the layer has 64 tokens (a quad's
// weights are then decoded once per 64 tokens), else 16.
template <int NT, typename X>
__global__ void __launch_bounds__(kMfmaThreads)
__attribute__((amdgpu_waves_per_eu(kMfmaWavesPerEu)))
shared_gate_up_kernel(GemmArgs a) {
    __shared__ f32x4_t red[kRedGateUp * NT];
    shared_gate_up_block<NT, X>(a, blockIdx.x, red);
}

template <int NT>
__global__ void __launch_bounds__(kMfmaThreads)
__attribute__((amdgpu_waves_per_eu(kMfmaWavesPerEu)))
shared_down_kernel(GemmArgs a) {
    __shared__ f32x4_t red[kRedDown * NT];
    shared_down_block<NT>(a, blockIdx.x, red);
}

// gate_up: blockIdx.x = item * quads + quad; quad q = gate rows 32q..32q+31
// (groups 0, 1) with up rows I+32q..I+32q+31 (groups 2, 3).  WIDE: items of
// up to kMfmaItemTok tokens (1..4 column tiles of 16); otherwise items of
// at most 16 tokens, compiled without the wider cases (fewer registers).
__global__ void __launch_bounds__(kMfmaThreads)
__attribute__((amdgpu_waves_per_eu(kMfmaWavesPerEu)))
mfma_gate_up_kernel(GemmArgs a) {
    __shared__ f32x4_t red[kRedGateUp];
    const int quads = a.I / 32;
    int b = blockIdx.x;
    if (a.sh_wgu) {  // the shared expert's blocks first (16-token tiles)
        const int nb = shared_blocks(quads, (a.T + 15) / 16);
        if (b < nb) {
            shared_gate_up_block<1, XB>(a, b, red);
            return;
        }
        b -= nb;
    }
    const int item = b / quads, quad = b % quads;
    if (item >= uniform(a.meta[kMetaNumMfmaItems])) return;
    const int4 it = a.items[item];
    const int e = uniform(it.x), row0 = uniform(it.y), m = uniform(it.z);
    gate_up_item<1, W4, XB>(a, quad, a.wgu + (int64_t)e * (a.I / 32) * (a.H / 128) * 4096,
                            a.sgu + (int64_t)e * (a.I / 32) * (a.H / 128) * 256, SortedRows{row0, m}, red);
}

// down: a workgroup takes two quads (output rows 64q..64q+63), each split
// in two K halves over two waves; blockIdx.x = item * ceil(quads / 2) +
// pair.  The wave holding a quad's summed accumulator writes its y rows;
// the combine kernel reads them after this kernel.
__global__ void __launch_bounds__(kMfmaThreads)
__attribute__((amdgpu_waves_per_eu(3)))
mfma_down_kernel(GemmArgs a) {
    __shared__ f32x4_t red[kRedDown];
    const int quads = a.H / 64, pairs = (quads + 1) / 2;
    int b = blockIdx.x;
    if (a.sh_wdn) {  // the shared expert's blocks first (16-token tiles)
        const int nb = shared_blocks(pairs, (a.T + 15) / 16);
        if (b < nb) {
            shared_down_block<1>(a, b, red);
            return;
        }
        b -= nb;
    }
    const int item = b / pairs, pair = b % pairs;
    if (item >= uniform(a.meta[kMetaNumMfmaItems])) return;
    const int4 it = a.items[item];
    const int e = uniform(it.x), row0 = uniform(it.y), m = uniform(it.z);
    down_item<1, false, W4>(a, pair, a.wdn + (int64_t)e * (a.H / 64) * (a.I / 128) * 4096,
                                a.sdn + (int64_t)e * (a.H / 64) * (a.I / 128) * 256,
                                SortedRows{row0, m}, red);
}

// ---- self-routed layer (up to kSelfMaxTok tokens): no routing pass.  The
// pages name the launches, synchronisations and global-memory round trips
// at operator boundaries as the fixed costs that surface once a step takes
// microseconds (tilert.ai blog, first leap; HyperAI transcript, system
// efficiency); a routing pass ahead of the GEMMs, over a few tokens, is
// such a cost: a kernel of its own and a boundary.  Here every workgroup ranks
// its own expert for each token from the router logits (expert_slots: one
// round of loads, compares and a ballot, about the latency of the item
// load it replaces), so gate_up starts streaming weights at once.  The
// GEMM arithmetic and its order are those of the routed kernels, and the
// weights come from the same rank-count code, so the output has the same
// bits as the routed layer's.

// LDS of the weight pass: the logits, then the chosen ids and logits
constexpr int kSelfLdsFloats = kSelfMaxPairs + 2 * kSelfMaxTok * kMaxTopK;

// The rows of expert e for a self-routed GEMM workgroup: from its slot list
// (one scalar load of m before any weight load; the slots are read after
// the first weight loads are issued), or ranked here from the logits.
template <bool LISTS>
struct SelfRows;
template <>
struct SelfRows<true> {
    static __device__ ListRows get(const GemmArgs& a, int e) {
        const int32_t* list = a.slot_lists + e * kSlotListInts;
        return ListRows{uniform(list[0]), list + 1};
    }
};
template <>
struct SelfRows<false> {
    static __device__ SlotRows get(const GemmArgs& a, int e) {
        int slot;
        const int m = uniform(expert_slots(a.logits, a.T, a.E, a.k, e, &slot));
        return SlotRows{m, slot};
    }
};

// blockIdx.x = 0: the routing weights w[t, j] (and expert ids) of every
// slot, for the combine.  With a shared expert, blockIdx.x = 1 + quad for
// its I/32 quads (every token, h rows sh_row0 + t), and the routed blocks
// follow.  Routed block 1 + e * (I/32) + quad: gate_up quad `quad` of
// expert e, for the tokens that chose e, h rows by slot.
template <bool LISTS>
__global__ void __launch_bounds__(kMfmaThreads)
__attribute__((amdgpu_waves_per_eu(kMfmaWavesPerEu)))
self_gate_up_kernel(GemmArgs a) {
    __shared__ __attribute__((aligned(16)))
    float smem[kSelfLdsFloats > 4 * kRedGateUp ? kSelfLdsFloats : 4 * kRedGateUp];
    if (blockIdx.x == 0) {
        const int T = a.T, E = a.E;
        for (int i = threadIdx.x; i < T * E; i += blockDim.x) smem[i] = a.logits[i];
        __syncthreads();
        float* sel_l = smem + T * E;
        int* sel_id = reinterpret_cast<int*>(sel_l + T * a.k);
        topk_tokens(smem, T, 0, E, a.k, sel_id, sel_l, a.route_ids, a.route_wts);
        return;
    }
    const int quads = a.I / 32;
    int b = blockIdx.x - 1;
    if (a.sh_wgu) {  // the shared expert's quads first (the longest workgroups)
        if (b < quads) {
            gate_up_item<1, W8, XB>(a, b, a.sh_wgu, a.sh_sgu, TokenRows{0, a.T, a.sh_row0},
                                    reinterpret_cast<f32x4_t*>(smem));
            return;
        }
        b -= quads;
    }
    const int e = b / quads, quad = b % quads;
    const auto rows = SelfRows<LISTS>::get(a, e);
    if (rows.m == 0) return;  // no token chose e
    gate_up_item<1, W4, XB>(a, quad, a.wgu + (int64_t)e * quads * (a.H / 128) * 4096,
                            a.sgu + (int64_t)e * quads * (a.H / 128) * 256, rows,
                            reinterpret_cast<f32x4_t*>(smem));
}

// blockIdx.x = e * ceil(H/128) + pair: the down quads 2*pair, 2*pair+1 of
// expert e for the tokens that chose it, y rows by slot (after the shared
// expert's ceil(H/128) pairs, if there is one: every token, y rows
// sh_row0 + t).
template <bool LISTS>
__global__ void __launch_bounds__(kMfmaThreads)
__attribute__((amdgpu_waves_per_eu(LISTS ? 3 : 2)))
self_down_kernel(GemmArgs a) {
    __shared__ f32x4_t red[kRedDown];
    const int pairs = (a.H / 64 + 1) / 2;
    int b = blockIdx.x;
    if (a.sh_wdn) {  // the shared expert's quad pairs first
        if (b < pairs) {
            down_item<1, false, W8P>(a, b, a.sh_wdn, a.sh_sdn, TokenRows{0, a.T, a.sh_row0}, red);
            return;
        }
        b -= pairs;
    }
    const int e = b / pairs, pair = b % pairs;
    const auto rows = SelfRows<LISTS>::get(a, e);
    if (rows.m == 0) return;
    down_item<1, false, W4>(a, pair, a.wdn + (int64_t)e * (a.H / 64) * (a.I / 128) * 4096,
                                a.sdn + (int64_t)e * (a.H / 64) * (a.I / 128) * 256, rows, red);
}

constexpr int kFusedWavesPerEu = 2;  // launch bound of the single-launch kernel

// The expert layer after routing in one persistent launch: every workgroup
// dequeues units from one counter, first the gate_up units (item, quad),
// then the down units (item, quad pair), until the queue is exhausted, and
// then the grid combines (grid_combine).  A down unit first waits until
// all I/32 gate_up units of its item are done.
// No wait can deadlock: the units a down unit waits for were dequeued
// before it, by workgroups that are running and never wait themselves.
// The wait is bounded (wait_count) and raises queue[kQueueError] if it ever
// gives up.
//
// Each unit has a workgroup barrier inside (the split-K sum, or the wait),
// which keeps the four waves within one unit of each other; the LDS of the
// sums alternates between two buffers, so no barrier is needed between
// units.  The next unit is dequeued while the current one runs.  Wave 0
// stores a gate_up unit's h (agent-coherent stores) and alone waits for
// them to complete before it counts the unit done for its item; the other
// waves go on with the next unit meanwhile.  Holding a dequeued unit cannot
// block anyone: a workgroup holds a gate_up unit only while running a
// gate_up unit, which never waits.
__global__ void __launch_bounds__(kMfmaThreads)
__attribute__((amdgpu_waves_per_eu(kFusedWavesPerEu)))
mfma_fused_kernel(GemmArgs a) {
    __shared__ f32x4_t red[2][kRedGateUp];
    __shared__ int s_unit[2];
    const int n_items = uniform(a.meta[kMetaNumMfmaItems]);
    const int gu_units = a.I / 32, dn_units = (a.H / 64 + 1) / 2;
    const int n_gu = n_items * gu_units, n_all = n_gu + n_items * dn_units;
    if (threadIdx.x == 0) s_unit[0] = atomicAdd(&a.queue[kQueueNext], 1);
    __syncthreads();
    int n_run = 0;  // units this workgroup ran
    for (int cur = 0;; cur ^= 1) {
        const int u = uniform(s_unit[cur]);
        if (u >= n_all) break;
        n_run++;
        // read by every wave after this unit's barrier
        if (threadIdx.x == 0) s_unit[cur ^ 1] = atomicAdd(&a.queue[kQueueNext], 1);
        if (u < n_gu) {
            const int item = u / gu_units;
            const int4 it = a.items[item];
            const int64_t e = uniform(it.x);
            gate_up_item<1, W4, XB, true>(a, u % gu_units, a.wgu + e * gu_units * (a.H / 128) * 4096,
                                    a.sgu + e * gu_units * (a.H / 128) * 256,
                                    SortedRows{uniform(it.y), uniform(it.z)}, red[cur]);
            if (threadIdx.x < kWave) {  // wave 0 stored the h rows
                __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): they are complete
                if (threadIdx.x == 0) atomicAdd(&a.gu_done[(int64_t)item * kLineInts], 1);
            }
        } else {
            const int v = u - n_gu, item = v / dn_units;
            const int4 it = a.items[item];
            if (threadIdx.x == 0) wait_count(&a.gu_done[(int64_t)item * kLineInts], gu_units, &a.queue[kQueueError]);
            __syncthreads();
            const int64_t e = uniform(it.x);
            down_item<1, true, W4>(a, v % dn_units, a.wdn + e * (a.H / 64) * (a.I / 128) * 4096,
                                       a.sdn + e * (a.H / 64) * (a.I / 128) * 256,
                                       SortedRows{uniform(it.y), uniform(it.z)}, red[cur]);
        }
    }
    grid_combine(a, n_run, n_all, &a.queue[kQueueDone], &a.queue[kQueueGo], &a.queue[kQueueError]);
}

// The same units as one launch of one workgroup per unit (see
// wide_queue_kernel in mfma_wide.hip): each workgroup dequeues one unit --
// gate_up (item, quad), then down (item, quad pair) -- runs it and exits; a
// down unit first waits (bounded) for the I/32 gate_up units of its item,
// dequeued earlier by running workgroups that never wait.  The combine is a
// launch of its own; arithmetic and order are the split launch's.
__global__ void __launch_bounds__(kMfmaThreads)
__attribute__((amdgpu_waves_per_eu(kMfmaWavesPerEu)))
mfma_queue_kernel(GemmArgs a) {
    __shared__ f32x4_t red[kRedGateUp];
    __shared__ int s_unit;
    const int n_items = uniform(a.meta[kMetaNumMfmaItems]);
    const int gu_units = a.I / 32, dn_units = (a.H / 64 + 1) / 2;
    const int n_gu = n_items * gu_units, n_all = n_gu + n_items * dn_units;
    if (threadIdx.x == 0) s_unit = atomicAdd(&a.queue[kQueueNext], 1);
    __syncthreads();
    const int u = uniform(s_unit);
    if (u >= n_all) return;
    if (u < n_gu) {
        const int item = u / gu_units;
        const int4 it = a.items[item];
        const int64_t e = uniform(it.x);
        gate_up_item<1, W4, XB, true>(a, u % gu_units, a.wgu + e * gu_units * (a.H / 128) * 4096,
                                      a.sgu + e * gu_units * (a.H / 128) * 256,
                                      SortedRows{uniform(it.y), uniform(it.z)}, red);
        if (threadIdx.x < kWave) {  // wave 0 stored the h rows
            __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): they are complete
            if (threadIdx.x == 0) atomicAdd(&a.gu_done[(int64_t)item * kLineInts], 1);
        }
    } else {
        const int v = u - n_gu, item = v / dn_units;
        const int4 it = a.items[item];
        if (threadIdx.x == 0) wait_count(&a.gu_done[(int64_t)item * kLineInts], gu_units, &a.queue[kQueueError]);
        __syncthreads();
        const int64_t e = uniform(it.x);
        down_item<1, false, W4>(a, v % dn_units, a.wdn + e * (a.H / 64) * (a.I / 128) * 4096,
                                a.sdn + e * (a.H / 64) * (a.I / 128) * 256,
                                SortedRows{uniform(it.y), uniform(it.z)}, red);
    }
}

constexpr int kSharedWideTok = 64;

// ---- the self-routed layer in one launch.  The pages run a model as one
// persistent engine kernel so that no launch, synchronisation or
// global-memory round trip between operators is left exposed once a step
// takes microseconds (tilert.ai blog, first leap; bjdmk.com.cn news page,
// road to 1000 tokens/s); here the whole expert layer of at most 16 tokens
// -- routing weights, per-expert slot lists, gate_up, down and the combine
// -- is one launch of resident workgroups dequeuing units from one counter,
// in this order:
//   0                the routing weights (rank-count top-k of every token)
//   1 .. L           slot lists of experts 4(u-1) .. 4(u-1)+3, one per wave
//   shared gate_up   (with a shared expert) its I/32 quads over all tokens
//   routed gate_up   (e, quad) for e < E, quad < I/32
//   shared down      (with a shared expert) its quad pairs over all tokens
//   routed down      (e, pair) for e < E, pair < ceil(H/128)
// and then the combine of every output over the whole grid (grid_combine).
// A gate_up unit of e waits until e's list is written; a down unit until
// every gate_up unit of its expert has published h.  Every wait is on units
// dequeued earlier by running workgroups that never wait on later ones, so
// none can deadlock; each is bounded (wait_count) and raises the error flag
// if it ever gives up.  Units of experts no token chose exit after reading
// m = 0.  The arithmetic and its order are those of the split launch (same
// item bodies; the combine's fmaf chain is the combine kernel's), so the
// output has its bits.  The last workgroup to finish the combine clears the
// counters for the next launch (every other workgroup has passed its last
// wait by then).
__device__ inline void wait_flag(const int32_t* count, int need, int32_t* err) {
    if (threadIdx.x == 0) wait_count(count, need, err);
    __syncthreads();
}

__global__ void __launch_bounds__(kMfmaThreads)
__attribute__((amdgpu_waves_per_eu(kFusedWavesPerEu)))
self_fused_kernel(GemmArgs a, int32_t* flags) {
    __shared__ __attribute__((aligned(16))) float s_lg[kSelfLdsFloats];  // the weights unit
    __shared__ f32x4_t red[2][kRedGateUp];
    __shared__ int s_unit[2];
    const int E = a.E, quads = a.I / 32, pairs = (a.H / 64 + 1) / 2;
    const bool sh = a.sh_wgu != nullptr;
    // one line per counter (kLineInts words apart): list ready of expert e,
    // gate_up units done of expert e (index E: the shared expert)
    int32_t* list_ready = flags;
    int32_t* gu_done = flags + (int64_t)(E + 1) * kLineInts;
    int32_t* misc = flags + self_misc_word(E);  // SelfFlags
    int32_t* go = flags + self_go_word(E);
    const int n_lists = (E + 3) / 4;
    const int u_sgu = 1 + n_lists, u_gu = u_sgu + (sh ? quads : 0);
    const int u_sdn = u_gu + E * quads, u_dn = u_sdn + (sh ? pairs : 0);
    const int n_all = u_dn + E * pairs;
    const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
    if (threadIdx.x == 0) s_unit[0] = atomicAdd(&misc[kSelfNext], 1);
    __syncthreads();
    int n_run = 0;  // units this workgroup ran
    for (int cur = 0;; cur ^= 1) {
        const int u = uniform(s_unit[cur]);
        if (u >= n_all) break;
        n_run++;
        if (threadIdx.x == 0) s_unit[cur ^ 1] = atomicAdd(&misc[kSelfNext], 1);
        if (u == 0) {  // the routing weights and ids of every slot (read by the combine)
            for (int i = threadIdx.x; i < a.T * E; i += blockDim.x) s_lg[i] = a.logits[i];
            __syncthreads();
            float* sel_l = s_lg + a.T * E;
            int* sel_id = reinterpret_cast<int*>(sel_l + a.T * a.k);
            topk_tokens<true>(s_lg, a.T, 0, E, a.k, sel_id, sel_l, a.route_ids, a.route_wts);
        } else if (u < u_sgu) {  // slot lists, one expert per wave
            const int e = 4 * (u - 1) + w;
            if (e < E) {
                int slot;
                const int m = expert_slots(a.logits, a.T, E, a.k, e, &slot);
                int32_t* list = a.slot_lists + e * kSlotListInts;
                if (lane < m) __hip_atomic_store(&list[1 + lane], slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (lane == 0) __hip_atomic_store(&list[0], m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the list is stored
                if (lane == 0) __hip_atomic_store(&list_ready[(int64_t)e * kLineInts], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            __syncthreads();
        } else if (u < u_gu) {  // the shared expert's gate_up quads (every token)
            gate_up_item<1, W8, XB, true>(a, u - u_sgu, a.sh_wgu, a.sh_sgu, TokenRows{0, a.T, a.sh_row0},
                                          red[cur]);
            if (threadIdx.x < kWave) {  // wave 0 stored the h rows
                __builtin_amdgcn_s_waitcnt(0x0f70);
                if (threadIdx.x == 0) atomicAdd(&gu_done[(int64_t)E * kLineInts], 1);
            }
        } else if (u < u_sdn) {  // routed gate_up (e, quad)
            const int e = (u - u_gu) / quads, quad = (u - u_gu) % quads;
            wait_flag(&list_ready[(int64_t)e * kLineInts], 1, &misc[kSelfError]);
            const int32_t* list = a.slot_lists + e * kSlotListInts;
            const int m = uniform(__hip_atomic_load(list, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
            if (m > 0) {
                gate_up_item<1, W4, XB, true>(a, quad, a.wgu + (int64_t)e * quads * (a.H / 128) * 4096,
                                              a.sgu + (int64_t)e * quads * (a.H / 128) * 256,
                                              ListRows{m, list + 1}, red[cur]);
                if (threadIdx.x < kWave) {
                    __builtin_amdgcn_s_waitcnt(0x0f70);
                    if (threadIdx.x == 0) atomicAdd(&gu_done[(int64_t)e * kLineInts], 1);
                }
            }
        } else if (u < u_dn) {  // the shared expert's down quad pairs
            wait_flag(&gu_done[(int64_t)E * kLineInts], quads, &misc[kSelfError]);
            down_item<1, true, W8P>(a, u - u_sdn, a.sh_wdn, a.sh_sdn, TokenRows{0, a.T, a.sh_row0},
                                    red[cur]);
        } else {  // routed down (e, pair)
            const int e = (u - u_dn) / pairs, pair = (u - u_dn) % pairs;
            wait_flag(&list_ready[(int64_t)e * kLineInts], 1, &misc[kSelfError]);
            const int32_t* list = a.slot_lists + e * kSlotListInts;
            const int m = uniform(__hip_atomic_load(list, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
            if (m > 0) {
                wait_flag(&gu_done[(int64_t)e * kLineInts], quads, &misc[kSelfError]);
                down_item<1, true, W4>(a, pair, a.wdn + (int64_t)e * (a.H / 64) * (a.I / 128) * 4096,
                                       a.sdn + (int64_t)e * (a.H / 64) * (a.I / 128) * 256,
                                       ListRows{m, list + 1}, red[cur]);
            }
        }
    }
    grid_combine(a, n_run, n_all, &misc[kSelfDone], go, &misc[kSelfError]);
    // exit: the last workgroup out clears the counters for the next launch
    __shared__ int s_last;
    if (threadIdx.x == 0) s_last = atomicAdd(&misc[kSelfExits], 1) == (int)gridDim.x - 1;
    __syncthreads();
    if (!s_last) return;
    for (int i = threadIdx.x; i < 2 * (E + 1); i += blockDim.x) flags[(int64_t)i * kLineInts] = 0;
    for (int i = threadIdx.x; i < kGoLines; i += blockDim.x) go[i * kGoStride] = 0;
    if (threadIdx.x == 0) {
        misc[kSelfErrorOut] = misc[kSelfError];
        misc[kSelfError] = 0;
        misc[kSelfNext] = 0;
        misc[kSelfDone] = 0;
        misc[kSelfExits] = 0;
    }
}

}  // namespace

hipError_t launch_shared_gate_up(const GemmArgs& a, hipStream_t stream) {
    const bool wide = a.T >= kSharedWideTok;
    const int tok = wide ? kSharedWideTok : 16;
    const int grid = shared_blocks(a.I / 32, (a.T + tok - 1) / tok);
    if (wide)
        shared_gate_up_kernel<4, XB><<<grid, kMfmaThreads, 0, stream>>>(a);
    else
        shared_gate_up_kernel<1, XB><<<grid, kMfmaThreads, 0, stream>>>(a);
    return hipGetLastError();
}

// down reads h as hi/lo pairs (twice the B operand of gate_up), so its
// wide tiles are 32 tokens: four 16-token tiles would spill
hipError_t launch_shared_down(const GemmArgs& a, hipStream_t stream) {
    const bool wide = a.T >= kSharedWideTok;
    const int tok = wide ? 32 : 16;
    const int grid = shared_blocks((a.H / 64 + 1) / 2, (a.T + tok - 1) / tok);
    if (wide)
        shared_down_kernel<2><<<grid, kMfmaThreads, 0, stream>>>(a);
    else
        shared_down_kernel<1><<<grid, kMfmaThreads, 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_mfma_gate_up(const GemmArgs& a, int max_items, hipStream_t stream) {
    const int quads = a.I / 32;
    const int sh = a.sh_wgu ? shared_blocks(quads, (a.T + 15) / 16) : 0;
    mfma_gate_up_kernel<<<sh + max_items * quads, kMfmaThreads, 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_mfma_down(const GemmArgs& a, int max_items, hipStream_t stream) {
    const int pairs = (a.H / 64 + 1) / 2;
    const int sh = a.sh_wdn ? shared_blocks(pairs, (a.T + 15) / 16) : 0;
    mfma_down_kernel<<<sh + max_items * pairs, kMfmaThreads, 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_self_gate_up(const GemmArgs& a, bool lists, hipStream_t stream) {
    const int grid = 1 + (a.E + (a.sh_wgu ? 1 : 0)) * (a.I / 32);
    if (lists)
        self_gate_up_kernel<true><<<grid, kMfmaThreads, 0, stream>>>(a);
    else
        self_gate_up_kernel<false><<<grid, kMfmaThreads, 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_self_down(const GemmArgs& a, bool lists, hipStream_t stream) {
    const int grid = (a.E + (a.sh_wdn ? 1 : 0)) * ((a.H / 64 + 1) / 2);
    if (lists)
        self_down_kernel<true><<<grid, kMfmaThreads, 0, stream>>>(a);
    else
        self_down_kernel<false><<<grid, kMfmaThreads, 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_self_fused(const GemmArgs& a, int32_t* flags, hipStream_t stream) {
    const int quads = a.I / 32, pairs = (a.H / 64 + 1) / 2;
    const int64_t units = 1 + (a.E + 3) / 4 + (int64_t)(a.E + (a.sh_wgu ? 1 : 0)) * (quads + pairs);
    int grid = 0;
    hipError_t err = resident_grid(reinterpret_cast<const void*>(self_fused_kernel), kMfmaThreads, &grid);
    if (err != hipSuccess) return err;
    self_fused_kernel<<<(int)(units < grid ? units : grid), kMfmaThreads, 0, stream>>>(a, flags);
    return hipGetLastError();
}

hipError_t launch_mfma_queue(const GemmArgs& a, int max_items, hipStream_t stream) {
    mfma_queue_kernel<<<max_items * (a.I / 32 + (a.H / 64 + 1) / 2), kMfmaThreads, 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_mfma_fused(const GemmArgs& a, int max_items, hipStream_t stream) {
    const int64_t units = (int64_t)max_items * (a.I / 32 + (a.H / 64 + 1) / 2);
    int grid = 0;
    hipError_t err = resident_grid(reinterpret_cast<const void*>(mfma_fused_kernel), kMfmaThreads, &grid);
    if (err != hipSuccess) return err;
    mfma_fused_kernel<<<(int)(units < grid ? units : grid), kMfmaThreads, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace moe
