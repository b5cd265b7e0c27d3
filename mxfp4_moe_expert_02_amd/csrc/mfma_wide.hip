// mfma_wide.hip -- the bf16 expert GEMMs for items of up to 64 tokens
// (layers whose experts average several tokens each, e.g. the batched and
// skewed verify steps), over the prepacked MFMA tile layout.
//
// With wide items the activation loads, not the weight bytes, limit the
// split-K kernels of mfma.hip: every quad workgroup loads every token row of
// its item, so x costs NT times the address and cache work of the weights.
// Here a workgroup owns four quads (256 weight rows) and the whole K; each
// 128-k chunk of the item's x rows (NT x 16 tokens, bf16) is loaded once
// into LDS and read by all four waves.  Wave w computes quad 4qb+w against
// all NT column tiles:
//   A: the quad's 4 KB tile of the chunk, 16 bytes per lane per row group,
//      decoded with v_cvt_scalef32_pk_bf16_fp4 (block scale applied), the
//      next chunk's weights loaded during the MFMAs;
//   B: lane (c, g) reads elements 32g + 8q .. +7 of token row c from LDS
//      (rows padded to 272 bytes: a quarter-wave's 16-byte reads then cover
//      all banks once);
//   D: 16 rows x 16 tokens per (row group, tile), fp32.
// x is staged one chunk ahead through double-buffered LDS with
// unconditional loads (rows past the item repeat its last token: they only
// feed output columns that are never stored).  No cross-wave reduction is
// needed: each wave ends with its quad's complete sums.
#include "mfma_items.h"

namespace moe {
namespace {

#ifndef MOE_WIDE_WAVES_PER_EU
#define MOE_WIDE_WAVES_PER_EU 2
#endif

constexpr int kWThreads = 256;
constexpr int kWQuads = 4;                     // quads per workgroup (one per wave)
constexpr int kWMaxTiles = kMfmaItemTok / 16;  // 4
constexpr int kXRow = 272;                     // LDS bytes per staged token row (256 + 16)

struct WSmem {
    alignas(16) uint8_t x[2][kWMaxTiles * 16 * kXRow];  // [buffer][token row][272]
};

struct WChunk {
    uint4 w[kGroups];
    uint32_t s;
};

__device__ inline void load_chunk(const uint8_t* tiles, const uint8_t* tscales, int chunk, WChunk& b) {
    const int lane = threadIdx.x % kWave;
    const uint8_t* t = tiles + (int64_t)chunk * 4096 + lane * 16;
#pragma unroll
    for (int rg = 0; rg < kGroups; rg++) b.w[rg] = load_stream16(t + rg * 1024);
    b.s = *reinterpret_cast<const uint32_t*>(tscales + (int64_t)chunk * 256 + lane * 4);
}

// x staging: thread tid copies 16 bytes (8 bf16) of token row 16n + tid/16
// for n < NT: elements 8*(tid % 16) .. +7 of the chunk.
template <int NT>
struct XStage {
    uint4 v[NT];
};

template <int NT>
__device__ inline void x_load(const uint16_t* const (&rows)[NT], int chunk, XStage<NT>& st) {
#pragma unroll
    for (int n = 0; n < NT; n++)
        st.v[n] = *reinterpret_cast<const uint4*>(rows[n] + chunk * 128);
}

template <int NT>
__device__ inline void x_store(WSmem& sm, int buf, const XStage<NT>& st) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int n = 0; n < NT; n++)
        *reinterpret_cast<uint4*>(&sm.x[buf][(16 * n + tid / 16) * kXRow + 16 * (tid % 16)]) = st.v[n];
}

// The 16*NT MFMAs of one chunk: weights b (this wave's quad), x from LDS
// buffer `buf`.
template <int NT>
__device__ inline void chunk_mfma(const WSmem& sm, int buf, const WChunk& b,
                                  f32x4_t (&acc)[kGroups][NT]) {
    const int lane = threadIdx.x % kWave, c = lane % 16, g = lane / 16;
#pragma unroll
    for (int q = 0; q < 4; q++) {
        bf16x8_t B[NT];
#pragma unroll
        for (int t = 0; t < NT; t++)
            B[t] = *reinterpret_cast<const bf16x8_t*>(
                &sm.x[buf][(16 * t + c) * kXRow + 64 * g + 16 * q]);
#pragma unroll
        for (int rg = 0; rg < kGroups; rg++) {
            const bf16x8_t A = decode8(word_of(b.w[rg], q), e8m0_as_scale((b.s >> (8 * rg)) & 0xffu));
#pragma unroll
            for (int t = 0; t < NT; t++)
                acc[rg][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B[t], acc[rg][t], 0, 0, 0);
        }
    }
}

// Main loop of one workgroup over all `chunks` chunks.  live: this wave's
// quad exists (all waves stage x and meet every barrier either way).  Two
// weight buffers alternate: chunk s+1 is loaded into the buffer that chunk
// s-1 just left while chunk s is computed.  (Written as a loop over two
// unrolled steps with exits, which the compiler allocates in 164 VGPRs --
// three workgroups per CU -- where other forms of the same loop take 242.)
template <int NT>
__device__ inline void wide_mainloop(const uint8_t* tiles, const uint8_t* tscales, bool live,
                                     const uint16_t* const (&rows)[NT], int chunks, WSmem& sm,
                                     f32x4_t (&acc)[kGroups][NT]) {
    constexpr int WB = 2;
#pragma unroll
    for (int rg = 0; rg < kGroups; rg++)
#pragma unroll
        for (int t = 0; t < NT; t++) acc[rg][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    XStage<NT> st;
    x_load<NT>(rows, 0, st);
    WChunk w[WB];
    if (live) {
#pragma unroll
        for (int i = 0; i < WB - 1; i++)
            if (i < chunks) load_chunk(tiles, tscales, i, w[i]);
    }
    x_store<NT>(sm, 0, st);
    __syncthreads();
    auto step = [&](int s, WChunk& cur, WChunk& ahead) {
        const int nxt = s + 1 < chunks ? s + 1 : s;
        x_load<NT>(rows, nxt, st);
        if (live && s + WB - 1 < chunks) load_chunk(tiles, tscales, s + WB - 1, ahead);
        if (live) chunk_mfma<NT>(sm, s & 1, cur, acc);
        x_store<NT>(sm, (s & 1) ^ 1, st);
        __syncthreads();
    };
    for (int s0 = 0; s0 < chunks; s0 += WB) {
#pragma unroll
        for (int i = 0; i < WB; i++) {
            if (s0 + i >= chunks) break;
            step(s0 + i, w[i], w[(i + WB - 1) % WB]);
        }
    }
}

template <int NT>
__device__ inline void wide_gate_up(const GemmArgs& a, int qb, int e, int row0, int m, WSmem& sm) {
    const int tid = threadIdx.x, w = tid / kWave, lane = tid % kWave, c = lane % 16, g = lane / 16;
    const int K = a.H, chunks = K / 128, quads = a.I / 32;
    const int quad = kWQuads * qb + w;  // quads % 4 == 0: always live
    const int64_t quad_id = (int64_t)e * quads + quad;
    const uint16_t* rows[NT];
#pragma unroll
    for (int n = 0; n < NT; n++) {
        const int j = min(16 * n + tid / 16, m - 1);
        rows[n] = a.x + (int64_t)(a.sorted[row0 + j] / a.k) * K + 8 * (tid % 16);
    }
    f32x4_t acc[kGroups][NT];
    wide_mainloop<NT>(a.wgu + quad_id * chunks * 4096, a.sgu + quad_id * chunks * 256, true, rows,
                      chunks, sm, acc);
#pragma unroll
    for (int t = 0; t < NT; t++) {
        const int j = 16 * t + c;
        if (j >= m) continue;
        uint16_t* hrow = a.h + (int64_t)(row0 + j) * a.I + 32 * quad + 4 * g;
#pragma unroll
        for (int rg = 0; rg < 2; rg++) {
            ushort4 o;
            o.x = f32_to_bf16_rne(silu_mul(acc[rg][t][0], acc[rg + 2][t][0]));
            o.y = f32_to_bf16_rne(silu_mul(acc[rg][t][1], acc[rg + 2][t][1]));
            o.z = f32_to_bf16_rne(silu_mul(acc[rg][t][2], acc[rg + 2][t][2]));
            o.w = f32_to_bf16_rne(silu_mul(acc[rg][t][3], acc[rg + 2][t][3]));
            store_h4(hrow + 16 * rg, o);
        }
    }
}

template <int NT, bool COMBINE>
__device__ inline void wide_down(const GemmArgs& a, int qb, int e, int row0, int m, WSmem& sm) {
    const int tid = threadIdx.x, w = tid / kWave;
    const int K = a.I, chunks = K / 128, quads = a.H / 64;
    const int quad = kWQuads * qb + w;
    const bool live = quad < quads;
    const int64_t quad_id = (int64_t)e * quads + (live ? quad : 0);
    const uint16_t* rows[NT];
#pragma unroll
    for (int n = 0; n < NT; n++) {
        const int j = min(16 * n + tid / 16, m - 1);
        rows[n] = a.h + (int64_t)(row0 + j) * K + 8 * (tid % 16);
    }
    f32x4_t acc[kGroups][NT];
    wide_mainloop<NT>(a.wdn + quad_id * chunks * 4096, a.sdn + quad_id * chunks * 256, live, rows,
                      chunks, sm, acc);
    if (!live) return;
    store_down_tile<NT, COMBINE>(a, quad, SortedRows{row0, m}, acc);
}

// gate_up: blockIdx.x = item * (I / 128) + quad block (quads 4qb..4qb+3)
__global__ void __launch_bounds__(kWThreads, MOE_WIDE_WAVES_PER_EU) wide_gate_up_kernel(GemmArgs a) {
    __shared__ WSmem sm;
    static_assert(sizeof(WSmem) >= sizeof(f32x4_t) * kRedGateUp * 2, "LDS of the shared blocks");
    const int qblocks = a.I / 128;
    int b = blockIdx.x;
    if (a.sh_wgu) {  // the shared expert's blocks first (32-token tiles, split-K)
        const int nb = shared_blocks(a.I / 32, (a.T + 31) / 32);
        if (b < nb) {
            shared_gate_up_block<2, XB>(a, b, reinterpret_cast<f32x4_t*>(&sm));
            return;
        }
        b -= nb;
    }
    const int item = b / qblocks, qb = b % qblocks;
    if (item >= uniform(a.meta[kMetaNumMfmaItems])) return;
    const int4 it = a.items[item];
    const int e = uniform(it.x), row0 = uniform(it.y), m = uniform(it.z);
    switch ((m + 15) / 16) {
        case 1: wide_gate_up<1>(a, qb, e, row0, m, sm); break;
#if MOE_WIDE_ITEM_TOK > 32
        case 2: wide_gate_up<2>(a, qb, e, row0, m, sm); break;
        case 3: wide_gate_up<3>(a, qb, e, row0, m, sm); break;
        default: wide_gate_up<4>(a, qb, e, row0, m, sm); break;
#else
        default: wide_gate_up<2>(a, qb, e, row0, m, sm); break;
#endif
    }
}

// down: blockIdx.x = item * ceil(H / 256) + quad block; a quad is also the
// combine tile (the last finisher of a token's k experts combines it)
__global__ void __launch_bounds__(kWThreads, MOE_WIDE_WAVES_PER_EU) wide_down_kernel(GemmArgs a) {
    __shared__ WSmem sm;
    static_assert(sizeof(WSmem) >= sizeof(f32x4_t) * kRedDown * 2, "LDS of the shared blocks");
    const int qblocks = (a.H / 64 + kWQuads - 1) / kWQuads;
    int b = blockIdx.x;
    if (a.sh_wdn) {  // the shared expert's blocks first
        const int nb = shared_blocks((a.H / 64 + 1) / 2, (a.T + 31) / 32);
        if (b < nb) {
            shared_down_block<2, XB>(a, b, reinterpret_cast<f32x4_t*>(&sm));
            return;
        }
        b -= nb;
    }
    const int item = b / qblocks, qb = b % qblocks;
    if (item >= uniform(a.meta[kMetaNumMfmaItems])) return;
    const int4 it = a.items[item];
    const int e = uniform(it.x), row0 = uniform(it.y), m = uniform(it.z);
    switch ((m + 15) / 16) {
        case 1: wide_down<1, false>(a, qb, e, row0, m, sm); break;
#if MOE_WIDE_ITEM_TOK > 32
        case 2: wide_down<2, false>(a, qb, e, row0, m, sm); break;
        case 3: wide_down<3, false>(a, qb, e, row0, m, sm); break;
        default: wide_down<4, false>(a, qb, e, row0, m, sm); break;
#else
        default: wide_down<2, false>(a, qb, e, row0, m, sm); break;
#endif
    }
}


// The wide kernels in one persistent launch (see mfma_fused_kernel in
// mfma.hip: the same queue, publication and bounded wait; a gate_up unit
// is (item, quad block of four quads), and every wave stores h of its quad).
__global__ void __launch_bounds__(kWThreads, MOE_WIDE_WAVES_PER_EU) wide_fused_kernel(GemmArgs a) {
    __shared__ WSmem sm;
    __shared__ int s_unit[2];
    const int n_items = uniform(a.meta[kMetaNumMfmaItems]);
    const int gu_units = a.I / 128, dn_units = (a.H / 64 + kWQuads - 1) / kWQuads;
    const int n_gu = n_items * gu_units, n_all = n_gu + n_items * dn_units;
    // the next unit is dequeued while the current one runs (the atomic's
    // round trip then costs nothing); holding it cannot block anyone: a
    // workgroup holds a gate_up unit only while running a gate_up unit,
    // which never waits
    if (threadIdx.x == 0) s_unit[0] = atomicAdd(&a.queue[kQueueNext], 1);
    __syncthreads();
    for (int cur = 0;; cur ^= 1) {
        const int u = uniform(s_unit[cur]);
        if (u >= n_all) return;
        if (threadIdx.x == 0) s_unit[cur ^ 1] = atomicAdd(&a.queue[kQueueNext], 1);
        if (u < n_gu) {
            const int item = u / gu_units, qb = u % gu_units;
            const int4 it = a.items[item];
            const int e = uniform(it.x), row0 = uniform(it.y), m = uniform(it.z);
            switch ((m + 15) / 16) {
                case 1: wide_gate_up<1>(a, qb, e, row0, m, sm); break;
#if MOE_WIDE_ITEM_TOK > 32
                case 2: wide_gate_up<2>(a, qb, e, row0, m, sm); break;
                case 3: wide_gate_up<3>(a, qb, e, row0, m, sm); break;
                default: wide_gate_up<4>(a, qb, e, row0, m, sm); break;
#else
                default: wide_gate_up<2>(a, qb, e, row0, m, sm); break;
#endif
            }
            __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's h stores completed
            __syncthreads();
            if (threadIdx.x == 0) atomicAdd(&a.gu_done[item], 1);
        } else {
            const int v = u - n_gu, item = v / dn_units, qb = v % dn_units;
            const int4 it = a.items[item];
            const int e = uniform(it.x), row0 = uniform(it.y), m = uniform(it.z);
            if (threadIdx.x == 0) wait_count(&a.gu_done[item], gu_units, &a.queue[kQueueError]);
            __syncthreads();
            switch ((m + 15) / 16) {
                case 1: wide_down<1, true>(a, qb, e, row0, m, sm); break;
#if MOE_WIDE_ITEM_TOK > 32
                case 2: wide_down<2, true>(a, qb, e, row0, m, sm); break;
                case 3: wide_down<3, true>(a, qb, e, row0, m, sm); break;
                default: wide_down<4, true>(a, qb, e, row0, m, sm); break;
#else
                default: wide_down<2, true>(a, qb, e, row0, m, sm); break;
#endif
            }
        }
        __syncthreads();  // LDS free for the next unit, whose index is now visible
    }
}

}  // namespace

hipError_t launch_wide_gate_up(const GemmArgs& a, int max_items, hipStream_t stream) {
    const int sh = a.sh_wgu ? shared_blocks(a.I / 32, (a.T + 31) / 32) : 0;
    wide_gate_up_kernel<<<sh + max_items * (a.I / 128), kWThreads, 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_wide_down(const GemmArgs& a, int max_items, hipStream_t stream) {
    const int qblocks = (a.H / 64 + kWQuads - 1) / kWQuads;
    const int sh = a.sh_wdn ? shared_blocks((a.H / 64 + 1) / 2, (a.T + 31) / 32) : 0;
    wide_down_kernel<<<sh + max_items * qblocks, kWThreads, 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_wide_fused(const GemmArgs& a, int max_items, hipStream_t stream) {
    const int qblocks = (a.H / 64 + kWQuads - 1) / kWQuads;
    const int64_t units = (int64_t)max_items * (a.I / 128 + qblocks);
    int grid = 0;
    hipError_t err = resident_grid(reinterpret_cast<const void*>(wide_fused_kernel), kWThreads, &grid);
    if (err != hipSuccess) return err;
    wide_fused_kernel<<<(int)(units < grid ? units : grid), kWThreads, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace moe
