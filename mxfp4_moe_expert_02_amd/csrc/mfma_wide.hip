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
#include <type_traits>

#include "mfma_items.h"

namespace moe {
namespace {

constexpr int kWideWavesPerEu = 2;  // launch bound: at least 2 waves per SIMD
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

// ---- the down GEMM: B is h as three MXFP8 terms (store_h3), on the scaled
// FP4 x FP8 matrix cores.  Per chunk a staged token row is 400 bytes of LDS:
// the chunk's 384 code bytes ([g][term][32], as stored) and its 16 scale
// bytes ([g][term]); at that stride a quarter-wave's 16-byte reads of 16
// rows cover all 64 banks once.  Each staged row (16 NT rows, or 64 for
// NT = 3) is copied by kTpr threads, thread (n, l) = (tid / kTpr, tid %
// kTpr) taking 16-byte units l, l + kTpr, ... of its 25: units 0..23 are
// code bytes, unit 24 the scales; a thread's last unit past 24 loads the
// scales again and is not stored.  Rows past the item's m tokens repeat
// row m - 1 (they only feed output columns that are never stored).  The
// loads are issued at the start of a step and written to the other buffer
// after its MFMAs.
constexpr int kQRow = 400;
constexpr int kQUnits = kQRow / 16;  // 24 code units, then 1 scale unit

struct WQSmem {
    alignas(16) uint8_t q[2][kWMaxTiles * 16 * kQRow];
};

template <int NT>
struct QStage {
    static constexpr int kTpr = NT == 1 ? 16 : NT == 2 ? 8 : 4;  // threads per staged row
    static constexpr int kPer = (kQUnits + kTpr - 1) / kTpr;      // units per thread
    const uint8_t* q;   // chunk 0 of this thread's first code unit
    const uint8_t* sc;  // chunk 0 of its row's scales
    uint4 v[kPer];
};

// staged row n is h row rows.row(min(n, m - 1)) (Rows: SortedRows, or the
// slot list of a self-routed expert)
template <int NT, typename Rows>
__device__ inline void q_stage_init(const GemmArgs& a, const Rows& rows, QStage<NT>& st) {
    constexpr int kTpr = QStage<NT>::kTpr;
    const int n = threadIdx.x / kTpr, l = threadIdx.x % kTpr;
    const int64_t r = rows.row(min(n, rows.m - 1));
    st.q = a.h3q + r * 3 * a.I + 16 * l;
    st.sc = a.h3s + r * h3s_stride(a.I);
}

template <int NT>
__device__ inline void q_load(QStage<NT>& st, int chunk) {
    constexpr int kTpr = QStage<NT>::kTpr, kPer = QStage<NT>::kPer;
    const int l = threadIdx.x % kTpr;
#pragma unroll
    for (int i = 0; i < kPer; i++) {
        const uint8_t* p = st.q + chunk * 384 + 16 * kTpr * i;
        if (i == kPer - 1 && l + kTpr * i >= kQUnits - 1) p = st.sc + chunk * 16;
        st.v[i] = *reinterpret_cast<const uint4*>(p);
    }
}

template <int NT>
__device__ inline void q_store(WQSmem& sm, int buf, const QStage<NT>& st) {
    constexpr int kTpr = QStage<NT>::kTpr, kPer = QStage<NT>::kPer;
    const int n = threadIdx.x / kTpr, l = threadIdx.x % kTpr;
#pragma unroll
    for (int i = 0; i < kPer; i++) {
        const int u = l + kTpr * i;
        if (u < kQUnits) *reinterpret_cast<uint4*>(&sm.q[buf][n * kQRow + 16 * u]) = st.v[i];
    }
}

// The 12*NT scaled MFMAs of one chunk: weights b (this wave's quad, FP4
// codes and scales as they are), h's terms from LDS buffer `buf`.
template <int NT>
__device__ inline void chunk_mfma_q3(const WQSmem& sm, int buf, const WChunk& b,
                                     f32x4_t (&acc)[kGroups][NT]) {
    const int lane = threadIdx.x % kWave, c = lane % 16, g = lane / 16;
#pragma unroll
    for (int t = 0; t < NT; t++) {
        const uint8_t* row = &sm.q[buf][(16 * t + c) * kQRow];
        const uint32_t sb = *reinterpret_cast<const uint32_t*>(row + 384 + 4 * g);
        static_for<kHTerms>([&](auto tm) {
            const uint4 lo = *reinterpret_cast<const uint4*>(row + 96 * g + 32 * tm);
            const uint4 hi = *reinterpret_cast<const uint4*>(row + 96 * g + 32 * tm + 16);
            const i32x8_t B = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                               (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            static_for<kGroups>([&](auto rg) {
                const uint4& w = b.w[rg];
                const i32x8_t A = {(int)w.x, (int)w.y, (int)w.z, (int)w.w, 0, 0, 0, 0};
                // scale bytes: rg of the lane's weight scales, tm of its h scales
                acc[rg][t] = mfma_scaled<4, rg, tm>(A, B, acc[rg][t], b.s, sb);
            });
        });
    }
}

// Main loop of the down GEMM over all `chunks` chunks: chunk s + 1's h is
// staged and its weights loaded while chunk s is computed (weights in the
// buffer chunk s - 1 left), as in wide_mainloop.
template <int NT, typename Rows>
__device__ inline void wide_mainloop_q3(const GemmArgs& a, const uint8_t* tiles, const uint8_t* tscales,
                                        bool live, const Rows& rows, int chunks, WQSmem& sm,
                                        f32x4_t (&acc)[kGroups][NT]) {
#pragma unroll
    for (int rg = 0; rg < kGroups; rg++)
#pragma unroll
        for (int t = 0; t < NT; t++) acc[rg][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    QStage<NT> st;
    q_stage_init<NT>(a, rows, st);
    q_load<NT>(st, 0);
    WChunk w[2];
    if (live) load_chunk(tiles, tscales, 0, w[0]);
    q_store<NT>(sm, 0, st);
    __syncthreads();
    auto step = [&](int s, WChunk& cur, WChunk& ahead) {
        q_load<NT>(st, s + 1 < chunks ? s + 1 : s);
        if (live && s + 1 < chunks) load_chunk(tiles, tscales, s + 1, ahead);
        if (live) chunk_mfma_q3<NT>(sm, s & 1, cur, acc);
        q_store<NT>(sm, (s & 1) ^ 1, st);
        __syncthreads();
    };
    for (int s0 = 0; s0 < chunks; s0 += 2) {
        step(s0, w[0], w[1]);
        if (s0 + 1 >= chunks) break;
        step(s0 + 1, w[1], w[0]);
    }
}

template <int NT, bool PUBLISH>
__device__ inline void wide_gate_up(const GemmArgs& a, int qb, int e, int row0, int m, WSmem& sm) {
    const int tid = threadIdx.x, w = tid / kWave;
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
    store_h_tile<NT, PUBLISH>(a, quad, SortedRows{row0, m}, acc);
}

// Down quads 4qb .. 4qb+3 of expert e (one per wave) for the token rows
// `rows` (SortedRows of a routed item, or ListRows of a self-routed expert)
template <int NT, bool PUBLISH, typename Rows>
__device__ inline void wide_down(const GemmArgs& a, int qb, int e, const Rows& rows, WQSmem& sm) {
    const int w = threadIdx.x / kWave;
    const int chunks = a.I / 128, quads = a.H / 64;
    const int quad = kWQuads * qb + w;
    const bool live = quad < quads;
    const int64_t quad_id = (int64_t)e * quads + (live ? quad : 0);
    f32x4_t acc[kGroups][NT];
    wide_mainloop_q3<NT>(a, a.wdn + quad_id * chunks * 4096, a.sdn + quad_id * chunks * 256, live, rows,
                         chunks, sm, acc);
    if (!live) return;
    store_down_tile<NT, PUBLISH>(a, quad, rows, acc);
}

// Call fn(std::integral_constant<int, NT>) for an item of m tokens: NT =
// its 16-token column tiles (1..4).
template <typename Fn>
__device__ inline void by_tiles(int m, Fn fn) {
    switch ((m + 15) / 16) {
        case 1: fn(std::integral_constant<int, 1>{}); break;
        case 2: fn(std::integral_constant<int, 2>{}); break;
        case 3: fn(std::integral_constant<int, 3>{}); break;
        default: fn(std::integral_constant<int, 4>{}); break;
    }
}

// gate_up: blockIdx.x = item * (I / 128) + quad block (quads 4qb..4qb+3)
__global__ void __launch_bounds__(kWThreads, kWideWavesPerEu) wide_gate_up_kernel(GemmArgs a) {
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
    by_tiles(m, [&](auto nt) { wide_gate_up<decltype(nt)::value, false>(a, qb, e, row0, m, sm); });
}

// down: blockIdx.x = item * ceil(H / 256) + quad block
__global__ void __launch_bounds__(kWThreads, kWideWavesPerEu) wide_down_kernel(GemmArgs a) {
    __shared__ WQSmem sm;
    static_assert(sizeof(WQSmem) >= sizeof(f32x4_t) * kRedDown, "LDS of the shared blocks");
    const int qblocks = (a.H / 64 + kWQuads - 1) / kWQuads;
    int b = blockIdx.x;
    if (a.sh_wdn) {  // the shared expert's blocks first (16-token tiles, split-K)
        const int nb = shared_blocks((a.H / 64 + 1) / 2, (a.T + 15) / 16);
        if (b < nb) {
            shared_down_block<1>(a, b, reinterpret_cast<f32x4_t*>(&sm));
            return;
        }
        b -= nb;
    }
    const int item = b / qblocks, qb = b % qblocks;
    if (item >= uniform(a.meta[kMetaNumMfmaItems])) return;
    const int4 it = a.items[item];
    const int e = uniform(it.x), row0 = uniform(it.y), m = uniform(it.z);
    by_tiles(m, [&](auto nt) { wide_down<decltype(nt)::value, false>(a, qb, e, SortedRows{row0, m}, sm); });
}

// The wide kernels in one persistent launch (see mfma_fused_kernel in
// mfma.hip: the same queue, publication and bounded wait; a gate_up unit
// is (item, quad block of four quads), and every wave stores h of its quad;
// a down unit is (item, quad block); the grid combines at the end).
__global__ void __launch_bounds__(kWThreads, kWideWavesPerEu) wide_fused_kernel(GemmArgs a) {
    __shared__ union {
        WSmem x;
        WQSmem q;
    } sm;
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
    int n_run = 0;  // units this workgroup ran
    for (int cur = 0;; cur ^= 1) {
        const int u = uniform(s_unit[cur]);
        if (u >= n_all) break;
        n_run++;
        if (threadIdx.x == 0) s_unit[cur ^ 1] = atomicAdd(&a.queue[kQueueNext], 1);
        if (u < n_gu) {
            const int item = u / gu_units, qb = u % gu_units;
            const int4 it = a.items[item];
            const int e = uniform(it.x), row0 = uniform(it.y), m = uniform(it.z);
            by_tiles(m, [&](auto nt) { wide_gate_up<decltype(nt)::value, true>(a, qb, e, row0, m, sm.x); });
            __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's h stores completed
            __syncthreads();
            if (threadIdx.x == 0) atomicAdd(&a.gu_done[(int64_t)item * kLineInts], 1);
        } else {
            const int v = u - n_gu, item = v / dn_units, qb = v % dn_units;
            const int4 it = a.items[item];
            const int e = uniform(it.x), row0 = uniform(it.y), m = uniform(it.z);
            if (threadIdx.x == 0) wait_count(&a.gu_done[(int64_t)item * kLineInts], gu_units, &a.queue[kQueueError]);
            __syncthreads();
            by_tiles(m, [&](auto nt) {
                wide_down<decltype(nt)::value, true>(a, qb, e, SortedRows{row0, m}, sm.q);
            });
        }
        __syncthreads();  // LDS free for the next unit, whose index is now visible
    }
    grid_combine(a, n_run, n_all, &a.queue[kQueueDone], &a.queue[kQueueGo], &a.queue[kQueueError]);
}

// The wide kernels as one launch of one workgroup per unit: each
// workgroup dequeues its unit from a counter -- the gate_up units (item,
// quad block) first, then the down units (item, quad block) -- runs it and
// exits; the combine is a launch of its own.  A down unit first waits
// (bounded, raising queue[kQueueError] if it gives up) until all I/128
// gate_up units of its item are done; those were dequeued earlier, by
// workgroups that are running and never wait, so no wait can deadlock
// whatever the hardware's dispatch order.  The down units of finished items
// thus run while the last gate_up units do: with the split launch the end
// of gate_up's last round of workgroups, often a fraction of the CUs,
// leaves the rest of the GPU idle.  Unit bodies, arithmetic and order are
// the split launch's (h stores agent-coherent: other XCDs read them in
// this launch), so the output bits are too.
__global__ void __launch_bounds__(kWThreads, kWideWavesPerEu) wide_queue_kernel(GemmArgs a) {
    __shared__ union {
        WSmem x;
        WQSmem q;
    } sm;
    __shared__ int s_unit;
    const int n_items = uniform(a.meta[kMetaNumMfmaItems]);
    const int gu_units = a.I / 128, dn_units = (a.H / 64 + kWQuads - 1) / kWQuads;
    const int n_gu = n_items * gu_units, n_all = n_gu + n_items * dn_units;
    if (threadIdx.x == 0) s_unit = atomicAdd(&a.queue[kQueueNext], 1);
    __syncthreads();
    const int u = uniform(s_unit);
    if (u >= n_all) return;
    if (u < n_gu) {
        const int item = u / gu_units, qb = u % gu_units;
        const int4 it = a.items[item];
        const int e = uniform(it.x), row0 = uniform(it.y), m = uniform(it.z);
        by_tiles(m, [&](auto nt) { wide_gate_up<decltype(nt)::value, true>(a, qb, e, row0, m, sm.x); });
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's h stores completed
        __syncthreads();
        if (threadIdx.x == 0) atomicAdd(&a.gu_done[(int64_t)item * kLineInts], 1);
    } else {
        const int v = u - n_gu, item = v / dn_units, qb = v % dn_units;
        const int4 it = a.items[item];
        const int e = uniform(it.x), row0 = uniform(it.y), m = uniform(it.z);
        if (threadIdx.x == 0) wait_count(&a.gu_done[(int64_t)item * kLineInts], gu_units, &a.queue[kQueueError]);
        __syncthreads();
        by_tiles(m, [&](auto nt) { wide_down<decltype(nt)::value, false>(a, qb, e, SortedRows{row0, m}, sm.q); });
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
    const int sh = a.sh_wdn ? shared_blocks((a.H / 64 + 1) / 2, (a.T + 15) / 16) : 0;
    wide_down_kernel<<<sh + max_items * qblocks, kWThreads, 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_wide_queue(const GemmArgs& a, int max_items, hipStream_t stream) {
    const int qblocks = (a.H / 64 + kWQuads - 1) / kWQuads;
    wide_queue_kernel<<<max_items * (a.I / 128 + qblocks), kWThreads, 0, stream>>>(a);
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
