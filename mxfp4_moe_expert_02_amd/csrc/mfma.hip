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
#include "device_common.h"
#include "mx_encode.h"
#include "route_rank.h"

namespace moe {
namespace {

#ifndef MOE_MFMA_CHUNKS_PER_STEP
#define MOE_MFMA_CHUNKS_PER_STEP 2
#endif
#ifndef MOE_MFMA_WAVES_PER_EU
#define MOE_MFMA_WAVES_PER_EU 2
#endif

constexpr int kWaves = kMfmaThreads / kWave;  // 4, split K
constexpr int kChunksPerStep = MOE_MFMA_CHUNKS_PER_STEP;  // 128-column chunks per prefetch step
constexpr int kGroups = 4;                    // 16-row groups per quad

// ---- weight formats of the tile layout (one 64-row quad, one 128-k chunk)
// W4, MXFP4: 4 KB of codes, [group][lane][16 bytes], lane (r, g) holding
// the 32 codes of block g of row r.  W8, MXFP8 (the 8-bit weights beside
// the experts): 8 KB, [group][half][lane][16 bytes], half h holding codes
// 16h..16h+15 of the lane's block.  Both: 256 scale bytes [lane][group].
// a(b, rg, q) is the bf16 A operand of step q (codes 8q..8q+7 of the
// lane's block of group rg), block scale applied by the conversion.
struct W4 {
    static constexpr int kChunkBytes = 4096;
    struct Chunk {
        uint4 w[kGroups];
        uint32_t s;
    };
    static __device__ void load(const uint8_t* tiles, const uint8_t* tscales, int ci, Chunk& b) {
        const int lane = threadIdx.x % kWave;
        const uint8_t* t = tiles + (int64_t)ci * kChunkBytes + lane * 16;
#pragma unroll
        for (int rg = 0; rg < kGroups; rg++) b.w[rg] = load_stream16(t + rg * 1024);
        b.s = *reinterpret_cast<const uint32_t*>(tscales + (int64_t)ci * 256 + lane * 4);
    }
    static __device__ bf16x8_t a(const Chunk& b, int rg, int q) {
        return decode8(word_of(b.w[rg], q), e8m0_as_scale((b.s >> (8 * rg)) & 0xffu));
    }
};
struct W8 {
    static constexpr int kChunkBytes = 8192;
    struct Chunk {
        uint4 w[kGroups][2];
        uint32_t s;
    };
    static __device__ void load(const uint8_t* tiles, const uint8_t* tscales, int ci, Chunk& b) {
        const int lane = threadIdx.x % kWave;
        const uint8_t* t = tiles + (int64_t)ci * kChunkBytes + lane * 16;
#pragma unroll
        for (int rg = 0; rg < kGroups; rg++)
#pragma unroll
            for (int h = 0; h < 2; h++) b.w[rg][h] = load_stream16(t + rg * 2048 + h * 1024);
        b.s = *reinterpret_cast<const uint32_t*>(tscales + (int64_t)ci * 256 + lane * 4);
    }
    static __device__ bf16x8_t a(const Chunk& b, int rg, int q) {
        const uint4& v = b.w[rg][q >> 1];
        return decode8_e4m3((q & 1) ? v.z : v.x, (q & 1) ? v.w : v.y,
                            e8m0_as_scale((b.s >> (8 * rg)) & 0xffu));
    }
};

// ---- activation formats of the B operand (one token row, 128-k chunk):
// lane (c, g) takes block g of the chunk; b(x, q) is the bf16 B operand of
// step q (elements 8q..8q+7 of the block).  XB: bf16 rows.  X8: MXFP8 rows
// (E4M3 codes and one E8M0 scale per block, the prefill format), decoded
// to bf16 exactly.  row(a, token) is a token's x row, hrow(a, r) row r of h.
struct XB {
    static constexpr bool kMx8 = false;
    struct Row {
        const uint16_t* p;
    };
    struct Chunk {
        uint4 x[4];
    };
    static __device__ Row row(const GemmArgs& a, int t) { return Row{a.x + (int64_t)t * a.H}; }
    static __device__ Row hrow(const GemmArgs& a, int r) { return Row{a.h + (int64_t)r * a.I}; }
    static __device__ void load(const Row& r, int chunk, int g, Chunk& c) {
        const uint4* src = reinterpret_cast<const uint4*>(r.p + (int64_t)(4 * chunk + g) * 32);
#pragma unroll
        for (int q = 0; q < 4; q++) c.x[q] = src[q];
    }
    static __device__ bf16x8_t b(const Chunk& c, int q) { return __builtin_bit_cast(bf16x8_t, c.x[q]); }
};
struct X8 {
    static constexpr bool kMx8 = true;
    struct Row {
        const uint8_t* c;
        const uint8_t* s;
    };
    struct Chunk {
        uint4 x[2];
        uint32_t s;
    };
    static __device__ Row row(const GemmArgs& a, int t) {
        return Row{a.xq + (int64_t)t * a.H, a.xs + (int64_t)t * (a.H / 32)};
    }
    static __device__ Row hrow(const GemmArgs& a, int r) {
        return Row{a.hq + (int64_t)r * a.I, a.hs + (int64_t)r * (a.I / 32)};
    }
    static __device__ void load(const Row& r, int chunk, int g, Chunk& c) {
        const uint4* src = reinterpret_cast<const uint4*>(r.c + (int64_t)(4 * chunk + g) * 32);
        c.x[0] = src[0];
        c.x[1] = src[1];
        c.s = r.s[4 * chunk + g];
    }
    static __device__ bf16x8_t b(const Chunk& c, int q) {
        const uint4& v = c.x[q >> 1];
        return decode8_e4m3((q & 1) ? v.z : v.x, (q & 1) ? v.w : v.y, e8m0_as_scale(c.s));
    }
};

// chunks per prefetch step: MXFP4 single-tile items kChunksPerStep, wider
// ones one (their x operands alone fill 16 VGPRs per tile and chunk);
// MXFP8 weights one (a chunk is already twice the bytes)
#ifndef MOE_MFMA_WIDE_CPS
#define MOE_MFMA_WIDE_CPS 1
#endif

template <int NT, typename W>
struct Cps {
    static constexpr int value =
        W::kChunkBytes != 4096 ? 1 : NT == 1 ? kChunksPerStep : NT == 2 ? MOE_MFMA_WIDE_CPS : 1;
};

template <typename W, int CPS>
struct WStep {
    typename W::Chunk c[CPS];
};

template <typename X, int NT, int CPS>
struct XStep {
    typename X::Chunk x[CPS][NT];
};

// One wave: chunks [c_begin, c_end) of one quad against NT column tiles of
// 16 tokens.  tiles/tscales point at the quad's chunk 0; rows_of(xrow)
// fills this lane's token row of every tile -- a real row for every lane:
// lanes past the item's tokens repeat one of its rows, and their output
// columns are never stored -- and is called only after the first weight
// loads are in flight (it usually waits on an index load).  Each weight
// word is decoded once and feeds the NT tiles' MFMAs.
//
// Per step (CPS chunks): the x loads of this step, then the weight loads of
// the next step, then the MFMAs.  Loads complete in issue order, so the
// wait for x leaves the next step's weights in flight during the MFMAs.
// For that the loads must stay in this order (sched_barrier) and carry no
// conditions: a load skipped on some path makes the wait conservative, a
// full drain.  So every load is unconditional -- a partial last step loads
// its last chunk again (in the same step: a cache hit) and skips that
// chunk's MFMAs -- and the last step, which prefetches nothing, is peeled.
template <int NT, typename W, typename X, typename RowsFn>
__device__ inline void mfma_quad(const uint8_t* tiles, const uint8_t* tscales, RowsFn rows_of,
                                 int c_begin, int c_end, f32x4_t (&acc)[kGroups][NT]) {
    constexpr int CPS = Cps<NT, W>::value;
    const int lane = threadIdx.x % kWave, g = lane / 16;
    typename X::Row xrow[NT];
#pragma unroll
    for (int rg = 0; rg < kGroups; rg++)
#pragma unroll
        for (int t = 0; t < NT; t++) acc[rg][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (c_begin >= c_end) return;
    auto chunk_of = [&](int c0, int i) { return min(c0 + i, c_end - 1); };
    auto load_w = [&](int c0, WStep<W, CPS>& b) {
#pragma unroll
        for (int i = 0; i < CPS; i++) W::load(tiles, tscales, chunk_of(c0, i), b.c[i]);
    };
    auto load_x = [&](int c0, XStep<X, NT, CPS>& xb) {
#pragma unroll
        for (int i = 0; i < CPS; i++)
#pragma unroll
            for (int t = 0; t < NT; t++) X::load(xrow[t], chunk_of(c0, i), g, xb.x[i][t]);
    };
    auto compute = [&](int c0, const WStep<W, CPS>& b, const XStep<X, NT, CPS>& xb) {
#pragma unroll
        for (int i = 0; i < CPS; i++) {
            if (c0 + i >= c_end) break;  // the repeated chunk of a partial step
#pragma unroll
            for (int q = 0; q < 4; q++) {
#pragma unroll
                for (int rg = 0; rg < kGroups; rg++) {
                    const bf16x8_t A = W::a(b.c[i], rg, q);
#pragma unroll
                    for (int t = 0; t < NT; t++)
                        acc[rg][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, X::b(xb.x[i][t], q),
                                                                             acc[rg][t], 0, 0, 0);
                }
            }
        }
    };
    WStep<W, CPS> wa, wb;
    XStep<X, NT, CPS> xa;
    int c = c_begin;
    int left = (c_end - c_begin + CPS - 1) / CPS;  // steps
    load_w(c, wa);
    rows_of(xrow);
    while (left >= 3) {  // two steps, each with a successor to prefetch
        load_x(c, xa);
        __builtin_amdgcn_sched_barrier(0);
        load_w(c + CPS, wb);
        compute(c, wa, xa);
        c += CPS;
        load_x(c, xa);
        __builtin_amdgcn_sched_barrier(0);
        load_w(c + CPS, wa);
        compute(c, wb, xa);
        c += CPS;
        left -= 2;
    }
    if (left == 2) {
        load_x(c, xa);
        __builtin_amdgcn_sched_barrier(0);
        load_w(c + CPS, wb);
        compute(c, wa, xa);
        c += CPS;
        load_x(c, xa);
        compute(c, wb, xa);
    } else {
        load_x(c, xa);
        compute(c, wa, xa);
    }
}

// Sum the 4 waves' accumulators (split K) through LDS; wave 0 gets the total.
template <int NT>
__device__ inline void reduce_waves(f32x4_t (&acc)[kGroups][NT], f32x4_t* red) {
    const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
    if (w > 0) {
#pragma unroll
        for (int rg = 0; rg < kGroups; rg++)
#pragma unroll
            for (int t = 0; t < NT; t++)
                red[(((w - 1) * kGroups + rg) * NT + t) * kWave + lane] = acc[rg][t];
    }
    __syncthreads();
    if (w == 0) {
#pragma unroll
        for (int v = 1; v < kWaves; v++)
#pragma unroll
            for (int rg = 0; rg < kGroups; rg++)
#pragma unroll
                for (int t = 0; t < NT; t++)
                    acc[rg][t] += red[(((v - 1) * kGroups + rg) * NT + t) * kWave + lane];
    }
}

__device__ inline void wave_chunk_range(int chunks, int& c_begin, int& c_end) {
    const int per = (chunks + kWaves - 1) / kWaves;
    const int w = threadIdx.x / kWave;
    c_begin = min(chunks, w * per);
    c_end = min(chunks, c_begin + per);
}

// LDS for the cross-wave sums of single-tile items
constexpr int kRedGateUp = (kWaves - 1) * kGroups * kWave;
constexpr int kRedDown = 2 * kGroups * kWave;

// gate_up body for items of NT column tiles, token rows from `rows`
// (SortedRows, SlotRows, ListRows or TokenRows); gu/gus: the expert's
// gate_up tiles (format W), x and h in format X.
template <int NT, typename W, typename X, typename Rows>
__device__ inline void gate_up_item(const GemmArgs& a, int quad, const uint8_t* gu,
                                    const uint8_t* gus, const Rows& rows, f32x4_t* red) {
    const int lane = threadIdx.x % kWave, c = lane % 16, g = lane / 16;
    const int m = rows.m;
    const int chunks = a.H / 128;
    int cb, ce;
    wave_chunk_range(chunks, cb, ce);
    f32x4_t acc[kGroups][NT];
    mfma_quad<NT, W, X>(gu + (int64_t)quad * chunks * W::kChunkBytes,
                        gus + (int64_t)quad * chunks * 256,
                        [&](typename X::Row (&xrow)[NT]) {
#pragma unroll
                            for (int t = 0; t < NT; t++)
                                xrow[t] = X::row(a, rows.token(a, min(16 * t + c, m - 1)));
                        },
                        cb, ce, acc);
    reduce_waves<NT>(acc, red);
    if (threadIdx.x >= kWave) return;
#pragma unroll
    for (int t = 0; t < NT; t++) {
        const int j = 16 * t + c;
        if constexpr (!X::kMx8) {
            if (j >= m) continue;
            uint16_t* hrow = a.h + (int64_t)rows.row(j) * a.I + 32 * quad + 4 * g;
#pragma unroll
            for (int rg = 0; rg < 2; rg++) {
                ushort4 o;
                o.x = f32_to_bf16_rne(silu_mul(acc[rg][t][0], acc[rg + 2][t][0]));
                o.y = f32_to_bf16_rne(silu_mul(acc[rg][t][1], acc[rg + 2][t][1]));
                o.z = f32_to_bf16_rne(silu_mul(acc[rg][t][2], acc[rg + 2][t][2]));
                o.w = f32_to_bf16_rne(silu_mul(acc[rg][t][3], acc[rg + 2][t][3]));
                store_h4(hrow + 16 * rg, o);
            }
        } else {
            // h of this quad and token = one MX block of 32, held by lanes
            // (c, 0..3): they agree on its scale through two cross-lane
            // maxima (every lane takes part), then write their codes
            float hv[8];
            uint32_t amax = 0;
#pragma unroll
            for (int h2 = 0; h2 < 2; h2++)
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const float v = silu_mul(acc[h2][t][i], acc[h2 + 2][t][i]);
                    hv[4 * h2 + i] = v;
                    const uint32_t mb = __float_as_uint(v) & 0x7fffffffu;
                    amax = mb > amax ? mb : amax;
                }
            amax = max(amax, (uint32_t)__shfl_xor((int)amax, 16));
            amax = max(amax, (uint32_t)__shfl_xor((int)amax, 32));
            uint32_t code[2] = {0, 0};
            uint32_t scale = 255;
            if (amax < 0x7f800000u) {
                const int se = mxfp8_scale_exp(amax);
                scale = (uint32_t)(se + 127);
#pragma unroll
                for (int h2 = 0; h2 < 2; h2++)
#pragma unroll
                    for (int i = 0; i < 4; i++) code[h2] |= e4m3_code(hv[4 * h2 + i], se) << (8 * i);
            }
            if (j < m) {
                const int r = rows.row(j);
                uint8_t* hrow = a.hq + (int64_t)r * a.I + 32 * quad + 4 * g;
                *reinterpret_cast<uint32_t*>(hrow) = code[0];       // h 32q + 4g + i
                *reinterpret_cast<uint32_t*>(hrow + 16) = code[1];  // h 32q + 16 + 4g + i
                if (g == 0) a.hs[(int64_t)r * (a.I / 32) + quad] = (uint8_t)scale;
            }
        }
    }
}

// gate_up: blockIdx.x = item * quads + quad; quad q = gate rows 32q..32q+31
// (groups 0, 1) with up rows I+32q..I+32q+31 (groups 2, 3).  WIDE: items of
// up to kMfmaItemTok tokens (1..4 column tiles of 16); otherwise items of
// at most 16 tokens, compiled without the wider cases (fewer registers).
__global__ void __launch_bounds__(kMfmaThreads)
__attribute__((amdgpu_waves_per_eu(MOE_MFMA_WAVES_PER_EU)))
mfma_gate_up_kernel(GemmArgs a) {
    __shared__ f32x4_t red[kRedGateUp];
    const int quads = a.I / 32;
    const int item = blockIdx.x / quads, quad = blockIdx.x % quads;
    if (item >= uniform(a.meta[kMetaNumMfmaItems])) return;
    const int4 it = a.items[item];
    const int e = uniform(it.x), row0 = uniform(it.y), m = uniform(it.z);
    gate_up_item<1, W4, XB>(a, quad, a.wgu + (int64_t)e * (a.I / 32) * (a.H / 128) * 4096,
                            a.sgu + (int64_t)e * (a.I / 32) * (a.H / 128) * 256, SortedRows{row0, m}, red);
}

// down body for items of NT column tiles (see mfma_down_kernel), token rows
// from `rows`; dn/dns: the expert's down tiles (format W), h in format X;
// COMBINE: see store_down_tile
template <int NT, bool COMBINE, typename W, typename X, typename Rows>
__device__ inline void down_item(const GemmArgs& a, int pair, const uint8_t* dn,
                                 const uint8_t* dns, const Rows& rows, f32x4_t* red) {
    const int m = rows.m;
    const int quads = a.H / 64;
    const int w = threadIdx.x / kWave, half = w & 1;
    const int quad = pair * 2 + (w >> 1);
    const int lane = threadIdx.x % kWave, c = lane % 16;
    const int chunks = a.I / 128;
    const bool live = quad < quads;
    f32x4_t acc[kGroups][NT];
    if (live) {
        const int hc = (chunks + 1) / 2;
        mfma_quad<NT, W, X>(dn + (int64_t)quad * chunks * W::kChunkBytes,
                            dns + (int64_t)quad * chunks * 256,
                            [&](typename X::Row (&xrow)[NT]) {
#pragma unroll
                                for (int t = 0; t < NT; t++)
                                    xrow[t] = X::hrow(a, rows.row(min(16 * t + c, m - 1)));
                            },
                            half ? hc : 0, half ? chunks : hc, acc);
        if (half) {
#pragma unroll
            for (int rg = 0; rg < kGroups; rg++)
#pragma unroll
                for (int t = 0; t < NT; t++)
                    red[(((w >> 1) * kGroups + rg) * NT + t) * kWave + lane] = acc[rg][t];
        }
    }
    __syncthreads();
    if (!live || half) return;
#pragma unroll
    for (int rg = 0; rg < kGroups; rg++)
#pragma unroll
        for (int t = 0; t < NT; t++) acc[rg][t] += red[(((w >> 1) * kGroups + rg) * NT + t) * kWave + lane];
    store_down_tile<NT, COMBINE>(a, quad, rows, acc);
}

// down: a workgroup takes two quads (output rows 64q..64q+63), each split
// in two K halves over two waves; blockIdx.x = item * ceil(quads / 2) +
// pair.  The wave holding a quad's summed accumulator writes its y rows;
// the combine kernel reads them after this kernel.
__global__ void __launch_bounds__(kMfmaThreads)
__attribute__((amdgpu_waves_per_eu(MOE_MFMA_WAVES_PER_EU)))
mfma_down_kernel(GemmArgs a) {
    __shared__ f32x4_t red[kRedDown];
    const int quads = a.H / 64, pairs = (quads + 1) / 2;
    const int item = blockIdx.x / pairs, pair = blockIdx.x % pairs;
    if (item >= uniform(a.meta[kMetaNumMfmaItems])) return;
    const int4 it = a.items[item];
    const int e = uniform(it.x), row0 = uniform(it.y), m = uniform(it.z);
    down_item<1, false, W4, XB>(a, pair, a.wdn + (int64_t)e * (a.H / 64) * (a.I / 128) * 4096,
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
// slot, for the combine.  blockIdx.x = 1 + e * (I/32) + quad: gate_up quad
// `quad` of expert e, for the tokens that chose e, h rows by slot.
template <bool LISTS>
__global__ void __launch_bounds__(kMfmaThreads)
__attribute__((amdgpu_waves_per_eu(MOE_MFMA_WAVES_PER_EU)))
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
    const int e = (blockIdx.x - 1) / quads, quad = (blockIdx.x - 1) % quads;
    const auto rows = SelfRows<LISTS>::get(a, e);
    if (rows.m == 0) return;  // no token chose e
    gate_up_item<1, W4, XB>(a, quad, a.wgu + (int64_t)e * quads * (a.H / 128) * 4096,
                            a.sgu + (int64_t)e * quads * (a.H / 128) * 256, rows,
                            reinterpret_cast<f32x4_t*>(smem));
}

// blockIdx.x = e * ceil(H/128) + pair: the down quads 2*pair, 2*pair+1 of
// expert e for the tokens that chose it, y rows by slot.
template <bool LISTS>
__global__ void __launch_bounds__(kMfmaThreads)
__attribute__((amdgpu_waves_per_eu(MOE_MFMA_WAVES_PER_EU)))
self_down_kernel(GemmArgs a) {
    __shared__ f32x4_t red[kRedDown];
    const int pairs = (a.H / 64 + 1) / 2;
    const int e = blockIdx.x / pairs, pair = blockIdx.x % pairs;
    const auto rows = SelfRows<LISTS>::get(a, e);
    if (rows.m == 0) return;
    down_item<1, false, W4, XB>(a, pair, a.wdn + (int64_t)e * (a.H / 64) * (a.I / 128) * 4096,
                                a.sdn + (int64_t)e * (a.H / 64) * (a.I / 128) * 256, rows, red);
}

#ifndef MOE_FUSED_WAVES_PER_EU
#define MOE_FUSED_WAVES_PER_EU 2
#endif

// The expert layer after routing in one persistent launch: every workgroup
// dequeues units from one counter, first the gate_up units (item, quad),
// then the down units (item, quad pair), until the queue is exhausted.  A
// down unit first waits until all I/32 gate_up units of its item are done.
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
__attribute__((amdgpu_waves_per_eu(MOE_FUSED_WAVES_PER_EU)))
mfma_fused_kernel(GemmArgs a) {
    __shared__ f32x4_t red[2][kRedGateUp];
    __shared__ int s_unit[2];
    const int n_items = uniform(a.meta[kMetaNumMfmaItems]);
    const int gu_units = a.I / 32, dn_units = (a.H / 64 + 1) / 2;
    const int n_gu = n_items * gu_units, n_all = n_gu + n_items * dn_units;
    if (threadIdx.x == 0) s_unit[0] = atomicAdd(&a.queue[kQueueNext], 1);
    __syncthreads();
    for (int cur = 0;; cur ^= 1) {
        const int u = uniform(s_unit[cur]);
        if (u >= n_all) return;
        // read by every wave after this unit's barrier
        if (threadIdx.x == 0) s_unit[cur ^ 1] = atomicAdd(&a.queue[kQueueNext], 1);
        if (u < n_gu) {
            const int item = u / gu_units;
            const int4 it = a.items[item];
            const int64_t e = uniform(it.x);
            gate_up_item<1, W4, XB>(a, u % gu_units, a.wgu + e * gu_units * (a.H / 128) * 4096,
                                    a.sgu + e * gu_units * (a.H / 128) * 256,
                                    SortedRows{uniform(it.y), uniform(it.z)}, red[cur]);
            if (threadIdx.x < kWave) {  // wave 0 stored the h rows
                __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): they are complete
                if (threadIdx.x == 0) atomicAdd(&a.gu_done[item], 1);
            }
        } else {
            const int v = u - n_gu, item = v / dn_units;
            const int4 it = a.items[item];
            if (threadIdx.x == 0) wait_count(&a.gu_done[item], gu_units, &a.queue[kQueueError]);
            __syncthreads();
            const int64_t e = uniform(it.x);
            down_item<1, true, W4, XB>(a, v % dn_units, a.wdn + e * (a.H / 64) * (a.I / 128) * 4096,
                                       a.sdn + e * (a.H / 64) * (a.I / 128) * 256,
                                       SortedRows{uniform(it.y), uniform(it.z)}, red[cur]);
        }
    }
}

// ---- the shared expert: MXFP8 weights, every token.  The pages keep all
// but the MoE experts at 8 bits (bjdmk.com.cn news page, co-design
// section; yifor-blog digest, selective FP4 quantisation); a shared expert
// beside the routed ones is such a part.  Same quads, split-K waves and
// epilogues as the routed items, over 16-token tiles of all T tokens (h and
// y rows sh_row0 + t).  Unit u of `units` row units (gate_up quads or down
// quad pairs) and tile of `tiles`: blockIdx = x + 8 * (tile + tiles * g)
// with unit 8g + x, so the tiles of one unit run on one XCD (blockIdx mod 8)
// one after another, and its weights come from HBM about once.
__device__ inline bool shared_unit(int units, int tiles, int& unit, int& tile) {
    const int x = blockIdx.x % 8, r = blockIdx.x / 8;
    tile = r % tiles;
    unit = 8 * (r / tiles) + x;
    return unit < units;
}

template <typename X>
__global__ void __launch_bounds__(kMfmaThreads)
__attribute__((amdgpu_waves_per_eu(MOE_MFMA_WAVES_PER_EU)))
shared_gate_up_kernel(GemmArgs a) {
    __shared__ f32x4_t red[kRedGateUp];
    int quad, tile;
    if (!shared_unit(a.I / 32, (a.T + 15) / 16, quad, tile)) return;
    const int t0 = 16 * tile;
    gate_up_item<1, W8, X>(a, quad, a.sh_wgu, a.sh_sgu, TokenRows{t0, min(16, a.T - t0), a.sh_row0},
                           red);
}

template <typename X>
__global__ void __launch_bounds__(kMfmaThreads)
__attribute__((amdgpu_waves_per_eu(MOE_MFMA_WAVES_PER_EU)))
shared_down_kernel(GemmArgs a) {
    __shared__ f32x4_t red[kRedDown];
    int pair, tile;
    if (!shared_unit((a.H / 64 + 1) / 2, (a.T + 15) / 16, pair, tile)) return;
    const int t0 = 16 * tile;
    down_item<1, false, W8, X>(a, pair, a.sh_wdn, a.sh_sdn, TokenRows{t0, min(16, a.T - t0), a.sh_row0},
                               red);
}

}  // namespace

hipError_t launch_shared_gate_up(const GemmArgs& a, bool mx8, hipStream_t stream) {
    const int grid = 8 * ((a.T + 15) / 16) * ((a.I / 32 + 7) / 8);
    if (mx8)
        shared_gate_up_kernel<X8><<<grid, kMfmaThreads, 0, stream>>>(a);
    else
        shared_gate_up_kernel<XB><<<grid, kMfmaThreads, 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_shared_down(const GemmArgs& a, bool mx8, hipStream_t stream) {
    const int grid = 8 * ((a.T + 15) / 16) * (((a.H / 64 + 1) / 2 + 7) / 8);
    if (mx8)
        shared_down_kernel<X8><<<grid, kMfmaThreads, 0, stream>>>(a);
    else
        shared_down_kernel<XB><<<grid, kMfmaThreads, 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_mfma_gate_up(const GemmArgs& a, int max_items, hipStream_t stream) {
    const int quads = a.I / 32;
    mfma_gate_up_kernel<<<max_items * quads, kMfmaThreads, 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_mfma_down(const GemmArgs& a, int max_items, hipStream_t stream) {
    const int pairs = (a.H / 64 + 1) / 2;
    mfma_down_kernel<<<max_items * pairs, kMfmaThreads, 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_self_gate_up(const GemmArgs& a, bool lists, hipStream_t stream) {
    const int grid = 1 + a.E * (a.I / 32);
    if (lists)
        self_gate_up_kernel<true><<<grid, kMfmaThreads, 0, stream>>>(a);
    else
        self_gate_up_kernel<false><<<grid, kMfmaThreads, 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_self_down(const GemmArgs& a, bool lists, hipStream_t stream) {
    const int grid = a.E * ((a.H / 64 + 1) / 2);
    if (lists)
        self_down_kernel<true><<<grid, kMfmaThreads, 0, stream>>>(a);
    else
        self_down_kernel<false><<<grid, kMfmaThreads, 0, stream>>>(a);
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
