// mfma_items.h -- the split-K expert GEMM bodies on the bf16 matrix cores
// (weight formats of the tile layout, activation formats, the per-wave quad
// loop, the gate_up and down item bodies, and the shared expert's blocks),
// used by the kernels of mfma.hip and, for the shared expert's blocks, by
// the wide kernels.  See mfma.hip for the tile layout and the
// MFMA operand mapping.
#pragma once

#include "device_common.h"

namespace moe {
namespace {

constexpr int kMfmaWavesPerEu = 2;            // launch bound: at least 2 waves per SIMD
constexpr int kWaves = kMfmaThreads / kWave;  // 4, split K
constexpr int kChunksPerStep = 2;             // 128-column chunks per prefetch step
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
    // as the A operand of the scaled FP4 x FP8 matrix cores: the lane's 32
    // codes as they are (format 4 = FP4 E2M1); byte rg of s is its block scale
    static constexpr int kFmt = 4;
    static __device__ i32x8_t sop(const Chunk& b, int rg) {
        const uint4& w = b.w[rg];
        return i32x8_t{(int)w.x, (int)w.y, (int)w.z, (int)w.w, 0, 0, 0, 0};
    }
};
// W8P: MXFP8 weights (the MXFP8 tile layout) as the A operand of the scaled
// matrix cores: an 8-bit A operand gives lane (r, g) the 16-byte pieces g
// and g + 4 of row r's 128 codes, with the scale of MX block g (the pairing
// of the B operand); in the MXFP8 tile layout piece p of row r sits in half
// p % 2 of lane r + 16 (p / 2), so the lane loads those two 16-byte pieces.
struct W8P {
    static constexpr int kChunkBytes = 8192;
    static constexpr int kFmt = 0;  // FP8 E4M3
    struct Chunk {
        uint4 w[kGroups][2];
        uint32_t s;
    };
    static __device__ void load(const uint8_t* tiles, const uint8_t* tscales, int ci, Chunk& b) {
        const int lane = threadIdx.x % kWave, r = lane % 16, g = lane / 16;
        const uint8_t* t = tiles + (int64_t)ci * kChunkBytes + (g & 1) * 1024 + (r + 16 * (g >> 1)) * 16;
#pragma unroll
        for (int rg = 0; rg < kGroups; rg++) {
            b.w[rg][0] = load_stream16(t + rg * 2048);        // piece g
            b.w[rg][1] = load_stream16(t + rg * 2048 + 512);  // piece g + 4: lane r + 16 (g / 2 + 2)
        }
        b.s = *reinterpret_cast<const uint32_t*>(tscales + (int64_t)ci * 256 + lane * 4);
    }
    static __device__ i32x8_t sop(const Chunk& b, int rg) {
        const uint4& lo = b.w[rg][0];
        const uint4& hi = b.w[rg][1];
        return i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
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

// ---- the activation format of the B operand (one token row, 128-k
// chunk).  XB: bf16 rows of x (row(a, token)); lane (c, g) takes block g of
// the chunk and b(x, q) is the bf16 B operand of step q (elements
// 8q..8q+7 of the block).  XQ3: rows of h as three MXFP8 terms (store_h3,
// hrow(a, r)) for the scaled matrix cores; term(x, tm) is lane (c, g)'s
// 32 codes of term tm and byte tm of its s the block scale.
struct XB {
    static constexpr bool kScaled = false;
    struct Row {
        const uint16_t* p;
    };
    struct Chunk {
        uint4 x[4];
    };
    static __device__ Row row(const GemmArgs& a, int t) { return Row{a.x + (int64_t)t * a.H}; }
    static __device__ void load(const Row& r, int chunk, int g, Chunk& c) {
        const uint4* src = reinterpret_cast<const uint4*>(r.p + (int64_t)(4 * chunk + g) * 32);
#pragma unroll
        for (int q = 0; q < 4; q++) c.x[q] = src[q];
    }
    static __device__ bf16x8_t b(const Chunk& c, int q) { return __builtin_bit_cast(bf16x8_t, c.x[q]); }
};
struct XQ3 {
    static constexpr bool kScaled = true;
    struct Row {
        const uint8_t* q;  // codes of the row
        const uint8_t* s;  // scales of the row
    };
    struct Chunk {
        uint4 x[2 * kHTerms];
        uint32_t s;
    };
    static __device__ Row hrow(const GemmArgs& a, int r) {
        return Row{a.h3q + (int64_t)r * 3 * a.I, a.h3s + (int64_t)r * h3s_stride(a.I)};
    }
    static __device__ void load(const Row& r, int chunk, int g, Chunk& c) {
        const uint4* src = reinterpret_cast<const uint4*>(r.q + (chunk * 4 + g) * 96);
#pragma unroll
        for (int i = 0; i < 2 * kHTerms; i++) c.x[i] = src[i];
        c.s = *reinterpret_cast<const uint32_t*>(r.s + (chunk * 4 + g) * 4);
    }
    static __device__ i32x8_t term(const Chunk& c, int tm) {
        const uint4& lo = c.x[2 * tm];
        const uint4& hi = c.x[2 * tm + 1];
        return i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
};
// chunks per prefetch step: MXFP4 weights against one column tile
// kChunksPerStep; wider items one (their B operands alone fill 16 or 25
// VGPRs per tile and chunk); MXFP8 weights one (a chunk is already twice
// the bytes)
template <int NT, typename W, typename X>
struct Cps {
    static constexpr int value = W::kChunkBytes != 4096 || NT != 1 || X::kScaled ? 1 : kChunksPerStep;
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
    constexpr int CPS = Cps<NT, W, X>::value;
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
            if constexpr (X::kScaled) {  // one scaled MFMA per group, tile and term
                // terms outermost: consecutive MFMAs go to different accumulators
                static_for<kHTerms>([&](auto tm) {
#pragma unroll
                    for (int t = 0; t < NT; t++) {
                        const i32x8_t B = X::term(xb.x[i][t], tm);
                        static_for<kGroups>([&](auto rg) {
                            acc[rg][t] = mfma_scaled<W::kFmt, rg, tm>(W::sop(b.c[i], rg), B, acc[rg][t],
                                                                      b.c[i].s, xb.x[i][t].s);
                        });
                    }
                });
            } else {
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
        }
    };
    WStep<W, CPS> wa, wb;
    XStep<X, NT, CPS> xa;
    int c = c_begin;
    int left = (c_end - c_begin + CPS - 1) / CPS;  // steps
    load_w(c, wa);
    rows_of(xrow);
    if constexpr (X::kScaled) {
        // h (three terms per chunk) one step ahead as well: a step waits
        // only for loads issued a step earlier (its B operand's latency is
        // the loop's floor otherwise; the weights alone come from HBM)
        XStep<X, NT, CPS> xb;
        load_x(c, xa);
        while (left >= 3) {
            load_w(c + CPS, wb);
            load_x(c + CPS, xb);
            compute(c, wa, xa);
            c += CPS;
            load_w(c + CPS, wa);
            load_x(c + CPS, xa);
            compute(c, wb, xb);
            c += CPS;
            left -= 2;
        }
        if (left == 2) {
            load_w(c + CPS, wb);
            load_x(c + CPS, xb);
            compute(c, wa, xa);
            c += CPS;
            compute(c, wb, xb);
        } else {
            compute(c, wa, xa);
        }
        return;
    }
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

// The SiLU(gate) * up epilogue of a gate_up quad: acc[rg][t] of lane
// (c, g) holds rows 4g..4g+3 of group rg for token row 16t + c; groups 0, 1
// are gate rows 32*quad + 16*rg + 4g + i, groups 2, 3 the matching up rows,
// so the lane forms h elements 32*quad + 16*rg + 4g .. +3 of its token's h
// row (rows.row), h block `quad`, stored as three MXFP8 terms (PUBLISH:
// for readers in the same launch, see store_h3).
template <int NT, bool PUBLISH, typename Rows>
__device__ inline void store_h_tile(const GemmArgs& a, int quad, const Rows& rows,
                                    const f32x4_t (&acc)[kGroups][NT]) {
    const int c = threadIdx.x % 16;
#pragma unroll
    for (int t = 0; t < NT; t++) {
        const int j = 16 * t + c;
        float v[2][4];
#pragma unroll
        for (int rg = 0; rg < 2; rg++)
#pragma unroll
            for (int i = 0; i < 4; i++) v[rg][i] = silu_mul(acc[rg][t][i], acc[rg + 2][t][i]);
        store_h3<PUBLISH>(a, rows.row(min(j, rows.m - 1)), quad, v, j < rows.m);
    }
}

// gate_up body for items of NT column tiles, token rows from `rows`
// (SortedRows, SlotRows, ListRows or TokenRows); gu/gus: the expert's
// gate_up tiles (format W), x in format X; h goes out as three MXFP8 terms
// (PUBLISH: for a down unit of the same launch).
template <int NT, typename W, typename X, bool PUBLISH = false, typename Rows>
__device__ inline void gate_up_item(const GemmArgs& a, int quad, const uint8_t* gu,
                                    const uint8_t* gus, const Rows& rows, f32x4_t* red) {
    const int c = threadIdx.x % 16;
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
    store_h_tile<NT, PUBLISH>(a, quad, rows, acc);
}

// down body for items of NT column tiles (see mfma_down_kernel), token rows
// from `rows`; dn/dns: the expert's down tiles (format W: W4, or W8P for
// MXFP8 weights), h as three MXFP8 terms on the scaled matrix cores (XQ3);
// PUBLISH: see store_down_tile
template <int NT, bool PUBLISH, typename W, typename Rows>
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
        mfma_quad<NT, W, XQ3>(dn + (int64_t)quad * chunks * W::kChunkBytes,
                              dns + (int64_t)quad * chunks * 256,
                              [&](XQ3::Row (&xrow)[NT]) {
#pragma unroll
                                  for (int t = 0; t < NT; t++)
                                      xrow[t] = XQ3::hrow(a, rows.row(min(16 * t + c, m - 1)));
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
    store_down_tile<NT, PUBLISH>(a, quad, rows, acc);
}

// ---- the shared expert: MXFP8 weights, every token.  The pages keep all
// but the MoE experts at 8 bits (bjdmk.com.cn news page, co-design
// section; yifor-blog digest, selective FP4 quantisation); a shared expert
// beside the routed ones is such a part.  Same quads, split-K waves and
// epilogues as the routed items, over tiles of 16 * NT of the T tokens (h
// and y rows sh_row0 + t).  Block b of the shared blocks takes unit u of
// `units` row units (gate_up quads or down quad pairs) and tile `tile`:
// b = x + 8 * (tile + tiles * g) with u = 8g + x, so the tiles of one unit
// run on one XCD (block index mod 8) one after another, and its weights
// come from HBM about once (the prefill kernels map their one-quad blocks
// the same way).  The shared blocks are a multiple of 8 and come ahead of
// the routed blocks of the same launch (self-routed, split and wide
// kernels), or form a launch of their own (mfma.hip).
__device__ inline bool shared_unit(int b, int units, int tiles, int& unit, int& tile) {
    const int x = b % 8, r = b / 8;
    tile = r % tiles;
    unit = 8 * (r / tiles) + x;
    return unit < units;
}

__host__ __device__ inline int shared_blocks(int units, int tiles) { return 8 * tiles * ((units + 7) / 8); }

template <int NT, typename X>
__device__ inline void shared_gate_up_block(const GemmArgs& a, int b, f32x4_t* red) {
    const int tok = 16 * NT;
    int quad, tile;
    if (!shared_unit(b, a.I / 32, (a.T + tok - 1) / tok, quad, tile)) return;
    const int t0 = tok * tile;
    gate_up_item<NT, W8, X>(a, quad, a.sh_wgu, a.sh_sgu, TokenRows{t0, min(tok, a.T - t0), a.sh_row0},
                            red);
}

template <int NT>
__device__ inline void shared_down_block(const GemmArgs& a, int b, f32x4_t* red) {
    const int tok = 16 * NT;
    int pair, tile;
    if (!shared_unit(b, (a.H / 64 + 1) / 2, (a.T + tok - 1) / tok, pair, tile)) return;
    const int t0 = tok * tile;
    down_item<NT, false, W8P>(a, pair, a.sh_wdn, a.sh_sdn, TokenRows{t0, min(tok, a.T - t0), a.sh_row0},
                              red);
}

}  // namespace
}  // namespace moe
