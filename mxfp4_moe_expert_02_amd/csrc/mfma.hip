// mfma.hip -- MXFP4 expert GEMMs on the bf16 matrix cores of gfx950.
//
// The weight bytes are the cost of this layer (the pages quantise the MoE
// experts to 4 bits because the decode of a 1T model is bound by weight
// I/O: bjdmk.com.cn news page, co-design section; yifor-blog digest,
// memory-bandwidth section).  The VALU path (gemv.hip) spends about one
// VALU instruction per weight element on the dot products; here the
// products and the K reduction go to v_mfma_f32_16x16x32_bf16 and the VALU
// only decodes: one v_cvt_scalef32_pk_bf16_fp4 per two elements, with the
// E8M0 block scale applied in the same instruction (E2M1 * 2^k is exact in
// bf16).  Activations stay bf16 and accumulation fp32, as in the VALU path.
//
// Operand mapping for one 16x16x32 MFMA (A = 16 weight rows x 32 k,
// B = 32 k x 16 tokens, D = 16 rows x 16 tokens):
//   lane l = (r = l % 16, g = l / 16).  An iteration covers four MX blocks
//   of every row; lane (r, g) loads block 4*it + g of row r with one 128-bit
//   load and feeds its 4 words to 4 successive MFMAs (word q = elements
//   8q..8q+7).  The B lane (c, g) supplies the same 8 k values of token c,
//   read straight from global memory (16 bytes, an L1/L2 hit: every tile of
//   the expert reads the same few token rows).  D lane (c, g) holds rows
//   4g..4g+3 of token c.
// The 4 waves of a workgroup split K in four contiguous ranges and add
// their 16x16 accumulators through LDS at the end; no barrier is needed
// while the weights stream.
//
// Items come from the route: (expert slot, first token) with up to 16
// tokens each; tokens beyond the item's count are zero columns.
#include "device_common.h"

namespace moe {
namespace {

constexpr int kWaves = kMfmaThreads / kWave;  // 4, split K
constexpr int kIterPerStep = 2;               // 4-block iterations per prefetch step

// E8M0 code as the fp32 scale operand of v_cvt_scalef32_* (the code in the
// exponent field: 2^(s-127) for s in 1..254)
__device__ inline float e8m0_as_scale(uint32_t s) { return __uint_as_float(s << 23); }

// 8 E2M1 codes of one word (element 2i in the low nibble of byte i) -> 8 bf16
__device__ inline bf16x8_t decode8(uint32_t word, float scale) {
    const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 0);
    const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 1);
    const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 2);
    const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 3);
    return bf16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

__device__ inline uint32_t word_of(const uint4& v, int q) {
    return q == 0 ? v.x : q == 1 ? v.y : q == 2 ? v.z : v.w;
}

template <int R16>
struct WStep {
    uint4 w[kIterPerStep][R16];
    uint32_t s[kIterPerStep][R16];
};

struct XStep {
    uint4 x[kIterPerStep][4];
};

// Streams this wave's K range of R16 row groups against up to 16 tokens.
// rows[rg] / srows[rg]: packed row and scale row of this lane's row r in
// group rg.  xrow: this lane's token row (bf16), or null for a zero column.
template <int R16>
__device__ inline void mfma_rows(const uint8_t* const (&rows)[R16],
                                 const uint8_t* const (&srows)[R16], const uint16_t* xrow,
                                 int it_begin, int it_end, int nblk, f32x4_t (&acc)[R16]) {
    const int g = (threadIdx.x % kWave) / 16;
#pragma unroll
    for (int rg = 0; rg < R16; rg++) acc[rg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    auto load_w = [&](int it0, WStep<R16>& b) {
#pragma unroll
        for (int i = 0; i < kIterPerStep; i++) {
            const int blk = 4 * (it0 + i) + g;
            const bool ok = (it0 + i < it_end) && blk < nblk;
#pragma unroll
            for (int rg = 0; rg < R16; rg++) {
                b.w[i][rg] = ok ? load_stream16(rows[rg] + (int64_t)blk * 16) : make_uint4(0, 0, 0, 0);
                b.s[i][rg] = ok ? srows[rg][blk] : 127u;
            }
        }
    };
    auto load_x = [&](int it0, XStep& xb) {
#pragma unroll
        for (int i = 0; i < kIterPerStep; i++) {
            const int blk = 4 * (it0 + i) + g;
            const bool ok = xrow && (it0 + i < it_end) && blk < nblk;
            const uint4* src = reinterpret_cast<const uint4*>(xrow + (int64_t)blk * 32);
#pragma unroll
            for (int q = 0; q < 4; q++) xb.x[i][q] = ok ? src[q] : make_uint4(0, 0, 0, 0);
        }
    };
    auto compute = [&](const WStep<R16>& b, const XStep& xb) {
#pragma unroll
        for (int i = 0; i < kIterPerStep; i++) {
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const bf16x8_t B = __builtin_bit_cast(bf16x8_t, xb.x[i][q]);
#pragma unroll
                for (int rg = 0; rg < R16; rg++) {
                    const bf16x8_t A = decode8(word_of(b.w[i][rg], q), e8m0_as_scale(b.s[i][rg]));
                    acc[rg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, acc[rg], 0, 0, 0);
                }
            }
        }
    };
    WStep<R16> wa, wb;
    XStep xa;
    int it = it_begin;
    if (it < it_end) load_w(it, wa);
    while (it < it_end) {
        const int nxt = it + kIterPerStep;
        if (nxt < it_end) load_w(nxt, wb);  // prefetch the next step's weights
        load_x(it, xa);
        compute(wa, xa);
        it = nxt;
        if (it >= it_end) break;
        const int nxt2 = it + kIterPerStep;
        if (nxt2 < it_end) load_w(nxt2, wa);
        load_x(it, xa);
        compute(wb, xa);
        it = nxt2;
    }
}

// Sum the 4 waves' accumulators (split K) through LDS; wave 0 gets the total.
template <int R16>
__device__ inline void reduce_waves(f32x4_t (&acc)[R16], f32x4_t* red) {
    const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
    if (w > 0) {
#pragma unroll
        for (int rg = 0; rg < R16; rg++) red[((w - 1) * R16 + rg) * kWave + lane] = acc[rg];
    }
    __syncthreads();
    if (w == 0) {
#pragma unroll
        for (int v = 1; v < kWaves; v++)
#pragma unroll
            for (int rg = 0; rg < R16; rg++) acc[rg] += red[((v - 1) * R16 + rg) * kWave + lane];
    }
}

__device__ inline void wave_k_range(int nblk, int& it_begin, int& it_end) {
    const int iters = (nblk + 3) / 4;
    const int per = (iters + kWaves - 1) / kWaves;
    const int w = threadIdx.x / kWave;
    it_begin = min(iters, w * per);
    it_end = min(iters, it_begin + per);
}

// gate_up: blockIdx.x = item * tiles + tile; a tile is kMfmaRows gate rows
// and the matching up rows (group 0 = gate, group 1 = up).
__global__ void __launch_bounds__(kMfmaThreads)
mfma_gate_up_kernel(GemmArgs a) {
    __shared__ f32x4_t red[(kWaves - 1) * 2 * kWave];
    const int tiles = a.I / kMfmaRows;
    const int item = blockIdx.x / tiles, tile = blockIdx.x % tiles;
    if (item >= uniform(a.meta[kMetaNumMfmaItems])) return;
    const int2 it2 = a.items[item];
    const int slot = uniform(it2.x), tok0 = uniform(it2.y);
    const int e = uniform(a.list[slot]);
    const int M = uniform(a.counts[e]), off = uniform(a.offsets[e]);
    const int m = min(kMfmaTok, M - tok0);
    const int lane = threadIdx.x % kWave, r = lane % 16, c = lane % 16, g = lane / 16;
    const int K = a.H, nblk = K / 32;
    const int n = tile * kMfmaRows + r;
    const uint8_t* W = a.wgu + (int64_t)e * (2 * a.I) * (K / 2);
    const uint8_t* S = a.sgu + (int64_t)e * (2 * a.I) * nblk;
    const uint8_t* rows[2] = {W + (int64_t)n * (K / 2), W + (int64_t)(a.I + n) * (K / 2)};
    const uint8_t* srows[2] = {S + (int64_t)n * nblk, S + (int64_t)(a.I + n) * nblk};
    const uint16_t* xrow = nullptr;
    if (c < m) xrow = a.x + (int64_t)(a.sorted[off + tok0 + c] / a.k) * K;
    int ib, ie;
    wave_k_range(nblk, ib, ie);
    f32x4_t acc[2];
    mfma_rows<2>(rows, srows, xrow, ib, ie, nblk, acc);
    reduce_waves<2>(acc, red);
    if (threadIdx.x < kWave && c < m) {
        // rows 4g..4g+3 of this tile, token c
        ushort4 o;
        o.x = f32_to_bf16_rne(silu_mul(acc[0][0], acc[1][0]));
        o.y = f32_to_bf16_rne(silu_mul(acc[0][1], acc[1][1]));
        o.z = f32_to_bf16_rne(silu_mul(acc[0][2], acc[1][2]));
        o.w = f32_to_bf16_rne(silu_mul(acc[0][3], acc[1][3]));
        *reinterpret_cast<ushort4*>(a.h + (int64_t)(off + tok0 + c) * a.I + tile * kMfmaRows +
                                    4 * g) = o;
    }
}

// down: blockIdx.x = item * tiles + tile; a tile is kMfmaDownRows output
// rows (two groups of 16), which is also the combine tile: the block that
// completes a token's k experts on this tile combines it (see gemv.hip).
__global__ void __launch_bounds__(kMfmaThreads)
mfma_down_kernel(GemmArgs a) {
    __shared__ f32x4_t red[(kWaves - 1) * 2 * kWave];
    __shared__ int s_combine[kMfmaTok];
    const int tiles = a.H / kMfmaDownRows;
    const int item = blockIdx.x / tiles, tile = blockIdx.x % tiles;
    if (item >= uniform(a.meta[kMetaNumMfmaItems])) return;
    const int2 it2 = a.items[item];
    const int slot = uniform(it2.x), tok0 = uniform(it2.y);
    const int e = uniform(a.list[slot]);
    const int M = uniform(a.counts[e]), off = uniform(a.offsets[e]);
    const int m = min(kMfmaTok, M - tok0);
    const int lane = threadIdx.x % kWave, r = lane % 16, c = lane % 16, g = lane / 16;
    const int K = a.I, nblk = K / 32;
    const int n0 = tile * kMfmaDownRows;
    const uint8_t* W = a.wdn + (int64_t)e * a.H * (K / 2);
    const uint8_t* S = a.sdn + (int64_t)e * a.H * nblk;
    const uint8_t* rows[2] = {W + (int64_t)(n0 + r) * (K / 2), W + (int64_t)(n0 + 16 + r) * (K / 2)};
    const uint8_t* srows[2] = {S + (int64_t)(n0 + r) * nblk, S + (int64_t)(n0 + 16 + r) * nblk};
    const uint16_t* xrow = (c < m) ? a.h + (int64_t)(off + tok0 + c) * K : nullptr;
    int ib, ie;
    wave_k_range(nblk, ib, ie);
    f32x4_t acc[2];
    mfma_rows<2>(rows, srows, xrow, ib, ie, nblk, acc);
    reduce_waves<2>(acc, red);
    if (threadIdx.x < kWave && c < m) {
        float* dst = a.y + (int64_t)(off + tok0 + c) * a.H + n0 + 4 * g;
#pragma unroll
        for (int rg = 0; rg < 2; rg++) {
            // agent-coherent stores: the combining block may run on another XCD
            const uint64_t lo = (uint64_t)__float_as_uint(acc[rg][0]) |
                                ((uint64_t)__float_as_uint(acc[rg][1]) << 32);
            const uint64_t hi = (uint64_t)__float_as_uint(acc[rg][2]) |
                                ((uint64_t)__float_as_uint(acc[rg][3]) << 32);
            __hip_atomic_store(reinterpret_cast<uint64_t*>(dst + 16 * rg), lo, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(reinterpret_cast<uint64_t*>(dst + 16 * rg + 2), hi,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");  // this wave's y stores done
    __syncthreads();
    if (threadIdx.x < m) {
        const int token = a.sorted[off + tok0 + threadIdx.x] / a.k;
        const int old = atomicAdd(&a.tile_done[token * tiles + tile], 1);
        s_combine[threadIdx.x] = (old == a.k - 1) ? token : -1;
    }
    __syncthreads();
    for (int i = 0; i < m; i++) {
        const int token = uniform(s_combine[i]);
        if (token >= 0) combine_tile(a, token, n0, kMfmaDownRows);
    }
}

}  // namespace

hipError_t launch_mfma_gate_up(const GemmArgs& a, int max_items, hipStream_t stream) {
    const int tiles = a.I / kMfmaRows;
    mfma_gate_up_kernel<<<max_items * tiles, kMfmaThreads, 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_mfma_down(const GemmArgs& a, int max_items, hipStream_t stream) {
    const int tiles = a.H / kMfmaDownRows;
    mfma_down_kernel<<<max_items * tiles, kMfmaThreads, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace moe
