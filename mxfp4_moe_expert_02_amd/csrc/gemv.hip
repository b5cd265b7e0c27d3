// gemv.hip -- MXFP4 expert GEMV for few tokens per expert (gfx950, VALU).
//
// At verify token counts an expert sees a handful of tokens, so each expert
// matrix is read once from HBM and the arithmetic per weight byte is tiny;
// the pages put the decode cost of a 1T MoE in weight I/O and quantise the
// experts to 4 bits for exactly that reason (bjdmk.com.cn news page,
// co-design section; yifor-blog digest, memory-bandwidth section).
//
// Mapping (one work item = one expert x a tile of rows):
//   * 16 lanes (one DPP row) share a matrix row; lane i of the 16 reads
//     MX blocks i, i+16, i+32, ... of that row with 128-bit loads, so one
//     wave-wide load moves 4 rows x 256 contiguous bytes.  The E8M0 scale
//     of each block is one byte load from the scale row.
//   * The item's activation tile (up to 4 tokens x K bf16) is staged once in
//     LDS and shared by every row of the item; the 16-byte quarters of each
//     block are rotated by (block/2)%4 so that the 8 lanes of one LDS pass
//     hit 8 different bank groups.
//   * E2M1 pairs are decoded to bf16 pairs with v_cvt_scalef32_pk_bf16_fp4
//     (scale 1: exact), multiplied into the bf16 activation pairs with
//     v_dot2c_f32_bf16 into an fp32 partial per block, and the partial is
//     scaled by 2^(s-127) (exact) into the fp32 accumulator.
//   * The K-reduction across the 16 lanes is a DPP rotate butterfly
//     (row_ror 8, 4, 2, 1), leaving the sum in every lane.
// gate_up items also apply SiLU(gate) * up and store h in bf16; down items
// store the per-assignment outputs y in fp32.
#include "moe_internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte streaming load (the weights are read exactly once)
__device__ inline uint4 load_stream16(const uint8_t* p) {
    u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ inline bf16x2_t as_bf16x2(uint32_t u) { return __builtin_bit_cast(bf16x2_t, u); }

// sum over the 16 lanes of a DPP row, result in all 16 lanes
__device__ inline float row16_sum(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                               0x128, 0xf, 0xf, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                               0x124, 0xf, 0xf, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                               0x122, 0xf, 0xf, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                               0x121, 0xf, 0xf, false));
    return v;
}

// E8M0 code -> 2^(s-127) as fp32 (2^-127 is an fp32 subnormal; 0xFF -> NaN)
__device__ inline float e8m0_to_f32(uint32_t s) {
    float f = ldexpf(1.0f, (int)s - 127);
    return s == 255u ? __builtin_nanf("") : f;
}

__device__ inline float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

__device__ inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// LDS position (in 16-byte units) of quarter q of block b of a token row
__device__ inline int xs_unit(int b, int q) { return b * 4 + ((q + (b >> 1)) & 3); }

// Stage rows of bf16 activations into LDS: dst[t][...] for t < M, each row
// K elements, taken from src + row_index(t) * ld.  16-byte granularity.
template <typename RowFn>
__device__ inline void stage_rows(uint4* __restrict__ xs, int M, int K, RowFn row_ptr) {
    const int units = K / 8;  // 16-byte units per row
    for (int i = threadIdx.x; i < M * units; i += blockDim.x) {
        int t = i / units, u = i % units;
        const uint4* src = reinterpret_cast<const uint4*>(row_ptr(t));
        xs[t * units + xs_unit(u >> 2, u & 3)] = src[u];
    }
}

// Dot products of R matrix rows with MT staged tokens, for this lane's
// blocks of the rows.  rows[r] points at the packed row, srows[r] at its
// scale row.  Returns per-lane partial sums in acc (not yet reduced).
template <int MT, int R>
__device__ inline void rows_dot(const uint8_t* const (&rows)[R], const uint8_t* const (&srows)[R],
                                int nblk, const uint4* __restrict__ xs, int units_per_tok,
                                int lane16, float (&acc)[R][MT]) {
#pragma unroll
    for (int r = 0; r < R; r++)
#pragma unroll
        for (int t = 0; t < MT; t++) acc[r][t] = 0.f;

    for (int b0 = lane16; b0 < nblk; b0 += kGemvLanesPerRow * kGemvUnroll) {
        uint4 w[kGemvUnroll][R];
        uint32_t s[kGemvUnroll][R];
#pragma unroll
        for (int u = 0; u < kGemvUnroll; u++) {
            int b = b0 + u * kGemvLanesPerRow;
#pragma unroll
            for (int r = 0; r < R; r++) {
                if (b < nblk) {
                    w[u][r] = load_stream16(rows[r] + (int64_t)b * 16);
                    s[u][r] = srows[r][b];
                } else {
                    w[u][r] = make_uint4(0, 0, 0, 0);
                    s[u][r] = 127;
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kGemvUnroll; u++) {
            int b = b0 + u * kGemvLanesPerRow;
            if (b >= nblk) break;
            float part[R][MT];
#pragma unroll
            for (int r = 0; r < R; r++)
#pragma unroll
                for (int t = 0; t < MT; t++) part[r][t] = 0.f;
#pragma unroll
            for (int q = 0; q < 4; q++) {
                uint4 xv[MT];
#pragma unroll
                for (int t = 0; t < MT; t++) xv[t] = xs[t * units_per_tok + xs_unit(b, q)];
#pragma unroll
                for (int r = 0; r < R; r++) {
                    uint32_t word = (q == 0) ? w[u][r].x : (q == 1) ? w[u][r].y
                                  : (q == 2) ? w[u][r].z : w[u][r].w;
                    // byte j of the word holds elements 2j (low nibble), 2j+1
                    bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, 1.0f, 0);
                    bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, 1.0f, 1);
                    bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, 1.0f, 2);
                    bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, 1.0f, 3);
#pragma unroll
                    for (int t = 0; t < MT; t++) {
                        float a = part[r][t];
                        a = __builtin_amdgcn_fdot2_f32_bf16(p0, as_bf16x2(xv[t].x), a, false);
                        a = __builtin_amdgcn_fdot2_f32_bf16(p1, as_bf16x2(xv[t].y), a, false);
                        a = __builtin_amdgcn_fdot2_f32_bf16(p2, as_bf16x2(xv[t].z), a, false);
                        a = __builtin_amdgcn_fdot2_f32_bf16(p3, as_bf16x2(xv[t].w), a, false);
                        part[r][t] = a;
                    }
                }
            }
#pragma unroll
            for (int r = 0; r < R; r++) {
                float sc = e8m0_to_f32(s[u][r]);
#pragma unroll
                for (int t = 0; t < MT; t++) acc[r][t] = fmaf(part[r][t], sc, acc[r][t]);
            }
        }
    }
}

// Work item decode: blockIdx.x = slot * tiles + tile, slot indexes the
// path's active-expert list.  Returns false when the slot is unused.
__device__ inline bool item_of(const GemmArgs& a, int tiles, int& e, int& tile, int& M, int& off) {
    int slot = blockIdx.x / tiles;
    tile = blockIdx.x % tiles;
    if (slot >= a.meta[a.list_meta]) return false;
    e = a.list[slot];
    M = a.counts[e];
    off = a.offsets[e];
    return true;
}

template <int MT>
__device__ void gate_up_pass(const GemmArgs& a, int e, int tile, int off, int M,
                             const uint4* xs) {
    const int lane16 = threadIdx.x % kGemvLanesPerRow;
    const int slot = threadIdx.x / kGemvLanesPerRow;
    const int K = a.H, nblk = K / 32, units = K / 8;
    const uint8_t* W = a.wgu + (int64_t)e * (2 * a.I) * (K / 2);
    const uint8_t* S = a.sgu + (int64_t)e * (2 * a.I) * nblk;
    const int n0 = tile * kGateUpUnits;
    for (int unit = slot; unit < kGateUpUnits; unit += kGemvSlots) {
        int n = n0 + unit;
        if (n >= a.I) break;
        const uint8_t* rows[2] = {W + (int64_t)n * (K / 2), W + (int64_t)(a.I + n) * (K / 2)};
        const uint8_t* srows[2] = {S + (int64_t)n * nblk, S + (int64_t)(a.I + n) * nblk};
        float acc[2][MT];
        rows_dot<MT, 2>(rows, srows, nblk, xs, units, lane16, acc);
#pragma unroll
        for (int t = 0; t < MT; t++) {
            float g = row16_sum(acc[0][t]);
            float u = row16_sum(acc[1][t]);
            if (lane16 == t && t < M)
                a.h[(int64_t)(off + t) * a.I + n] = f32_to_bf16_rne(silu_mul(g, u));
        }
    }
}

template <int MT>
__device__ void down_pass(const GemmArgs& a, int e, int tile, int off, int M, const uint4* xs) {
    const int lane16 = threadIdx.x % kGemvLanesPerRow;
    const int slot = threadIdx.x / kGemvLanesPerRow;
    const int K = a.I, nblk = K / 32, units = K / 8;
    const uint8_t* W = a.wdn + (int64_t)e * a.H * (K / 2);
    const uint8_t* S = a.sdn + (int64_t)e * a.H * nblk;
    const int n0 = tile * kDownUnits * 2;
    for (int unit = slot; unit < kDownUnits; unit += kGemvSlots) {
        int n = n0 + 2 * unit;
        if (n >= a.H) break;
        const uint8_t* rows[2] = {W + (int64_t)n * (K / 2), W + (int64_t)(n + 1) * (K / 2)};
        const uint8_t* srows[2] = {S + (int64_t)n * nblk, S + (int64_t)(n + 1) * nblk};
        float acc[2][MT];
        rows_dot<MT, 2>(rows, srows, nblk, xs, units, lane16, acc);
#pragma unroll
        for (int t = 0; t < MT; t++) {
            float y0 = row16_sum(acc[0][t]);
            float y1 = row16_sum(acc[1][t]);
            if (lane16 == t && t < M)
                *reinterpret_cast<float2*>(a.y + (int64_t)(off + t) * a.H + n) =
                    make_float2(y0, y1);
        }
    }
}

extern __shared__ uint4 dyn_lds[];

__global__ void __launch_bounds__(kGemvThreads)
gemv_gate_up_kernel(GemmArgs a) {
    const int tiles = (a.I + kGateUpUnits - 1) / kGateUpUnits;
    int e, tile, M, off;
    if (!item_of(a, tiles, e, tile, M, off)) return;
    uint4* xs = dyn_lds;
    for (int t0 = 0; t0 < M; t0 += kGemvMaxTok) {
        int m = min(kGemvMaxTok, M - t0);
        __syncthreads();
        stage_rows(xs, m, a.H, [&](int t) {
            int token = a.sorted[off + t0 + t] / a.k;
            return a.x + (int64_t)token * a.H;
        });
        __syncthreads();
        switch (m) {
            case 1: gate_up_pass<1>(a, e, tile, off + t0, m, xs); break;
            case 2: gate_up_pass<2>(a, e, tile, off + t0, m, xs); break;
            case 3: gate_up_pass<3>(a, e, tile, off + t0, m, xs); break;
            default: gate_up_pass<4>(a, e, tile, off + t0, m, xs); break;
        }
    }
}

__global__ void __launch_bounds__(kGemvThreads)
gemv_down_kernel(GemmArgs a) {
    const int tiles = (a.H + 2 * kDownUnits - 1) / (2 * kDownUnits);
    int e, tile, M, off;
    if (!item_of(a, tiles, e, tile, M, off)) return;
    uint4* xs = dyn_lds;
    for (int t0 = 0; t0 < M; t0 += kGemvMaxTok) {
        int m = min(kGemvMaxTok, M - t0);
        __syncthreads();
        stage_rows(xs, m, a.I, [&](int t) { return a.h + (int64_t)(off + t0 + t) * a.I; });
        __syncthreads();
        switch (m) {
            case 1: down_pass<1>(a, e, tile, off + t0, m, xs); break;
            case 2: down_pass<2>(a, e, tile, off + t0, m, xs); break;
            case 3: down_pass<3>(a, e, tile, off + t0, m, xs); break;
            default: down_pass<4>(a, e, tile, off + t0, m, xs); break;
        }
    }
}

}  // namespace

hipError_t launch_gemv_gate_up(const GemmArgs& a, int max_active, hipStream_t stream) {
    int tiles = (a.I + kGateUpUnits - 1) / kGateUpUnits;
    size_t lds = (size_t)kGemvMaxTok * a.H * 2;
    gemv_gate_up_kernel<<<max_active * tiles, kGemvThreads, lds, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_gemv_down(const GemmArgs& a, int max_active, hipStream_t stream) {
    int tiles = (a.H + 2 * kDownUnits - 1) / (2 * kDownUnits);
    size_t lds = (size_t)kGemvMaxTok * a.I * 2;
    gemv_down_kernel<<<max_active * tiles, kGemvThreads, lds, stream>>>(a);
    return hipGetLastError();
}

}  // namespace moe
