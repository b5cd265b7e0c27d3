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
// gate_up items also apply SiLU(gate) * up and store h as bf16 hi/lo pairs
// (h2_pos); down items dot each weight pair with both halves and store the
// per-assignment outputs y in fp32.
#include "device_common.h"

namespace moe {
namespace {

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

// h between the GEMMs of this path: each fp32 value v as the bf16 pair
// (hi, lo) = (bf16(v), bf16(v - hi)) (split_bf16), which holds v to about
// 2^-17 relative where one bf16 rounding costs up to 2^-9 and, stacked on
// the bf16 rounding of out, can exceed the layer's error budget.  A row of
// I values is 2I bf16: [chunk n/128][half (n/16)%2][block (n/32)%4][hi,
// lo][16 values]; h2_pos(n) is the index of element n's hi, its lo 16 later.
__device__ inline int h2_pos(int n) {
    return (((n >> 7) * 2 + ((n >> 4) & 1)) * 4 + ((n >> 5) & 3)) * 32 + (n & 15);
}

// LDS position (in 16-byte units) of quarter q of block b of a token row
__device__ inline int xs_unit(int b, int q) { return b * 4 + ((q + (b >> 1)) & 3); }
// ... of an h row in hi/lo pairs (8 units per block: the four hi quarters,
// then the four lo quarters, each group rotated as above); its lo quarter
// sits 4 units after its hi quarter
__device__ inline int hs_unit(int b, int q) { return b * 8 + ((q + (b >> 1)) & 3); }

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

// Stage h rows in the hi/lo layout (2K bf16 each, see h2_pos) into LDS at
// the hs_unit positions: 16-byte unit u of a row holds quarter q = 2*hf +
// (u & 1) of part (u >> 1) & 1 (hi, lo) of block 4*(u >> 5) + ((u >> 2) & 3),
// hf = (u >> 4) & 1.
template <typename RowFn>
__device__ inline void stage_rows_h2(uint4* __restrict__ xs, int M, int K, RowFn row_ptr) {
    const int units = K / 4;  // 16-byte units per row of 2K bf16
    for (int i = threadIdx.x; i < M * units; i += blockDim.x) {
        const int t = i / units, u = i % units;
        const int b = 4 * (u >> 5) + ((u >> 2) & 3), q = 2 * ((u >> 4) & 1) + (u & 1);
        const uint4* src = reinterpret_cast<const uint4*>(row_ptr(t));
        xs[t * units + hs_unit(b, q) + 4 * ((u >> 1) & 1)] = src[u];
    }
}

// ---------------------------------------------------------------------------
// Software-pipelined row-pair GEMV core.
//
// A lane walks a flat sequence of steps; step s covers, for one unit (two
// matrix rows), kGemvUnroll of the lane's blocks in each row.  The loads of
// step s+1 are issued before step s is computed (two register buffers), so
// every lane keeps 128-256 bytes of weights in flight, and the first step is
// issued before the activation tile is staged.  A unit's 16 lanes reduce
// with DPP when its last step is done and hand the sums to `epi`.
// ---------------------------------------------------------------------------

template <int R>
struct StepBuf {
    uint4 w[kGemvUnroll][R];
    uint32_t s[kGemvUnroll][R];
};

// HL: the activations are h rows in hi/lo pairs (stage_rows_h2); each
// decoded weight pair is dotted with the hi pair, then the lo pair.
template <int MT, int R, bool HL, typename RowsFn>
struct RowGemv {
    RowsFn rows_of;      // rows_of(unit, rows[R], srows[R])
    int unit0, unit_step, n_units, n_iter, nblk, lane16;

    __device__ int steps() const { return n_units * n_iter; }

    __device__ void load(int s, StepBuf<R>& b) const {
        const int u = unit0 + (s / n_iter) * unit_step, it = s % n_iter;
        const uint8_t* rows[R];
        const uint8_t* srows[R];
        rows_of(u, rows, srows);
#pragma unroll
        for (int j = 0; j < kGemvUnroll; j++) {
            const int blk = lane16 + kGemvLanesPerRow * (kGemvUnroll * it + j);
#pragma unroll
            for (int r = 0; r < R; r++) {
                if (blk < nblk) {
                    b.w[j][r] = load_stream16(rows[r] + (int64_t)blk * 16);
                    b.s[j][r] = srows[r][blk];
                } else {
                    b.w[j][r] = make_uint4(0, 0, 0, 0);
                    b.s[j][r] = 127;
                }
            }
        }
    }

    // accumulate step s (whose loads are in b) into acc
    __device__ void compute(int s, const StepBuf<R>& b, const uint4* __restrict__ xs,
                            int units_per_tok, float (&acc)[R][MT]) const {
        const int it = s % n_iter;
        if (it == 0) {
#pragma unroll
            for (int r = 0; r < R; r++)
#pragma unroll
                for (int t = 0; t < MT; t++) acc[r][t] = 0.f;
        }
#pragma unroll
        for (int j = 0; j < kGemvUnroll; j++) {
            const int blk = lane16 + kGemvLanesPerRow * (kGemvUnroll * it + j);
            if (blk >= nblk) break;
            float part[R][MT];
#pragma unroll
            for (int r = 0; r < R; r++)
#pragma unroll
                for (int t = 0; t < MT; t++) part[r][t] = 0.f;
#pragma unroll
            for (int q = 0; q < 4; q++) {
                uint4 xv[MT], xl[MT];
#pragma unroll
                for (int t = 0; t < MT; t++) {
                    if constexpr (HL) {
                        xv[t] = xs[t * units_per_tok + hs_unit(blk, q)];
                        xl[t] = xs[t * units_per_tok + hs_unit(blk, q) + 4];
                    } else {
                        xv[t] = xs[t * units_per_tok + xs_unit(blk, q)];
                    }
                }
#pragma unroll
                for (int r = 0; r < R; r++) {
                    const uint32_t word = (q == 0) ? b.w[j][r].x : (q == 1) ? b.w[j][r].y
                                        : (q == 2) ? b.w[j][r].z : b.w[j][r].w;
                    // byte i of the word holds elements 2i (low nibble) and 2i+1
                    const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, 1.0f, 0);
                    const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, 1.0f, 1);
                    const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, 1.0f, 2);
                    const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, 1.0f, 3);
#pragma unroll
                    for (int t = 0; t < MT; t++) {
                        float v = part[r][t];
                        v = __builtin_amdgcn_fdot2_f32_bf16(p0, as_bf16x2(xv[t].x), v, false);
                        v = __builtin_amdgcn_fdot2_f32_bf16(p1, as_bf16x2(xv[t].y), v, false);
                        v = __builtin_amdgcn_fdot2_f32_bf16(p2, as_bf16x2(xv[t].z), v, false);
                        v = __builtin_amdgcn_fdot2_f32_bf16(p3, as_bf16x2(xv[t].w), v, false);
                        if constexpr (HL) {
                            v = __builtin_amdgcn_fdot2_f32_bf16(p0, as_bf16x2(xl[t].x), v, false);
                            v = __builtin_amdgcn_fdot2_f32_bf16(p1, as_bf16x2(xl[t].y), v, false);
                            v = __builtin_amdgcn_fdot2_f32_bf16(p2, as_bf16x2(xl[t].z), v, false);
                            v = __builtin_amdgcn_fdot2_f32_bf16(p3, as_bf16x2(xl[t].w), v, false);
                        }
                        part[r][t] = v;
                    }
                }
            }
#pragma unroll
            for (int r = 0; r < R; r++) {
                const float sc = e8m0_to_f32(b.s[j][r]);
#pragma unroll
                for (int t = 0; t < MT; t++) acc[r][t] = fmaf(part[r][t], sc, acc[r][t]);
            }
        }
    }
};

// Run a RowGemv over its steps: first loads, then stage() (which must end
// with a workgroup barrier), then the pipelined loop.  epi(unit, sums)
// receives the reduced sums (valid in every lane of the 16) after each unit.
template <int MT, int R, bool HL, typename RowsFn, typename StageFn, typename EpiFn>
__device__ void run_row_gemv(const RowGemv<MT, R, HL, RowsFn>& g, const uint4* xs, int units_per_tok,
                             StageFn stage, EpiFn epi) {
    const int S = g.steps();
    StepBuf<R> A, B;
    float acc[R][MT];
    if (S > 0) g.load(0, A);
    stage();
    auto finish = [&](int s) {
        if (s % g.n_iter == g.n_iter - 1) {
            float sums[R][MT];
#pragma unroll
            for (int r = 0; r < R; r++)
#pragma unroll
                for (int t = 0; t < MT; t++) sums[r][t] = row16_sum(acc[r][t]);
            epi(g.unit0 + (s / g.n_iter) * g.unit_step, sums);
        }
    };
    for (int s = 0; s < S; s += 2) {
        if (s + 1 < S) g.load(s + 1, B);
        g.compute(s, A, xs, units_per_tok, acc);
        finish(s);
        if (s + 1 < S) {
            if (s + 2 < S) g.load(s + 2, A);
            g.compute(s + 1, B, xs, units_per_tok, acc);
            finish(s + 1);
        }
    }
}

extern __shared__ uint4 dyn_lds[];

// One gate_up pass over up to MT tokens (rows off .. off+m of the sorted
// assignments): units are (gate row n, up row I+n) pairs of this tile.
template <int MT>
__device__ void gate_up_pass(const GemmArgs& a, int e, int tile, int off, int m, int tok0) {
    const int lane16 = threadIdx.x % kGemvLanesPerRow;
    const int slot = threadIdx.x / kGemvLanesPerRow;
    const int K = a.H, nblk = K / 32, units = K / 8;
    const uint8_t* W = a.wgu + (int64_t)e * (2 * a.I) * (K / 2);
    const uint8_t* S = a.sgu + (int64_t)e * (2 * a.I) * nblk;
    const int n0 = tile * kGateUpUnits;
    const int nu = min(kGateUpUnits, a.I - n0);
    auto rows_of = [&](int u, const uint8_t* (&rows)[2], const uint8_t* (&srows)[2]) {
        const int n = n0 + u;
        rows[0] = W + (int64_t)n * (K / 2);
        rows[1] = W + (int64_t)(a.I + n) * (K / 2);
        srows[0] = S + (int64_t)n * nblk;
        srows[1] = S + (int64_t)(a.I + n) * nblk;
    };
    RowGemv<MT, 2, false, decltype(rows_of)> g{rows_of, slot, kGemvSlots,
                                               slot < nu ? (nu - slot + kGemvSlots - 1) / kGemvSlots : 0,
                                               (nblk + kGemvLanesPerRow * kGemvUnroll - 1) /
                                                   (kGemvLanesPerRow * kGemvUnroll),
                                               nblk, lane16};
    uint4* xs = dyn_lds;
    auto stage = [&]() {
        stage_rows(xs, m, K, [&](int t) {
            const int token = a.sorted[off + t] / a.k;
            return a.x + (int64_t)token * K;
        });
        __syncthreads();
    };
    auto epi = [&](int u, float (&sums)[2][MT]) {
        const int n = n0 + u;
#pragma unroll
        for (int t = 0; t < MT; t++)
            if (lane16 == t && t < m) {
                uint16_t hi, lo;
                split_bf16(silu_mul(sums[0][t], sums[1][t]), hi, lo);
                uint16_t* row = a.h + (int64_t)(off + t) * 2 * a.I + h2_pos(n);
                row[0] = hi;
                row[16] = lo;
            }
    };
    run_row_gemv(g, xs, units, stage, epi);
    (void)tok0;
}

// One down pass: units are two adjacent output rows (n, n+1) of this tile.
template <int MT>
__device__ void down_pass(const GemmArgs& a, int e, int tile, int off, int m) {
    const int lane16 = threadIdx.x % kGemvLanesPerRow;
    const int slot = threadIdx.x / kGemvLanesPerRow;
    const int K = a.I, nblk = K / 32, units = K / 8;
    const uint8_t* W = a.wdn + (int64_t)e * a.H * (K / 2);
    const uint8_t* S = a.sdn + (int64_t)e * a.H * nblk;
    const int n0 = tile * kColTile;
    const int nu = min(kDownUnits, (a.H - n0) / 2);
    auto rows_of = [&](int u, const uint8_t* (&rows)[2], const uint8_t* (&srows)[2]) {
        const int n = n0 + 2 * u;
        rows[0] = W + (int64_t)n * (K / 2);
        rows[1] = W + (int64_t)(n + 1) * (K / 2);
        srows[0] = S + (int64_t)n * nblk;
        srows[1] = S + (int64_t)(n + 1) * nblk;
    };
    RowGemv<MT, 2, true, decltype(rows_of)> g{rows_of, slot, kGemvSlots,
                                              slot < nu ? (nu - slot + kGemvSlots - 1) / kGemvSlots : 0,
                                              (nblk + kGemvLanesPerRow * kGemvUnroll - 1) /
                                                  (kGemvLanesPerRow * kGemvUnroll),
                                              nblk, lane16};
    uint4* xs = dyn_lds;
    auto stage = [&]() {
        stage_rows_h2(xs, m, K, [&](int t) { return a.h + (int64_t)(off + t) * 2 * K; });
        __syncthreads();
    };
    auto epi = [&](int u, float (&sums)[2][MT]) {
        const int n = n0 + 2 * u;
#pragma unroll
        for (int t = 0; t < MT; t++)
            if (lane16 == t && t < m) {
                // agent-coherent store: the combining block may run on another XCD
                const uint64_t bits = (uint64_t)__float_as_uint(sums[0][t]) |
                                      ((uint64_t)__float_as_uint(sums[1][t]) << 32);
                __hip_atomic_store(reinterpret_cast<uint64_t*>(a.y + (int64_t)(off + t) * a.H + n),
                                   bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
    };
    run_row_gemv(g, xs, 2 * units, stage, epi);
}

// gate_up: blockIdx.x = slot * tg + tile over an upper bound of active
// experts; a tile is 32 gate rows with their 32 up rows.  Blocks past the
// routed experts exit at once.
__global__ void __launch_bounds__(kGemvThreads)
gemv_gate_up_kernel(GemmArgs a) {
    const int tg = (a.I + kGateUpUnits - 1) / kGateUpUnits;
    const int slot = blockIdx.x / tg, tile = blockIdx.x % tg;
    if (slot >= uniform(a.meta[a.list_meta])) return;
    const int e = uniform(a.list[slot]);
    const int M = uniform(a.counts[e]), off = uniform(a.offsets[e]);
    for (int t0 = 0; t0 < M; t0 += kGemvMaxTok) {
        const int m = min(kGemvMaxTok, M - t0);
        __syncthreads();  // the previous pass is done with the staged tile
        switch (m) {
            case 1: gate_up_pass<1>(a, e, tile, off + t0, m, t0); break;
            case 2: gate_up_pass<2>(a, e, tile, off + t0, m, t0); break;
            case 3: gate_up_pass<3>(a, e, tile, off + t0, m, t0); break;
            default: gate_up_pass<4>(a, e, tile, off + t0, m, t0); break;
        }
    }
}

// Tokens per down pass: the staged h rows (hi/lo pairs, 4*I bytes each)
// stay within 128 KB of LDS, so up to 4 tokens for I <= 8192 and 2 above.
__host__ __device__ inline int gemv_down_tokens(int I) {
    return (int64_t)kGemvMaxTok * I * 4 <= (128 << 10) ? kGemvMaxTok : 2;
}

// down: blockIdx.x = slot * td + tile; a tile is kColTile output columns.
// After writing its rows of y, a block counts the tile done for each of its
// tokens; the block whose count completes a token's k experts combines that
// token's tile.  Nothing waits: the last finisher does the work.  y moves
// between blocks through agent-coherent atomic stores and loads, ordered
// by waiting for this block's stores to complete before the counter update;
// no L2 writeback or invalidate is needed.
__global__ void __launch_bounds__(kGemvThreads) __attribute__((amdgpu_waves_per_eu(3)))
gemv_down_kernel(GemmArgs a) {
    __shared__ int s_combine[kGemvMaxTok];
    const int td = a.col_tiles;
    const int slot = blockIdx.x / td, tile = blockIdx.x % td;
    if (slot >= uniform(a.meta[a.list_meta])) return;
    const int e = uniform(a.list[slot]);
    const int M = uniform(a.counts[e]), off = uniform(a.offsets[e]);
    const int per = gemv_down_tokens(a.I);
    for (int t0 = 0; t0 < M; t0 += per) {
        const int m = min(per, M - t0);
        __syncthreads();
        switch (m) {
            case 1: down_pass<1>(a, e, tile, off + t0, m); break;
            case 2: down_pass<2>(a, e, tile, off + t0, m); break;
            case 3: down_pass<3>(a, e, tile, off + t0, m); break;
            default: down_pass<4>(a, e, tile, off + t0, m); break;
        }
        // every wave's y stores have completed before any of its tokens is
        // counted: the combining workgroup may run on another XCD and read y
        // as soon as the count completes (a workgroup-scope fence would not
        // wait for them)
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
        __syncthreads();
        if ((int)threadIdx.x < m) {
            const int token = a.sorted[off + t0 + threadIdx.x] / a.k;
            const int old = atomicAdd(&a.tile_done[token * td + tile], 1);
            s_combine[threadIdx.x] = (old == a.k - 1) ? token : -1;
        }
        __syncthreads();
        for (int i = 0; i < m; i++) {
            const int token = uniform(s_combine[i]);
            if (token >= 0) combine_tile(a, token, tile * kColTile, kColTile);
        }
    }
}

}  // namespace

hipError_t launch_gemv_gate_up(const GemmArgs& a, int max_active, hipStream_t stream) {
    const int tg = (a.I + kGateUpUnits - 1) / kGateUpUnits;
    const size_t lds = (size_t)kGemvMaxTok * a.H * 2;
    gemv_gate_up_kernel<<<max_active * tg, kGemvThreads, lds, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_gemv_down(const GemmArgs& a, int max_active, hipStream_t stream) {
    const size_t lds = (size_t)gemv_down_tokens(a.I) * a.I * 4;  // h rows as hi/lo pairs
    gemv_down_kernel<<<max_active * a.col_tiles, kGemvThreads, lds, stream>>>(a);
    return hipGetLastError();
}

}  // namespace moe
