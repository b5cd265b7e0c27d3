// mxfp8.hip -- the prefill path: MXFP8 activations against MXFP4 expert
// weights on the scaled matrix cores of gfx950.
//
// At a prefill chunk every expert sees hundreds of tokens and the layer is
// compute-bound, so the activations are encoded too: x per token along H and
// h per assignment along I, each block of 32 as E4M3 elements with one E8M0
// scale (the weights' block rule with the E4M3 element range), and both
// GEMMs run on v_mfma_scale_f32_16x16x128_f8f6f4 with the FP4 weights as
// operand A and the FP8 activations as operand B; the hardware applies both
// block scales.  The weights are the MXFP4 format the pages give the experts
// (bjdmk.com.cn news page, co-design section); the pages keep everything
// else at 8-bit or higher precision (tilert.ai blog, second leap), which is
// what MXFP8 activations are.
//
// Operands of one 16x16x128 MFMA (lane l = (r, g) = (l % 16, l / 16)):
//   A (FP4) = 16 weight rows x 128 k: lane (r, g) holds MX block g of row r,
//     i.e. 16 bytes -- exactly one group of the prepacked tile layout, and its
//     E8M0 scale is one byte of the lane's tile-scale dword.
//   B (FP8) = 128 k x 16 tokens: lane (c, g) holds k = 16g..16g+15 of token
//     c in bytes 0..15 and k = 64+16g..64+16g+15 in bytes 16..31 (two
//     16-byte pieces, not one MX block), and the scale of block g of token c
//     (the hardware pairs B's k with A's block layout this way; measured
//     with one-hot operands on gfx950).
//   D = 16 rows x 16 tokens; lane (c, g) holds rows 4g..4g+3 of token c.
//
// Tiling: a workgroup computes 128 weight rows (two 64-row quads of the tile
// layout) against one item of up to 128 tokens, over the whole K.  Its four
// waves form a 2 x 2 grid: wave (wr, wt) owns quad wr and the token tiles
// wt, wt+2, wt+4, wt+6 of 16 tokens (4 row groups x 4 column tiles = 16
// MFMAs per 128-k chunk).
// A comes straight from global memory in operand order (one 1 KB wave load
// per row group); B, shared by the two waves of a token half, goes from
// global memory directly into double-buffered LDS (global_load_lds, 16
// bytes per lane, lane l at byte 16l of the wave's 1 KB destination),
// XOR-swizzled so that operand reads are free of bank conflicts.  The token
// rows of x are gathered through the routing order; h rows are already in
// that order.
#include "mfma_items.h"

namespace moe {
namespace {

typedef int i32x8_t __attribute__((ext_vector_type(8)));

#ifndef MOE_PF_SCHED_BARRIERS
#define MOE_PF_SCHED_BARRIERS 0
#endif
#ifndef MOE_PF_WAVES_PER_EU
#define MOE_PF_WAVES_PER_EU 2
#endif

constexpr int kPfThreads = 256;
constexpr int kPfTiles = 4;               // 16-token column tiles per wave

static_assert(kMx8Tok == 128, "the prefill tiling assumes 128-token items");

constexpr int kQuantThreads = 256;

// MXFP8 encoding of x: one thread per block of 32 elements
__global__ void __launch_bounds__(kQuantThreads)
quantize_x_mxfp8_kernel(const uint16_t* __restrict__ x, int64_t nblocks,
                        uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
    const int64_t b = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x;
    if (b >= nblocks) return;
    const uint4* src = reinterpret_cast<const uint4*>(x + b * 32);
    float v[32];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const uint4 w = src[i];
        const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int j = 0; j < 4; j++) {
            v[8 * i + 2 * j] = __uint_as_float(u[j] << 16);
            v[8 * i + 2 * j + 1] = __uint_as_float(u[j] & 0xffff0000u);
        }
    }
    uint32_t amax = 0;
#pragma unroll
    for (int i = 0; i < 32; i++) {
        const uint32_t m = __float_as_uint(v[i]) & 0x7fffffffu;
        amax = m > amax ? m : amax;  // NaN bits order above every finite value
    }
    uint32_t c[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    uint8_t s = 255;
    if (amax < 0x7f800000u) {
        const int se = mxfp8_scale_exp(amax);
        s = (uint8_t)(se + 127);
#pragma unroll
        for (int i = 0; i < 32; i++) c[i / 4] |= e4m3_code(v[i], se) << (8 * (i % 4));
    }
    uint4* dst = reinterpret_cast<uint4*>(codes + b * 32);
    dst[0] = make_uint4(c[0], c[1], c[2], c[3]);
    dst[1] = make_uint4(c[4], c[5], c[6], c[7]);
    scales[b] = s;
}

typedef __attribute__((address_space(3))) void lds_void_t;

// Staged B of one chunk: 128 token rows of 128 code bytes, 16-byte piece p
// of row r stored in slot p ^ ((r >> 1) & 7).  A 16-lane quarter of an
// operand read (rows c = 0..15, one piece) then covers the 64 banks once.
struct PfSmem {
    alignas(16) uint8_t b[2][kMx8Tok * 128];
    alignas(16) uint32_t bs[2][kMx8Tok];  // the chunk's 4 block scales per token
};

__device__ inline int b_slot(int row, int piece) { return piece ^ ((row >> 1) & 7); }

// Where this lane's direct-to-LDS loads come from.  Wave w fills LDS rows
// 32w .. 32w+31 of a chunk with four 1 KB loads (lane l: row 32w + 8i +
// l/8, slot l % 8); waves 0 and 1 also load the scale words of tokens
// 64w + l.  Rows past the item's m tokens repeat row m-1: they only feed
// output columns that are never stored.
struct StageSrc {
    const uint8_t* row[4];  // code bytes of the row's piece for this lane, chunk 0
    const uint8_t* srow;    // scale bytes of this lane's token, chunk 0 (waves 0, 1)
};

__device__ inline void stage_issue(const StageSrc& src, int chunk, PfSmem& sm, int buf) {
    const int w = threadIdx.x / kWave;
#pragma unroll
    for (int i = 0; i < 4; i++)
        __builtin_amdgcn_global_load_lds(src.row[i] + chunk * 128,
                                         (lds_void_t*)&sm.b[buf][(32 * w + 8 * i) * 128], 16, 0, 0);
    if (w < 2)
        __builtin_amdgcn_global_load_lds(src.srow + chunk * 4, (lds_void_t*)&sm.bs[buf][64 * w], 4,
                                         0, 0);
}

// lane's LDS row for staging load i of wave w, and the piece it carries
__device__ inline int stage_row(int i) { return 32 * (threadIdx.x / kWave) + 8 * i + (threadIdx.x % kWave) / 8; }
__device__ inline int stage_piece(int i) { return b_slot(stage_row(i), threadIdx.x % 8); }

struct AOperand {
    uint4 w[4];  // row groups 0..3 of the quad
    uint32_t s;  // their four scale bytes
};

__device__ inline void load_a(const uint8_t* tiles, const uint8_t* tscales, int chunk, AOperand& a) {
    const int lane = threadIdx.x % kWave;
    const uint8_t* t = tiles + (int64_t)chunk * 4096 + lane * 16;
#pragma unroll
    for (int rg = 0; rg < 4; rg++) a.w[rg] = *reinterpret_cast<const uint4*>(t + rg * 1024);
    a.s = *reinterpret_cast<const uint32_t*>(tscales + (int64_t)chunk * 256 + lane * 4);
}

// Column tile t of wave (wr, wt) is token tile 2t + wt of the item
// (interleaved, so the two token waves stay balanced on ragged items).
__device__ inline int tile_token(int t, int wt, int c) { return 16 * (2 * t + wt) + c; }

template <int NT>
struct BOperands {
    i32x8_t v[NT > 0 ? NT : 1];
    int s[NT > 0 ? NT : 1];
};

// this wave's B operands of the chunk in LDS buffer `buf`
template <int NT>
__device__ inline void read_b(const PfSmem& sm, int buf, BOperands<NT>& b) {
    const int lane = threadIdx.x % kWave, c = lane % 16, g = lane / 16;
    const int wt = (threadIdx.x / kWave) >> 1;
#pragma unroll
    for (int t = 0; t < NT; t++) {
        const int row = tile_token(t, wt, c);
        const uint8_t* base = &sm.b[buf][row * 128];
        const uint4 lo = *reinterpret_cast<const uint4*>(base + 16 * b_slot(row, g));
        const uint4 hi = *reinterpret_cast<const uint4*>(base + 16 * b_slot(row, g + 4));
        b.s[t] = (int)((sm.bs[buf][row] >> (8 * g)) & 0xffu);
        b.v[t] = i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                         (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
}

template <int NT>
__device__ inline void chunk_mfma(const AOperand& ac, const BOperands<NT>& b,
                                  f32x4_t (&acc)[4][kPfTiles]) {
#pragma unroll
    for (int rg = 0; rg < 4; rg++) {
        const i32x8_t A = i32x8_t{(int)ac.w[rg].x, (int)ac.w[rg].y, (int)ac.w[rg].z,
                                  (int)ac.w[rg].w, 0, 0, 0, 0};
        const int sa = (int)((ac.s >> (8 * rg)) & 0xffu);
#pragma unroll
        for (int t = 0; t < NT; t++)
            acc[rg][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                A, b.v[t], acc[rg][t], 4 /* A: FP4 E2M1 */, 0 /* B: FP8 E4M3 */, 0, sa, 0, b.s[t]);
    }
}

// The main loop of one workgroup: acc[rg][t] = quad rows (group rg) x
// column tile t of this wave (t < NT), summed over all `chunks` 128-k
// chunks.  tiles/tscales point at this wave's quad.
//
// Step s: wait for this wave's loads (its share of chunk s in LDS buffer
// s%2, A of chunk s) and meet the other waves at a barrier; read the B
// operands of chunk s; issue A of chunk s+1 and the direct-to-LDS loads of
// chunk s+1 into the other buffer (whose readers all passed this barrier);
// run the MFMAs.  The loads of chunk s+1 thus fly during the MFMAs of chunk
// s, and no staging registers are needed.  Every wave runs the same number
// of barriers whatever its NT.
template <int NT>
__device__ inline void pf_mainloop(const uint8_t* tiles, const uint8_t* tscales, const StageSrc& src,
                                   int chunks, PfSmem& sm, f32x4_t (&acc)[4][kPfTiles]) {
#pragma unroll
    for (int rg = 0; rg < 4; rg++)
#pragma unroll
        for (int t = 0; t < kPfTiles; t++) acc[rg][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    AOperand a0, a1;
    stage_issue(src, 0, sm, 0);
    load_a(tiles, tscales, 0, a0);
    auto step = [&](int s, const AOperand& acur, AOperand& anext) {
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's loads of chunk s
        __syncthreads();                      // everyone's
        BOperands<NT> b;
        read_b<NT>(sm, s & 1, b);
        if (s + 1 < chunks) {
            load_a(tiles, tscales, s + 1, anext);
            stage_issue(src, s + 1, sm, (s & 1) ^ 1);
        }
        chunk_mfma<NT>(acur, b, acc);
    };
    for (int s = 0; s < chunks; s += 2) {
        step(s, a0, a1);
        if (s + 1 >= chunks) break;
        step(s + 1, a1, a0);
    }
}

__device__ inline void pf_gemm(const uint8_t* tiles, const uint8_t* tscales, const StageSrc& src,
                               int chunks, int ntile, PfSmem& sm, f32x4_t (&acc)[4][kPfTiles]) {
    switch (ntile) {
        case 4: pf_mainloop<4>(tiles, tscales, src, chunks, sm, acc); break;
        case 3: pf_mainloop<3>(tiles, tscales, src, chunks, sm, acc); break;
        case 2: pf_mainloop<2>(tiles, tscales, src, chunks, sm, acc); break;
        case 1: pf_mainloop<1>(tiles, tscales, src, chunks, sm, acc); break;
        default: pf_mainloop<0>(tiles, tscales, src, chunks, sm, acc); break;
    }
}

// column tiles of token wave wt that hold any of the item's m tokens
__device__ inline int wave_tiles(int m, int wt) {
    const int all = (m + 15) / 16;
    return (all - wt + 1) / 2;
}

// gate_up, MXFP8 activations: blockIdx.x = item * (I / 64) + row block; the
// row block holds quads 2rb, 2rb+1, each 32 gate rows (groups 0, 1) with
// their 32 up rows (groups 2, 3), so SiLU(gate) * up is formed in
// registers, and the 32 h values of one quad and token -- one MX block of h
// -- sit in the four lanes (c, 0..3), which agree on the block scale through
// two cross-lane maxima.
__global__ void __launch_bounds__(kPfThreads, MOE_PF_WAVES_PER_EU)
mx8_gate_up_kernel(GemmArgs a) {
    __shared__ union {
        PfSmem pf;
        f32x4_t red[kRedGateUp * 4];  // the shared expert's blocks
    } lds;
    PfSmem& sm = lds.pf;
    const int rowblocks = a.I / 64;
    int b = blockIdx.x;
    if (a.sh_wgu) {  // the shared expert's blocks first (64-token tiles, split-K)
        const int nb = shared_blocks(a.I / 32, (a.T + 63) / 64);
        if (b < nb) {
            shared_gate_up_block<4, X8>(a, b, lds.red);
            return;
        }
        b -= nb;
    }
    const int item = b / rowblocks, rb = b % rowblocks;
    if (item >= uniform(a.meta[kMetaNumMfmaItems])) return;
    const int4 it = a.items[item];
    const int e = uniform(it.x), row0 = uniform(it.y), m = uniform(it.z);
    const int tid = threadIdx.x, w = tid / kWave, lane = tid % kWave, c = lane % 16, g = lane / 16;
    const int wr = w & 1, wt = w >> 1;
    const int K = a.H, chunks = K / 128, quads = a.I / 32;
    const int quad = 2 * rb + wr;
    const int64_t quad_id = (int64_t)e * quads + quad;
    StageSrc src;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int j = min(stage_row(i), m - 1);
        src.row[i] = a.xq + (int64_t)(a.sorted[row0 + j] / a.k) * K + 16 * stage_piece(i);
    }
    src.srow = a.xs + (int64_t)(a.sorted[row0 + min(64 * (w & 1) + lane, m - 1)] / a.k) * (K / 32);
    const int ntile = uniform(wave_tiles(m, wt));
    f32x4_t acc[4][kPfTiles];
    pf_gemm(a.wgu + quad_id * chunks * 4096, a.sgu + quad_id * chunks * 256, src, chunks, ntile, sm,
            acc);
#pragma unroll
    for (int t = 0; t < kPfTiles; t++) {
        if (t >= ntile) break;
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
        const int j = tile_token(t, wt, c);
        if (j < m) {
            uint8_t* hrow = a.hq + (int64_t)(row0 + j) * a.I + 32 * quad + 4 * g;
            *reinterpret_cast<uint32_t*>(hrow) = code[0];       // h rows 32q + 4g + i
            *reinterpret_cast<uint32_t*>(hrow + 16) = code[1];  // h rows 32q + 16 + 4g + i
            if (g == 0) a.hs[(int64_t)(row0 + j) * (a.I / 32) + quad] = (uint8_t)scale;
        }
    }
}

// down, MXFP8 h: blockIdx.x = item * (H / 128) + row block (quads 2rb,
// 2rb+1 of the output rows).  y goes out through plain 16-byte stores; the
// combine runs as its own kernel after this one (combine.hip).
__global__ void __launch_bounds__(kPfThreads, MOE_PF_WAVES_PER_EU)
mx8_down_kernel(GemmArgs a) {
    __shared__ union {
        PfSmem pf;
        f32x4_t red[kRedDown * 4];  // the shared expert's blocks
    } lds;
    PfSmem& sm = lds.pf;
    const int rowblocks = a.H / 128;
    int b = blockIdx.x;
    if (a.sh_wdn) {  // the shared expert's blocks first
        const int nb = shared_blocks((a.H / 64 + 1) / 2, (a.T + 63) / 64);
        if (b < nb) {
            shared_down_block<4, X8>(a, b, lds.red);
            return;
        }
        b -= nb;
    }
    const int item = b / rowblocks, rb = b % rowblocks;
    if (item >= uniform(a.meta[kMetaNumMfmaItems])) return;
    const int4 it = a.items[item];
    const int e = uniform(it.x), row0 = uniform(it.y), m = uniform(it.z);
    const int tid = threadIdx.x, w = tid / kWave, lane = tid % kWave, c = lane % 16, g = lane / 16;
    const int wr = w & 1, wt = w >> 1;
    const int K = a.I, chunks = K / 128, quads = a.H / 64;
    const int quad = 2 * rb + wr;
    const int64_t quad_id = (int64_t)e * quads + quad;
    StageSrc src;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int j = min(stage_row(i), m - 1);
        src.row[i] = a.hq + (int64_t)(row0 + j) * K + 16 * stage_piece(i);
    }
    src.srow = a.hs + (int64_t)(row0 + min(64 * (w & 1) + lane, m - 1)) * (K / 32);
    const int ntile = uniform(wave_tiles(m, wt));
    f32x4_t acc[4][kPfTiles];
    pf_gemm(a.wdn + quad_id * chunks * 4096, a.sdn + quad_id * chunks * 256, src, chunks, ntile, sm,
            acc);
    const int n0 = 64 * quad;
#pragma unroll
    for (int t = 0; t < kPfTiles; t++) {
        const int j = tile_token(t, wt, c);
        if (t < ntile && j < m) {
            float* dst = a.y + (int64_t)(row0 + j) * a.H + n0 + 4 * g;
#pragma unroll
            for (int rg = 0; rg < 4; rg++)
                *reinterpret_cast<float4*>(dst + 16 * rg) =
                    make_float4(acc[rg][t][0], acc[rg][t][1], acc[rg][t][2], acc[rg][t][3]);
        }
    }
}

}  // namespace

hipError_t launch_quantize_x_mxfp8(const uint16_t* x, int T, int H, uint8_t* codes,
                                   uint8_t* scales, hipStream_t stream) {
    const int64_t nblocks = (int64_t)T * H / 32;
    if (nblocks == 0) return hipSuccess;
    quantize_x_mxfp8_kernel<<<(unsigned)((nblocks + kQuantThreads - 1) / kQuantThreads),
                              kQuantThreads, 0, stream>>>(x, nblocks, codes, scales);
    return hipGetLastError();
}

hipError_t launch_mx8_gate_up(const GemmArgs& a, int max_items, hipStream_t stream) {
    const int sh = a.sh_wgu ? shared_blocks(a.I / 32, (a.T + 63) / 64) : 0;
    mx8_gate_up_kernel<<<sh + max_items * (a.I / 64), kPfThreads, 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_mx8_down(const GemmArgs& a, int max_items, hipStream_t stream) {
    const int sh = a.sh_wdn ? shared_blocks((a.H / 64 + 1) / 2, (a.T + 63) / 64) : 0;
    mx8_down_kernel<<<sh + max_items * (a.H / 128), kPfThreads, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace moe
