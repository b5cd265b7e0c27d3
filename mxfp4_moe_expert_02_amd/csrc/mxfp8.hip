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
// Both operands go from global memory straight into LDS (direct global ->
// LDS loads, 16 bytes per lane), three chunks deep: A (the two quads' tiles,
// already in operand order) and B (XOR-swizzled rows, so that operand reads
// are free of bank conflicts); each wave then reads its A and B operands of
// the chunk from LDS.  The token rows of x are gathered through the routing
// order; h rows are already in that order.
#include "mfma_items.h"
#include "mx_encode.h"

namespace moe {
namespace {

constexpr int kPfWavesPerEu = 2;  // launch bound of the prefill kernels

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

// Staged operands of one 128-k chunk, three chunks deep:
//   B: 128 token rows of 128 code bytes, 16-byte piece p of row r in slot
//      p ^ ((r >> 1) & 7) (a 16-lane quarter of an operand read then covers
//      the 64 banks once), and the chunk's 4 block scales per token;
//   A: the two quads' 4 KB weight tiles (the global tile layout as is) and
//      their 256 scale bytes.
constexpr int kPfStages = 3;
struct PfSmem {
    alignas(16) uint8_t b[kPfStages][kMx8Tok * 128];
    alignas(16) uint8_t a[kPfStages][2][4096];
    alignas(16) uint32_t bs[kPfStages][kMx8Tok];
    alignas(16) uint32_t as[kPfStages][2][kWave];
};

__device__ inline int b_slot(int row, int piece) { return piece ^ ((row >> 1) & 7); }

// Direct global -> LDS loads (16 or 4 bytes per lane; lane l's bytes land
// at lds + 16 l, or 4 l).  Written as inline asm so that the compiler does
// not treat every later LDS read as depending on them (it would wait for all
// of them, a full drain, before each read); the main loop waits for them
// itself.  M0 (the LDS base) is saved and restored inside the block.
typedef __attribute__((address_space(3))) const void lds_cvoid_t;
__device__ inline uint32_t lds_addr(const void* p) {
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_cvoid_t*)p);
}
__device__ inline void dma16(const uint8_t* src, uint32_t lds) {
    uint32_t save;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(save)
        : "v"(src), "s"(lds)
        : "memory");
}
__device__ inline void dma4(const uint8_t* src, uint32_t lds) {
    uint32_t save;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %1, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(save)
        : "v"(src), "s"(lds)
        : "memory");
}

// Two workgroup shapes share the loop below.  The routed experts (F8 =
// false): two quads of MXFP4 weights (4 KB per quad and chunk), waves (wr,
// wt) = (w & 1, w >> 1), token tiles wt, wt+2, wt+4, wt+6.  The shared
// expert (F8 = true): one quad of MXFP8 weights (8 KB per chunk, the
// MXFP8 tile layout), waves wt = w, token tiles wt, wt+4.  Both stage the
// same 8 KB of A per chunk.
//
// Where this lane's loads of a chunk come from.  Wave w fills B rows
// 32w .. 32w+31 with four 1 KB loads (lane l: row 32w + 8i + l/8, slot
// l % 8); waves 0, 1 load the scale words of tokens 64w + l; wave 2 (and,
// with two quads, wave 3) the scale dword of lane l of quad w - 2 (with one
// quad, wave 3 loads B's scale words again into a spare slot); and wave w
// loads the two 1 KB pieces 2w, 2w + 1 of the chunk's 8 KB of A.  Seven
// loads per wave per chunk.  Rows past the item's m tokens repeat row m-1:
// they only feed output columns that are never stored.
struct StageSrc {
    const uint8_t* row[4];  // code bytes of the row's piece for this lane, chunk 0
    const uint8_t* sc;      // this lane's scale bytes, chunk 0 (B or A scales)
    int sc_step;            // bytes per chunk of sc: 4 (B) or 256 (A)
    const uint8_t* a[2];    // this wave's two A pieces, chunk 0 (lane offset included)
    int a_step;             // bytes per chunk of a quad's A: 4096 (MXFP4) or 8192 (MXFP8)
};
constexpr int kPfLoadsPerChunk = 7;  // the vmcnt(7) of pf_mainloop

__device__ inline void stage_issue(const StageSrc& src, int chunk, PfSmem& sm, int buf) {
    const int w = threadIdx.x / kWave;
#pragma unroll
    for (int i = 0; i < 4; i++) dma16(src.row[i] + chunk * 128, lds_addr(&sm.b[buf][(32 * w + 8 * i) * 128]));
    dma4(src.sc + chunk * src.sc_step,
         lds_addr(w < 2 ? (const void*)&sm.bs[buf][64 * w] : (const void*)&sm.as[buf][w - 2][0]));
#pragma unroll
    for (int j = 0; j < 2; j++)
        dma16(src.a[j] + (int64_t)chunk * src.a_step, lds_addr(&sm.a[buf][0][(2 * w + j) * 1024]));
}

// lane's LDS row for staging load i of wave w, and the piece it carries
__device__ inline int stage_row(int i) { return 32 * (threadIdx.x / kWave) + 8 * i + (threadIdx.x % kWave) / 8; }
__device__ inline int stage_piece(int i) { return b_slot(stage_row(i), threadIdx.x % 8); }

// The loads of a workgroup's chunks: B rows from `code_row`, this lane's
// scale bytes, and the A tiles of the workgroup's quads (tiles/tscales at
// its first quad; consecutive quads are consecutive in the tile layout).
template <bool F8, typename RowFn>
__device__ inline StageSrc stage_src(RowFn code_row, const uint8_t* scale_row, const uint8_t* tiles,
                                     const uint8_t* tscales, int chunks) {
    const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    constexpr int kQuadChunk = F8 ? 8192 : 4096;
    StageSrc src;
#pragma unroll
    for (int i = 0; i < 4; i++) src.row[i] = code_row(stage_row(i)) + 16 * stage_piece(i);
    if (w < 2 || (F8 && w == 3)) {
        src.sc = scale_row;
        src.sc_step = 4;
    } else {
        src.sc = tscales + (int64_t)(w - 2) * chunks * 256 + lane * 4;
        src.sc_step = 256;
    }
    src.a_step = kQuadChunk;
#pragma unroll
    for (int j = 0; j < 2; j++) {
        const int piece = 2 * w + j;  // 1 KB piece of the workgroup's 8 KB of A per chunk
        src.a[j] = tiles + (int64_t)(piece * 1024 / kQuadChunk) * chunks * kQuadChunk +
                   (piece * 1024) % kQuadChunk + lane * 16;
    }
    return src;
}

// A operand of one chunk: row groups 0..3 of the wave's quad (MXFP4: one
// 16-byte word per group; MXFP8: two), and their four scale bytes
template <bool F8>
struct AOperand {
    uint4 w[4][F8 ? 2 : 1];
    uint32_t s;
};

// this wave's A operand of the chunk in LDS buffer `buf`.  An 8-bit
// operand takes, in lane (r, g), the 16-byte pieces g and g + 4 of row r's
// 128 bytes (as B does), with the scale of block g; the MXFP8 tile layout
// keeps pieces 2g', 2g' + 1 in lane (r, g') -- piece p of row r sits in
// half p % 2 of lane r + 16 (p / 2).
template <bool F8>
__device__ inline void read_a(const PfSmem& sm, int buf, AOperand<F8>& a) {
    const int lane = threadIdx.x % kWave, wr = F8 ? 0 : (threadIdx.x / kWave) & 1;
    const uint8_t* base = &sm.a[buf][0][0] + wr * 4096;
    if constexpr (F8) {
        const int r = lane % 16, g = lane / 16;
        const int lo = (g & 1) * 1024 + (r + 16 * (g >> 1)) * 16;  // piece g
        const int hi = (g & 1) * 1024 + (r + 16 * ((g >> 1) + 2)) * 16;  // piece g + 4
#pragma unroll
        for (int rg = 0; rg < 4; rg++) {
            a.w[rg][0] = *reinterpret_cast<const uint4*>(base + rg * 2048 + lo);
            a.w[rg][F8 ? 1 : 0] = *reinterpret_cast<const uint4*>(base + rg * 2048 + hi);
        }
    } else {
#pragma unroll
        for (int rg = 0; rg < 4; rg++)
            a.w[rg][0] = *reinterpret_cast<const uint4*>(base + rg * 1024 + lane * 16);
    }
    a.s = sm.as[buf][wr][lane];
}

// Column tile t of a wave is token tile 2t + wt of the item (two token
// waves) or 4t + wt (four): interleaved, so the waves stay balanced on
// ragged items.
template <bool F8>
__device__ inline int tile_token(int t, int wt, int c) { return 16 * ((F8 ? 4 : 2) * t + wt) + c; }
template <bool F8>
__device__ inline int token_wave() { return F8 ? threadIdx.x / kWave : (threadIdx.x / kWave) >> 1; }

template <int NT>
struct BOperands {
    i32x8_t v[NT > 0 ? NT : 1];
    int s[NT > 0 ? NT : 1];
};

// this wave's B operands of the chunk in LDS buffer `buf`
template <int NT, bool F8>
__device__ inline void read_b(const PfSmem& sm, int buf, BOperands<NT>& b) {
    const int lane = threadIdx.x % kWave, c = lane % 16, g = lane / 16;
    const int wt = token_wave<F8>();
#pragma unroll
    for (int t = 0; t < NT; t++) {
        const int row = tile_token<F8>(t, wt, c);
        const uint8_t* base = &sm.b[buf][row * 128];
        const uint4 lo = *reinterpret_cast<const uint4*>(base + 16 * b_slot(row, g));
        const uint4 hi = *reinterpret_cast<const uint4*>(base + 16 * b_slot(row, g + 4));
        b.s[t] = (int)((sm.bs[buf][row] >> (8 * g)) & 0xffu);
        b.v[t] = i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                         (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
}

template <int NT, bool F8>
__device__ inline void chunk_mfma(const AOperand<F8>& ac, const BOperands<NT>& b,
                                  f32x4_t (&acc)[4][kPfTiles]) {
#pragma unroll
    for (int rg = 0; rg < 4; rg++) {
        const uint4& lo = ac.w[rg][0];
        const uint4& hi = ac.w[rg][F8 ? 1 : 0];
        const i32x8_t A = F8 ? i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                                       (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w}
                             : i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, 0, 0, 0, 0};
        const int sa = (int)((ac.s >> (8 * rg)) & 0xffu);
#pragma unroll
        for (int t = 0; t < NT; t++)
            acc[rg][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                A, b.v[t], acc[rg][t], F8 ? 0 : 4 /* A: FP8 E4M3 or FP4 E2M1 */, 0 /* B: FP8 E4M3 */,
                0, sa, 0, b.s[t]);
    }
}

// The main loop of one workgroup: acc[rg][t] = this wave's quad (group rg)
// x column tile t (t < NT), summed over all `chunks` 128-k chunks.
//
// Chunks are staged three deep: step s waits for this wave's loads of chunk
// s (vmcnt: only chunk s+1's seven loads may still be in flight) and meets
// the other waves at a barrier (without a fence: only LDS is exchanged);
// then it issues chunk s+2's loads into the buffer chunk s-1 left (every
// wave finished reading it before this barrier), reads chunk s's operands
// from LDS and runs its MFMAs.  A load thus has two steps of MFMAs to land.
// Every wave runs the same number of barriers whatever its NT.
template <int NT, bool F8>
__device__ inline void pf_mainloop(const StageSrc& src, int chunks, PfSmem& sm,
                                   f32x4_t (&acc)[4][kPfTiles]) {
#pragma unroll
    for (int rg = 0; rg < 4; rg++)
#pragma unroll
        for (int t = 0; t < kPfTiles; t++) acc[rg][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    stage_issue(src, 0, sm, 0);
    if (chunks > 1) stage_issue(src, 1, sm, 1);
    int buf = 0;
    for (int s = 0; s < chunks; s++) {
        static_assert(kPfLoadsPerChunk == 7, "the wait below counts a chunk's loads");
        if (s + 1 < chunks)
            asm volatile("s_waitcnt vmcnt(7)\n\ts_barrier" ::: "memory");
        else
            asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
        if (s + 2 < chunks) stage_issue(src, s + 2, sm, buf == 0 ? 2 : buf - 1);
        AOperand<F8> ac;
        read_a<F8>(sm, buf, ac);
        BOperands<NT> b;
        read_b<NT, F8>(sm, buf, b);
        chunk_mfma<NT, F8>(ac, b, acc);
        buf = buf == 2 ? 0 : buf + 1;
    }
}

template <bool F8>
__device__ inline void pf_gemm(const StageSrc& src, int chunks, int ntile, PfSmem& sm,
                               f32x4_t (&acc)[4][kPfTiles]) {
    if constexpr (F8) {
        switch (ntile) {
            case 2: pf_mainloop<2, true>(src, chunks, sm, acc); break;
            case 1: pf_mainloop<1, true>(src, chunks, sm, acc); break;
            default: pf_mainloop<0, true>(src, chunks, sm, acc); break;
        }
    } else {
        switch (ntile) {
            case 4: pf_mainloop<4, false>(src, chunks, sm, acc); break;
            case 3: pf_mainloop<3, false>(src, chunks, sm, acc); break;
            case 2: pf_mainloop<2, false>(src, chunks, sm, acc); break;
            case 1: pf_mainloop<1, false>(src, chunks, sm, acc); break;
            default: pf_mainloop<0, false>(src, chunks, sm, acc); break;
        }
    }
}

// column tiles of a token wave that hold any of the item's m tokens
template <bool F8>
__device__ inline int wave_tiles(int m, int wt) {
    const int all = (m + 15) / 16, waves = F8 ? 4 : 2;
    return (all - wt + waves - 1) / waves;
}

// gate_up epilogue: SiLU(gate) * up of this wave's quad for its token
// tiles, encoded to MXFP8 -- the 32 h values of one quad and token (one MX
// block of h) sit in the four lanes (c, 0..3), which agree on the block
// scale through two cross-lane maxima -- into h rows row_base + j.
template <bool F8>
__device__ inline void store_h_mx8(const GemmArgs& a, const f32x4_t (&acc)[4][kPfTiles], int ntile,
                                   int m, int row_base, int quad) {
    const int lane = threadIdx.x % kWave, c = lane % 16, g = lane / 16, wt = token_wave<F8>();
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
        const int j = tile_token<F8>(t, wt, c);
        if (j < m) {
            uint8_t* hrow = a.hq + (int64_t)(row_base + j) * a.I + 32 * quad + 4 * g;
            *reinterpret_cast<uint32_t*>(hrow) = code[0];       // h rows 32q + 4g + i
            *reinterpret_cast<uint32_t*>(hrow + 16) = code[1];  // h rows 32q + 16 + 4g + i
            if (g == 0) a.hs[(int64_t)(row_base + j) * (a.I / 32) + quad] = (uint8_t)scale;
        }
    }
}

// down epilogue: this wave's quad (64 output columns) for its token tiles
// into y rows row_base + j, plain 16-byte stores
template <bool F8>
__device__ inline void store_y_mx8(const GemmArgs& a, const f32x4_t (&acc)[4][kPfTiles], int ntile,
                                   int m, int row_base, int quad) {
    const int lane = threadIdx.x % kWave, c = lane % 16, g = lane / 16, wt = token_wave<F8>();
    const int n0 = 64 * quad;
#pragma unroll
    for (int t = 0; t < kPfTiles; t++) {
        const int j = tile_token<F8>(t, wt, c);
        if (t < ntile && j < m) {
            float* dst = a.y + (int64_t)(row_base + j) * a.H + n0 + 4 * g;
#pragma unroll
            for (int rg = 0; rg < 4; rg++)
                *reinterpret_cast<float4*>(dst + 16 * rg) =
                    make_float4(acc[rg][t][0], acc[rg][t][1], acc[rg][t][2], acc[rg][t][3]);
        }
    }
}

// The shared expert (MXFP8 weights, every token) on the same matrix cores:
// one quad x 128 tokens per workgroup, x / h rows of the tokens themselves,
// h and y rows sh_row0 + t.  Blocks as in mfma_items.h (shared_unit): the
// token tiles of one quad on one XCD.
__device__ inline void mx8_shared_gate_up(const GemmArgs& a, int b, PfSmem& sm) {
    int quad, tile;
    if (!shared_unit(b, a.I / 32, (a.T + kMx8Tok - 1) / kMx8Tok, quad, tile)) return;
    const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
    const int K = a.H, chunks = K / 128, t0 = kMx8Tok * tile, m = min(kMx8Tok, a.T - t0);
    const StageSrc src = stage_src<true>(
        [&](int r) { return a.xq + (int64_t)(t0 + min(r, m - 1)) * K; },
        a.xs + (int64_t)(t0 + min(64 * (w & 1) + lane, m - 1)) * (K / 32),
        a.sh_wgu + (int64_t)quad * chunks * 8192, a.sh_sgu + (int64_t)quad * chunks * 256, chunks);
    const int ntile = uniform(wave_tiles<true>(m, w));
    f32x4_t acc[4][kPfTiles];
    pf_gemm<true>(src, chunks, ntile, sm, acc);
    store_h_mx8<true>(a, acc, ntile, m, a.sh_row0 + t0, quad);
}

__device__ inline void mx8_shared_down(const GemmArgs& a, int b, PfSmem& sm) {
    int quad, tile;
    if (!shared_unit(b, a.H / 64, (a.T + kMx8Tok - 1) / kMx8Tok, quad, tile)) return;
    const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
    const int K = a.I, chunks = K / 128, t0 = kMx8Tok * tile, m = min(kMx8Tok, a.T - t0);
    const int r0 = a.sh_row0 + t0;
    const StageSrc src = stage_src<true>(
        [&](int r) { return a.hq + (int64_t)(r0 + min(r, m - 1)) * K; },
        a.hs + (int64_t)(r0 + min(64 * (w & 1) + lane, m - 1)) * (K / 32),
        a.sh_wdn + (int64_t)quad * chunks * 8192, a.sh_sdn + (int64_t)quad * chunks * 256, chunks);
    const int ntile = uniform(wave_tiles<true>(m, w));
    f32x4_t acc[4][kPfTiles];
    pf_gemm<true>(src, chunks, ntile, sm, acc);
    store_y_mx8<true>(a, acc, ntile, m, r0, quad);
}

// gate_up, MXFP8 activations: blockIdx.x = item * (I / 64) + row block; the
// row block holds quads 2rb, 2rb+1, each 32 gate rows (groups 0, 1) with
// their 32 up rows (groups 2, 3), so SiLU(gate) * up is formed in
// registers.  With a shared expert its blocks come first.
__global__ void __launch_bounds__(kPfThreads, kPfWavesPerEu)
mx8_gate_up_kernel(GemmArgs a) {
    __shared__ PfSmem sm;
    const int rowblocks = a.I / 64;
    int b = blockIdx.x;
    if (a.sh_wgu) {
        const int nb = shared_blocks(a.I / 32, (a.T + kMx8Tok - 1) / kMx8Tok);
        if (b < nb) {
            mx8_shared_gate_up(a, b, sm);
            return;
        }
        b -= nb;
    }
    const int item = b / rowblocks, rb = b % rowblocks;
    if (item >= uniform(a.meta[kMetaNumMfmaItems])) return;
    const int4 it = a.items[item];
    const int e = uniform(it.x), row0 = uniform(it.y), m = uniform(it.z);
    const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
    const int K = a.H, chunks = K / 128, quads = a.I / 32;
    const int64_t pair_id = (int64_t)e * quads + 2 * rb;
    const StageSrc src = stage_src<false>(
        [&](int r) { return a.xq + (int64_t)(a.sorted[row0 + min(r, m - 1)] / a.k) * K; },
        a.xs + (int64_t)(a.sorted[row0 + min(64 * (w & 1) + lane, m - 1)] / a.k) * (K / 32),
        a.wgu + pair_id * chunks * 4096, a.sgu + pair_id * chunks * 256, chunks);
    const int ntile = uniform(wave_tiles<false>(m, token_wave<false>()));
    f32x4_t acc[4][kPfTiles];
    pf_gemm<false>(src, chunks, ntile, sm, acc);
    store_h_mx8<false>(a, acc, ntile, m, row0, 2 * rb + (w & 1));
}

// down, MXFP8 h: blockIdx.x = item * (H / 128) + row block (quads 2rb,
// 2rb+1 of the output rows).  y goes out through plain 16-byte stores; the
// combine runs as its own kernel after this one (combine.hip).  With a
// shared expert its blocks come first.
__global__ void __launch_bounds__(kPfThreads, kPfWavesPerEu)
mx8_down_kernel(GemmArgs a) {
    __shared__ PfSmem sm;
    const int rowblocks = a.H / 128;
    int b = blockIdx.x;
    if (a.sh_wdn) {
        const int nb = shared_blocks(a.H / 64, (a.T + kMx8Tok - 1) / kMx8Tok);
        if (b < nb) {
            mx8_shared_down(a, b, sm);
            return;
        }
        b -= nb;
    }
    const int item = b / rowblocks, rb = b % rowblocks;
    if (item >= uniform(a.meta[kMetaNumMfmaItems])) return;
    const int4 it = a.items[item];
    const int e = uniform(it.x), row0 = uniform(it.y), m = uniform(it.z);
    const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
    const int K = a.I, chunks = K / 128, quads = a.H / 64;
    const int64_t pair_id = (int64_t)e * quads + 2 * rb;
    const StageSrc src = stage_src<false>(
        [&](int r) { return a.hq + (int64_t)(row0 + min(r, m - 1)) * K; },
        a.hs + (int64_t)(row0 + min(64 * (w & 1) + lane, m - 1)) * (K / 32),
        a.wdn + pair_id * chunks * 4096, a.sdn + pair_id * chunks * 256, chunks);
    const int ntile = uniform(wave_tiles<false>(m, token_wave<false>()));
    f32x4_t acc[4][kPfTiles];
    pf_gemm<false>(src, chunks, ntile, sm, acc);
    store_y_mx8<false>(a, acc, ntile, m, row0, 2 * rb + (w & 1));
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
    const int sh = a.sh_wgu ? shared_blocks(a.I / 32, (a.T + kMx8Tok - 1) / kMx8Tok) : 0;
    mx8_gate_up_kernel<<<sh + max_items * (a.I / 64), kPfThreads, 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_mx8_down(const GemmArgs& a, int max_items, hipStream_t stream) {
    const int sh = a.sh_wdn ? shared_blocks(a.H / 64, (a.T + kMx8Tok - 1) / kMx8Tok) : 0;
    mx8_down_kernel<<<sh + max_items * (a.H / 128), kPfThreads, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace moe
