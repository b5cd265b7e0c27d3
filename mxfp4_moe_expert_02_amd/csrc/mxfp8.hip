// mxfp8.hip -- the prefill path: MXFP8 activations against MXFP4 expert
// weights on the scaled matrix cores of gfx950.
//
// At a prefill chunk every expert sees hundreds of tokens and the layer is
// compute-bound, so the activations are encoded too: x per token along H and
// h per assignment along I, each block of 32 as E4M3 elements with one E8M0
// scale (the same block rule as the weights, with the E4M3 element range),
// and both GEMMs run on v_mfma_scale_f32_16x16x128_f8f6f4 with the FP4
// weights as operand A and the FP8 activations as operand B; the hardware
// applies both block scales.  The weights are the MXFP4 format the pages
// give the experts (bjdmk.com.cn news page, co-design section); the pages
// keep everything else at 8-bit or higher precision (tilert.ai blog, second
// leap), which is what MXFP8 activations are.
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
// A workgroup covers one 64-row quad (wave w = group w) against up to 64
// tokens (four 16-token column tiles) over the whole K.
#include "device_common.h"

namespace moe {
namespace {

typedef int i32x8_t __attribute__((ext_vector_type(8)));

constexpr int kMx8Threads = 256;
constexpr int kTiles = kMx8Tok / 16;  // 4 column tiles

// nearest E4M3 (OCP FN) magnitude code of a >= 0: ties to the even code,
// saturating at 448 (code 126); subnormals below 2^-6 in steps of 2^-9
__device__ inline uint32_t e4m3_mag_code(float a) {
    if (!(a < 448.f)) return 126u;
    if (a < 0.015625f) return (uint32_t)rintf(a * 512.f);
    const int e = (int)((__float_as_uint(a) >> 23) & 0xffu) - 127;  // floor(log2 a)
    const uint32_t t = (uint32_t)rintf(ldexpf(a, 3 - e));             // 8..16
    const uint32_t code = (uint32_t)((e + 7) << 3) + t - 8u;          // t = 16 carries into e+1
    return code > 126u ? 126u : code;
}

// floor(log2(a)) of a finite a > 0 given as float bits
__device__ inline int floor_log2_bits(uint32_t bits) {
    const int ef = (int)(bits >> 23) & 0xff;
    if (ef) return ef - 127;
    return (31 - __clz((int)(bits & 0x7fffffu))) - 149;
}

// MXFP8 encoding of one block of 32 values: scale 2^(floor(log2 amax) - 8)
// (exponent clamped to [-127, 127]; amax == 0 -> code 0), elements RNE to
// E4M3 with saturation; a non-finite value gives scale 0xFF and codes 0.
__device__ inline void encode_block_mxfp8(const float (&v)[32], uint32_t (&codes)[8], uint8_t& scale) {
    uint32_t amax_bits = 0;
    bool finite = true;
#pragma unroll
    for (int i = 0; i < 32; i++) {
        const uint32_t b = __float_as_uint(v[i]) & 0x7fffffffu;
        finite = finite && b < 0x7f800000u;
        amax_bits = b > amax_bits ? b : amax_bits;
    }
#pragma unroll
    for (int i = 0; i < 8; i++) codes[i] = 0;
    if (!finite) {
        scale = 255;
        return;
    }
    int se = amax_bits == 0 ? -127 : floor_log2_bits(amax_bits) - 8;
    se = se < -127 ? -127 : (se > 127 ? 127 : se);
    scale = (uint8_t)(se + 127);
#pragma unroll
    for (int i = 0; i < 32; i++) {
        const float q = ldexpf(v[i], -se);  // exact: a power-of-two scaling
        const uint32_t c = e4m3_mag_code(fabsf(q)) | ((__float_as_uint(q) >> 24) & 0x80u);
        codes[i / 4] |= c << (8 * (i % 4));
    }
}

constexpr int kQuantThreads = 256;

// one thread per block of 32 elements of x
__global__ void __launch_bounds__(kQuantThreads)
quantize_x_mxfp8_kernel(const uint16_t* __restrict__ x, int64_t nblocks, int H,
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
    uint32_t c[8];
    uint8_t s;
    encode_block_mxfp8(v, c, s);
    uint4* dst = reinterpret_cast<uint4*>(codes + b * 32);
    dst[0] = make_uint4(c[0], c[1], c[2], c[3]);
    dst[1] = make_uint4(c[4], c[5], c[6], c[7]);
    scales[b] = s;
    (void)H;
}

// Operand B of one column tile for chunk `chunk`: codes k = 16g..16g+15 and
// 64+16g..64+16g+15 of the chunk and the scale of block 4*chunk+g of this
// lane's token row (zero column if null).
struct BOperand {
    i32x8_t v;
    int scale;
};

__device__ inline BOperand load_b(const uint8_t* row, const uint8_t* srow, int chunk, int g) {
    BOperand b;
    if (row) {
        const uint4* p = reinterpret_cast<const uint4*>(row + chunk * 128 + 16 * g);
        const uint4 lo = p[0], hi = p[4];
        b.v = i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                      (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        b.scale = srow[4 * chunk + g];
    } else {
        b.v = i32x8_t{0, 0, 0, 0, 0, 0, 0, 0};
        b.scale = 127;
    }
    return b;
}

// One wave: group w of a quad over all chunks against up to kTiles token
// tiles.  rows[t] / srows[t]: this lane's token row (codes, scales) in
// column tile t, or null.
__device__ inline void mx8_group(const uint8_t* tiles, const uint8_t* tscales, int w,
                                 const uint8_t* const (&rows)[kTiles],
                                 const uint8_t* const (&srows)[kTiles], int chunks,
                                 f32x4_t (&acc)[kTiles]) {
    const int lane = threadIdx.x % kWave, g = lane / 16;
#pragma unroll
    for (int t = 0; t < kTiles; t++) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    uint4 wa = make_uint4(0, 0, 0, 0);
    uint32_t sa = 0;
    if (chunks > 0) {
        wa = load_stream16(tiles + w * 1024 + lane * 16);
        sa = *reinterpret_cast<const uint32_t*>(tscales + lane * 4);
    }
    for (int c = 0; c < chunks; c++) {
        uint4 wn = make_uint4(0, 0, 0, 0);
        uint32_t sn = 0;
        if (c + 1 < chunks) {  // prefetch the next chunk's weights
            wn = load_stream16(tiles + (int64_t)(c + 1) * 4096 + w * 1024 + lane * 16);
            sn = *reinterpret_cast<const uint32_t*>(tscales + (int64_t)(c + 1) * 256 + lane * 4);
        }
        BOperand b[kTiles];
#pragma unroll
        for (int t = 0; t < kTiles; t++) b[t] = load_b(rows[t], srows[t], c, g);
        const i32x8_t A = i32x8_t{(int)wa.x, (int)wa.y, (int)wa.z, (int)wa.w, 0, 0, 0, 0};
        const int sca = (int)((sa >> (8 * w)) & 0xffu);
#pragma unroll
        for (int t = 0; t < kTiles; t++)
            acc[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                A, b[t].v, acc[t], 4 /* A: FP4 E2M1 */, 0 /* B: FP8 E4M3 */, 0, sca, 0, b[t].scale);
        wa = wn;
        sa = sn;
    }
}

// gate_up, MXFP8 activations: blockIdx.x = item * quads + quad.  Waves 0, 1
// hold gate groups, waves 2, 3 the matching up groups; SiLU(gate) * up is
// formed through LDS and h (32 rows = one MX block per token) is encoded to
// MXFP8 straight from fp32.
__global__ void __launch_bounds__(kMx8Threads)
mx8_gate_up_kernel(GemmArgs a) {
    __shared__ f32x4_t up[2][kTiles][kWave];
    __shared__ float hbuf[kMx8Tok][33];
    const int quads = a.I / 32;
    const int item = blockIdx.x / quads, quad = blockIdx.x % quads;
    if (item >= uniform(a.meta[kMetaNumMfmaItems])) return;
    const int4 it = a.items[item];
    const int e = uniform(it.x), row0 = uniform(it.y), m = uniform(it.z);
    const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave, c = lane % 16, g = lane / 16;
    const int K = a.H, chunks = K / 128;
    const int64_t quad_id = (int64_t)e * quads + quad;
    const uint8_t* rows[kTiles];
    const uint8_t* srows[kTiles];
#pragma unroll
    for (int t = 0; t < kTiles; t++) {
        const int j = 16 * t + c;
        if (j < m) {
            const int token = a.sorted[row0 + j] / a.k;
            rows[t] = a.xq + (int64_t)token * K;
            srows[t] = a.xs + (int64_t)token * (K / 32);
        } else {
            rows[t] = nullptr;
            srows[t] = nullptr;
        }
    }
    f32x4_t acc[kTiles];
    mx8_group(a.wgu + quad_id * chunks * 4096, a.sgu + quad_id * chunks * 256, w, rows, srows,
              chunks, acc);
    if (w >= 2) {
#pragma unroll
        for (int t = 0; t < kTiles; t++) up[w - 2][t][lane] = acc[t];
    }
    __syncthreads();
    if (w < 2) {
#pragma unroll
        for (int t = 0; t < kTiles; t++) {
            const f32x4_t u = up[w][t][lane];
#pragma unroll
            for (int i = 0; i < 4; i++) hbuf[16 * t + c][16 * w + 4 * g + i] = silu_mul(acc[t][i], u[i]);
        }
    }
    __syncthreads();
    if (threadIdx.x < m) {
        const int j = threadIdx.x;
        float v[32];
#pragma unroll
        for (int i = 0; i < 32; i++) v[i] = hbuf[j][i];
        uint32_t cw[8];
        uint8_t s;
        encode_block_mxfp8(v, cw, s);
        uint4* dst = reinterpret_cast<uint4*>(a.hq + (int64_t)(row0 + j) * a.I + 32 * quad);
        dst[0] = make_uint4(cw[0], cw[1], cw[2], cw[3]);
        dst[1] = make_uint4(cw[4], cw[5], cw[6], cw[7]);
        a.hs[(int64_t)(row0 + j) * (a.I / 32) + quad] = s;
    }
}

// down, MXFP8 h: blockIdx.x = item * quads + quad (output rows 64q..64q+63,
// wave w = rows 64q+16w..).  y goes out through agent-coherent stores; the
// block that completes a token's k experts on this quad combines it.
__global__ void __launch_bounds__(kMx8Threads)
mx8_down_kernel(GemmArgs a) {
    __shared__ int s_last[kMx8Tok];
    __shared__ int s_nlast;
    const int quads = a.H / 64;
    const int item = blockIdx.x / quads, quad = blockIdx.x % quads;
    if (item >= uniform(a.meta[kMetaNumMfmaItems])) return;
    const int4 it = a.items[item];
    const int e = uniform(it.x), row0 = uniform(it.y), m = uniform(it.z);
    const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave, c = lane % 16, g = lane / 16;
    const int K = a.I, chunks = K / 128;
    const int64_t quad_id = (int64_t)e * quads + quad;
    const uint8_t* rows[kTiles];
    const uint8_t* srows[kTiles];
#pragma unroll
    for (int t = 0; t < kTiles; t++) {
        const int j = 16 * t + c;
        rows[t] = j < m ? a.hq + (int64_t)(row0 + j) * K : nullptr;
        srows[t] = j < m ? a.hs + (int64_t)(row0 + j) * (K / 32) : nullptr;
    }
    f32x4_t acc[kTiles];
    mx8_group(a.wdn + quad_id * chunks * 4096, a.sdn + quad_id * chunks * 256, w, rows, srows,
              chunks, acc);
    const int n0 = 64 * quad;
#pragma unroll
    for (int t = 0; t < kTiles; t++) {
        const int j = 16 * t + c;
        if (j < m) {
            float* dst = a.y + (int64_t)(row0 + j) * a.H + n0 + 16 * w + 4 * g;
            const uint64_t lo = (uint64_t)__float_as_uint(acc[t][0]) |
                                ((uint64_t)__float_as_uint(acc[t][1]) << 32);
            const uint64_t hi = (uint64_t)__float_as_uint(acc[t][2]) |
                                ((uint64_t)__float_as_uint(acc[t][3]) << 32);
            __hip_atomic_store(reinterpret_cast<uint64_t*>(dst), lo, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(reinterpret_cast<uint64_t*>(dst + 2), hi, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");  // this wave's y stores done
    if (threadIdx.x == 0) s_nlast = 0;
    __syncthreads();
    if (threadIdx.x < m) {
        const int token = a.sorted[row0 + threadIdx.x] / a.k;
        if (atomicAdd(&a.tile_done[token * quads + quad], 1) == a.k - 1)
            s_last[atomicAdd(&s_nlast, 1)] = token;
    }
    __syncthreads();
    const int nlast = s_nlast;
    // combine: four tokens at a time, one column per thread
    for (int i0 = 0; i0 < nlast; i0 += kMx8Threads / 64) {
        const int i = i0 + (int)(threadIdx.x / 64);
        if (i < nlast) {
            const int t = s_last[i], n = n0 + lane;
            float v = 0.f;
            for (int j = 0; j < a.k; j++) {
                const float wt = a.wts[(int64_t)t * a.k + j];
                const int p = a.pos[(int64_t)t * a.k + j];
                v = fmaf(wt, __hip_atomic_load(a.y + (int64_t)p * a.H + n, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT), v);
            }
            a.out[(int64_t)t * a.H + n] = f32_to_bf16_rne(v);
        }
    }
}

}  // namespace

hipError_t launch_quantize_x_mxfp8(const uint16_t* x, int T, int H, uint8_t* codes,
                                   uint8_t* scales, hipStream_t stream) {
    const int64_t nblocks = (int64_t)T * H / 32;
    if (nblocks == 0) return hipSuccess;
    quantize_x_mxfp8_kernel<<<(unsigned)((nblocks + kQuantThreads - 1) / kQuantThreads),
                              kQuantThreads, 0, stream>>>(x, nblocks, H, codes, scales);
    return hipGetLastError();
}

hipError_t launch_mx8_gate_up(const GemmArgs& a, int max_items, hipStream_t stream) {
    mx8_gate_up_kernel<<<max_items * (a.I / 32), kMx8Threads, 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_mx8_down(const GemmArgs& a, int max_items, hipStream_t stream) {
    mx8_down_kernel<<<max_items * (a.H / 64), kMx8Threads, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace moe
