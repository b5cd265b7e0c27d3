// device_common.h -- small device helpers shared by the expert GEMM kernels.
#pragma once

#include <utility>

#include "moe_internal.h"
#include "mx_encode.h"

namespace moe {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

// 16-byte streaming load (expert weights are read exactly once)
__device__ inline uint4 load_stream16(const uint8_t* p) {
    u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ inline bf16x2_t as_bf16x2(uint32_t u) { return __builtin_bit_cast(bf16x2_t, u); }

// E8M0 code -> 2^(s-127) as fp32 (2^-127 is an fp32 subnormal; 0xFF -> NaN)
__device__ inline float e8m0_to_f32(uint32_t s) {
    float f = ldexpf(1.0f, (int)s - 127);
    return s == 255u ? __builtin_nanf("") : f;
}

// E8M0 code as the fp32 scale operand of v_cvt_scalef32_* (the code in the
// exponent field: 2^(s-127) for s in 1..254)
__device__ inline float e8m0_as_scale(uint32_t s) { return __uint_as_float(s << 23); }

// 8 E2M1 codes of one word (element 2i in the low nibble of byte i) -> 8
// bf16, block scale applied by the conversion (exact for scale codes 1..254)
__device__ inline bf16x8_t decode8(uint32_t word, float scale) {
    const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 0);
    const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 1);
    const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 2);
    const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 3);
    return bf16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// 8 E4M3 codes (bytes of lo, then of hi; element i in byte i) -> 8 bf16,
// block scale applied by the conversion (E4M3 * 2^k is exact in bf16 while
// the result stays inside bf16's normal range)
__device__ inline bf16x8_t decode8_e4m3(uint32_t lo, uint32_t hi, float scale) {
    const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, scale, false);
    const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, scale, true);
    const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, scale, false);
    const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, scale, true);
    return bf16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

__device__ inline uint32_t word_of(const uint4& v, int q) {
    return q == 0 ? v.x : q == 1 ? v.y : q == 2 ? v.z : v.w;
}

// SiLU(g) * u with the hardware reciprocal (v_rcp_f32, about 1 ulp) in
// place of an IEEE division; 1 + exp(-g) overflowing to infinity gives 0
__device__ inline float silu_mul(float g, float u) {
    return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// fp32 -> bf16 bits, round to nearest even (NaN stays a quiet NaN)
__device__ inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ inline int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// f(std::integral_constant<int, i>) for i = 0 .. N-1 (for builtin operands
// that must be constants)
template <typename F, int... I>
__device__ inline void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ inline void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// One v_mfma_scale_f32_16x16x128_f8f6f4: A in format FA (4: FP4 E2M1, 0: FP8
// E4M3), B FP8 E4M3; the scales are byte SA of sa and byte SB of sb (the
// instruction's op_sel picks them, so packed scale dwords need no unpacking)
template <int FA, int SA, int SB>
__device__ inline f32x4_t mfma_scaled(const i32x8_t& A, const i32x8_t& B, const f32x4_t& c, uint32_t sa,
                                      uint32_t sb) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, c, FA, 0, SA, (int)sa, SB, (int)sb);
}

__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// v -> (hi, lo) = (bf16(v), bf16(v - hi)) (v - hi is exact in fp32); a
// non-finite remainder (v infinite or NaN, or hi rounded to infinity) gives
// lo = 0, so hi alone carries the special value.
__device__ inline void split_bf16(float v, uint16_t& hi, uint16_t& lo) {
    hi = f32_to_bf16_rne(v);
    const float d = v - bf16_to_f32(hi);
    lo = __builtin_isfinite(d) ? f32_to_bf16_rne(d) : (uint16_t)0;
}

// ---- h between the GEMMs on the matrix-core paths with bf16 activations.
// A single bf16 rounding of h costs up to 2^-9 relative per element, and
// stacked on the bf16 rounding of out it can exceed the layer's error
// budget.  So h is carried as three MXFP8 terms, h ~ t0 + t1 + t2: t0 is
// an MXFP8 encoding of h (E4M3 elements, one E8M0 scale per block of 32),
// t1 that of the remainder h - t0, t2 that of h - t0 - t1; each term leaves
// about 2^-4 of what it encodes (measured against its block's largest
// magnitude), so the three hold h to about 2^-12 of that magnitude (8 times
// closer than a bf16 rounding of it).  The down
// GEMM then runs on the scaled FP4 x FP8 matrix cores: per 128-k chunk and
// 16-row group, one v_mfma_scale_f32_16x16x128_f8f6f4 per term, the
// weights' FP4 codes and E8M0 scales taken as they are (no decode).
//
// Layout of row r of h (I values): codes h3q + r * 3I, scales h3s + r *
// h3s_stride(I) (I/8 bytes, the row padded to whole cache lines).
// The B operand of one scaled MFMA gives lane (c, g) the 32 codes of
// k = 16g .. 16g+15 and 64+16g .. 64+16g+15 of the chunk, with the scale
// of MX block g (see mxfp8.hip), so a chunk's codes are stored per lane:
// [chunk][g][term][32 bytes] (96 contiguous bytes per lane and chunk), and
// its scales as [chunk][block g][term 0, 1, 2, 0] (one dword per lane).
constexpr int kHTerms = 3;

// Encode, as three MXFP8 terms, the h values a lane holds for one token:
// v[rg][i] = element 16*rg + 4*g + i of h block `blk` (elements 32*blk ..
// 32*blk+31 of the row), the 32 values of the block spread over the lanes
// (c, 0..3) of the 16x16 MFMA D layout, which agree on each term's scale
// through two cross-lane maxima (every lane of the wave takes part; only
// lanes with `live` store, and the four lanes of a block agree on it).
// Each term's scale is 2^(floor(log2 amax) - 7), one above the OCP MX rule,
// so the scaled values stay below 256 and v_cvt_scalef32_pk_fp8_f32 (two
// values per instruction, rounding to nearest even, not saturating) never
// overflows; the same instruction's inverse gives the rounded values for
// the remainder.  A block holding a NaN or an infinity gets term 0 scale
// 0xFF (NaN) and zero codes.  Agent-coherent stores: in the single-launch
// layer the down unit that reads them may run on another XCD in the same
// launch, whose caches cannot hold these lines before it reads them (rows
// are whole cache lines, and only the row's own expert reads them, after
// its gate_up units are done); plain stores otherwise (PUBLISH = false:
// the kernel boundary makes them visible).
template <bool PUBLISH>
__device__ inline void store_h3(const GemmArgs& a, int64_t row, int blk, const float (&v)[2][4],
                                bool live) {
    typedef short s16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    const int g = (threadIdx.x % kWave) / 16;
    const int chunk = blk >> 2, b = blk & 3;
    float r[2][4];
#pragma unroll
    for (int rg = 0; rg < 2; rg++)
#pragma unroll
        for (int i = 0; i < 4; i++) r[rg][i] = v[rg][i];
    uint32_t code[kHTerms][2] = {};
    uint32_t scales = 0;
    bool special = false;  // a NaN or an infinity in the block (seen by term 0 only)
#pragma unroll
    for (int tm = 0; tm < kHTerms; tm++) {
        uint32_t amax = 0;
#pragma unroll
        for (int rg = 0; rg < 2; rg++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const uint32_t mb = __float_as_uint(r[rg][i]) & 0x7fffffffu;
                amax = mb > amax ? mb : amax;  // NaN bits order above every finite value
            }
        amax = max(amax, (uint32_t)__shfl_xor((int)amax, 16));
        amax = max(amax, (uint32_t)__shfl_xor((int)amax, 32));
        if (tm == 0) special = amax >= 0x7f800000u;
        const int se = special || amax == 0
                           ? -127
                           : min(__builtin_amdgcn_frexp_expf(__uint_as_float(amax)) - 8, 127);
        scales |= (uint32_t)(se + 127) << (8 * tm);
#pragma unroll
        for (int rg = 0; rg < 2; rg++) {
            float q[4];
#pragma unroll
            for (int i = 0; i < 4; i++) q[i] = special ? 0.f : ldexpf(r[rg][i], -se);
            s16x2_t w = {0, 0};
            w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, q[0], q[1], 1.0f, false);
            w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, q[2], q[3], 1.0f, true);
            const uint32_t c = (uint32_t)(uint16_t)w[0] | ((uint32_t)(uint16_t)w[1] << 16);
            code[tm][rg] = c;
            if (tm + 1 < kHTerms) {
                const f32x2_t d0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c, 1.0f, false);
                const f32x2_t d1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c, 1.0f, true);
                r[rg][0] -= ldexpf(d0[0], se);
                r[rg][1] -= ldexpf(d0[1], se);
                r[rg][2] -= ldexpf(d1[0], se);
                r[rg][3] -= ldexpf(d1[1], se);
            }
        }
    }
    if (special) scales = 0xffu;  // term 0 NaN; codes are those of zeros
    if (!live) return;
    uint8_t* crow = a.h3q + row * 3 * a.I;
#pragma unroll
    for (int rg = 0; rg < 2; rg++) {
        // elements 32b + 16rg + 4g .. +3 of the chunk: reader lane (2b + rg) % 4,
        // bytes 16 * (b / 2) + 4g .. +3 of its 32-byte piece
        uint8_t* p = crow + (chunk * 4 + ((2 * b + rg) & 3)) * 96 + (b >> 1) * 16 + 4 * g;
#pragma unroll
        for (int tm = 0; tm < kHTerms; tm++) {
            uint32_t* d = reinterpret_cast<uint32_t*>(p + 32 * tm);
            if constexpr (PUBLISH)
                __hip_atomic_store(d, code[tm][rg], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            else
                *d = code[tm][rg];
        }
    }
    if (g == 0) {
        uint32_t* d = reinterpret_cast<uint32_t*>(a.h3s + row * h3s_stride(a.I) + (chunk * 4 + b) * 4);
        if constexpr (PUBLISH)
            __hip_atomic_store(d, scales, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else
            *d = scales;
    }
}

// Spin (sleeping) until *count >= need, reading it agent-coherently.  Gives
// up after a bounded number of polls (well beyond any real wait) and raises
// *err instead of hanging; the caller goes on either way.
constexpr int kSpinLimit = 1 << 22;
__device__ inline void wait_count(const int32_t* count, int need, int32_t* err) {
    for (int it = 0;; it++) {
        if (__hip_atomic_load(count, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= need) return;
        if (it >= kSpinLimit) {
            atomicOr(err, 1);
            return;
        }
        __builtin_amdgcn_s_sleep(2);
    }
}

// sum_j w[t,j] * y[pos[t,j], n] over the k slots of token t, in slot order
// j = 0..k-1, fp32, plus the shared expert's y[sh_row0 + t, n] if there is
// one.  Everything is read with agent-coherent loads: other workgroups of
// the running kernel may have written it, on another XCD.  The slot indices
// and weights, then the y values, are fetched 8 slots at a time with
// unconditional loads (indices clamped to k-1), so each batch costs two
// memory latencies rather than two per slot.
__device__ inline float combine_column(const GemmArgs& a, int t, int n) {
    const int64_t base = (int64_t)t * a.k;
    float v = 0.f;
    for (int j0 = 0; j0 < a.k; j0 += 8) {
        int p[8];
        float w[8], yv[8];
#pragma unroll
        for (int u = 0; u < 8; u++) {
            const int j = min(j0 + u, a.k - 1);
            p[u] = a.pos ? __hip_atomic_load(a.pos + base + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                         : (int)(base + j);  // no pos: rows are the slots
            w[u] = __hip_atomic_load(a.wts + base + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int u = 0; u < 8; u++)
            yv[u] = __hip_atomic_load(a.y + (int64_t)p[u] * a.H + n, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (int u = 0; u < 8; u++)
            if (j0 + u < a.k) v = fmaf(w[u], yv[u], v);
    }
    if (a.sh_wgu)  // the shared expert, weight 1, after the k routed terms
        v += __hip_atomic_load(a.y + (int64_t)(a.sh_row0 + t) * a.H + n, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    return v;
}

// out[t, n0 .. n0+width) rounded to bf16, one column per thread of the block
__device__ inline void combine_tile(const GemmArgs& a, int t, int n0, int width) {
    for (int c = threadIdx.x; c < width; c += blockDim.x)
        a.out[(int64_t)t * a.H + n0 + c] = f32_to_bf16_rne(combine_column(a, t, n0 + c));
}

// The token rows of one MFMA item, for the lane's column j of a tile:
// row(j) is its h and y row, token(a, j) the token whose x it reads.
// SortedRows: a routed item, rows row0 .. row0+m-1 of the sorted order,
// slot sorted[row0 + j].  SlotRows: a self-routed expert of at most 16
// tokens (one column tile), where lane c holds the slot t*k + rank of its
// column's token, which is also its h and y row.  TokenRows: the shared
// expert, tokens t0 .. t0+m-1 in order, rows base + t.
struct SortedRows {
    int row0, m;
    __device__ int row(int j) const { return row0 + j; }
    __device__ int slot(const GemmArgs& a, int j) const { return a.sorted[row0 + j]; }
    __device__ int token(const GemmArgs& a, int j) const { return a.sorted[row0 + j] / a.k; }
};
struct TokenRows {
    int t0, m, base;
    __device__ int row(int j) const { return base + t0 + j; }
    __device__ int token(const GemmArgs&, int j) const { return t0 + j; }
};
struct SlotRows {
    int m, lane_slot;
    __device__ int token(const GemmArgs& a, int) const { return lane_slot / a.k; }
    __device__ int row(int) const { return lane_slot; }
    __device__ int slot(const GemmArgs&, int) const { return lane_slot; }
};
// ListRows: a self-routed expert whose slots sit in its slot list (read
// when needed, after the first weight loads are in flight)
struct ListRows {
    int m;
    const int32_t* slots;
    __device__ int row(int j) const { return slots[j]; }
    __device__ int slot(const GemmArgs&, int j) const { return slots[j]; }
    __device__ int token(const GemmArgs& a, int j) const { return slots[j] / a.k; }
};

// One wave's share of a down-projection tile: acc[rg][t] holds rows 4g..4g+3
// of row group rg of output quad `quad` (columns 64q + 16rg + 4g + i of out)
// for token row 16t + c of the item (lane (c, g), the 16x16 MFMA D layout).
// Each token's values go to its y row (rows.row): plain 16-byte stores when
// a later kernel combines (the kernel boundary makes them visible), or,
// with PUBLISH (a single-launch layer, whose own workgroups combine after
// grid_combine's barrier), agent-coherent stores.
template <int NT, bool PUBLISH, typename Rows>
__device__ inline void store_down_tile(const GemmArgs& a, int quad, const Rows& rows,
                                       const f32x4_t (&acc)[4][NT]) {
    const int m = rows.m;
    const int lane = threadIdx.x % kWave, c = lane % 16, g = lane / 16;
    const int n0 = 64 * quad;
#pragma unroll
    for (int t = 0; t < NT; t++) {
        const int j = 16 * t + c;
        if (j >= m) continue;
        float* dst = a.y + (int64_t)rows.row(j) * a.H + n0 + 4 * g;
#pragma unroll
        for (int rg = 0; rg < 4; rg++) {
            if (!PUBLISH) {
                *reinterpret_cast<float4*>(dst + 16 * rg) =
                    make_float4(acc[rg][t][0], acc[rg][t][1], acc[rg][t][2], acc[rg][t][3]);
                continue;
            }
            const uint64_t lo = (uint64_t)__float_as_uint(acc[rg][t][0]) |
                                ((uint64_t)__float_as_uint(acc[rg][t][1]) << 32);
            const uint64_t hi = (uint64_t)__float_as_uint(acc[rg][t][2]) |
                                ((uint64_t)__float_as_uint(acc[rg][t][3]) << 32);
            __hip_atomic_store(reinterpret_cast<uint64_t*>(dst + 16 * rg), lo, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(reinterpret_cast<uint64_t*>(dst + 16 * rg + 2), hi,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// The combine of a single-launch layer, run by every workgroup once its
// unit queue is exhausted.  Each wave first waits for its own stores (y
// rows, h, routing) to complete; then the workgroup adds the units it ran,
// `units`, to `done`.  The workgroup whose addition brings `done` to
// `total`, the units of the whole queue, has seen every y row of the layer
// completed and raises the kGoLines flags at `go` (kGoStride words apart);
// every other workgroup waits (bounded; `err` raised on giving up) for its
// flag, b % kGoLines (one line per 8 or so pollers, rather than the whole
// grid on `done`).  Units are held only by running workgroups, which finish
// them without waiting on anything dequeued later, so the wait ends whether
// or not the whole grid is resident at once.  Then out[t, n] for all T x H
// outputs, one per thread, grid-stride, in the combine kernel's order
// (combine_column).  A combine per (token, column tile) by its last
// finisher instead costs every down unit a store drain, a counter round
// trip and a share of the combines while its workgroup's other waves wait
// at the next unit's barrier: measured on the 9-token, 64-expert layer,
// about 13 us of epilogue per unit and twice the layer time.
__device__ inline void grid_combine(const GemmArgs& a, int units, int total, int32_t* done, int32_t* go,
                                    int32_t* err) {
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's stores completed
    __syncthreads();
    if (threadIdx.x == 0 && total > 0) {
        const bool last = units > 0 && atomicAdd(done, units) + units == total;
        if (last) {
            for (int i = 0; i < kGoLines; i++)
                __hip_atomic_store(go + i * kGoStride, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            wait_count(go + (blockIdx.x % kGoLines) * kGoStride, 1, err);
        }
    }
    __syncthreads();
    const int64_t n_out = (int64_t)a.T * a.H, stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_out; i += stride) {
        const int t = (int)(i / a.H), n = (int)(i % a.H);
        a.out[i] = f32_to_bf16_rne(combine_column(a, t, n));
    }
}

}  // namespace moe
