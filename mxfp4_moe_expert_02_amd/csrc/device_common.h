// device_common.h -- small device helpers shared by the expert GEMM kernels.
#pragma once

#include "moe_internal.h"

namespace moe {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

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

__device__ inline float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

// fp32 -> bf16 bits, round to nearest even (NaN stays a quiet NaN)
__device__ inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ inline int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Four bf16 of h through an agent-coherent 8-byte store: in the
// single-launch layer the down unit that reads them may run on another XCD
// in the same launch (its L2 never held these lines in this launch).
__device__ inline void store_h4(uint16_t* dst, ushort4 v) {
    const uint64_t u = (uint64_t)v.x | ((uint64_t)v.y << 16) | ((uint64_t)v.z << 32) |
                       ((uint64_t)v.w << 48);
    __hip_atomic_store(reinterpret_cast<uint64_t*>(dst), u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
// j = 0..k-1, fp32, plus the shared expert's y[sh_row0 + t, n] if there is one.  y is read with agent-coherent loads because other
// workgroups of the running kernel wrote it.  The slot indices and weights,
// then the y values, are fetched 8 slots at a time with unconditional loads
// (indices clamped to k-1), so each batch costs two memory latencies rather
// than two per slot.
__device__ inline float combine_column(const GemmArgs& a, int t, int n) {
    const int64_t base = (int64_t)t * a.k;
    float v = 0.f;
    for (int j0 = 0; j0 < a.k; j0 += 8) {
        int p[8];
        float w[8], yv[8];
#pragma unroll
        for (int u = 0; u < 8; u++) {
            const int j = min(j0 + u, a.k - 1);
            p[u] = a.pos[base + j];
            w[u] = a.wts[base + j];
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
// Each token's values go to its y row (rows.row).
//
// COMBINE = false (split launch): plain 16-byte stores; the combine runs as
// its own kernel after this one (combine.hip), which the kernel boundary
// makes see every y row.  COMBINE = true (single-launch layer): the y rows
// go out through agent-coherent stores, then the wave counts its (token,
// quad) tiles done and the wave that completes a token's k experts on the
// quad combines those 64 columns (the last finisher), in slot order.
template <int NT, bool COMBINE, typename Rows>
__device__ inline void store_down_tile(const GemmArgs& a, int quad, const Rows& rows,
                                       const f32x4_t (&acc)[4][NT]) {
    const int m = rows.m;
    const int quads = a.H / 64;
    const int lane = threadIdx.x % kWave, c = lane % 16, g = lane / 16;
    const int n0 = 64 * quad;
#pragma unroll
    for (int t = 0; t < NT; t++) {
        const int j = 16 * t + c;
        if (j >= m) continue;
        float* dst = a.y + (int64_t)rows.row(j) * a.H + n0 + 4 * g;
#pragma unroll
        for (int rg = 0; rg < 4; rg++) {
            if (!COMBINE) {
                *reinterpret_cast<float4*>(dst + 16 * rg) =
                    make_float4(acc[rg][t][0], acc[rg][t][1], acc[rg][t][2], acc[rg][t][3]);
                continue;
            }
            // agent-coherent stores: the combining wave may run on another XCD
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
    if constexpr (COMBINE) {  // routed items only (rows.row0)
        // every y store of this wave has completed before it counts the tiles
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
        for (int j0 = 0; j0 < m; j0 += kWave) {
            const int j = j0 + lane;
            int token = -1;
            bool last = false;
            if (j < m) {
                token = a.sorted[rows.row0 + j] / a.k;
                last = atomicAdd(&a.tile_done[token * quads + quad], 1) == a.k - 1;
            }
            uint64_t todo = __ballot(last);
            while (todo) {
                const int src = __builtin_ctzll(todo);
                todo &= todo - 1;
                const int t = __builtin_amdgcn_readlane(token, src);
                // out[t, n0 + lane] = sum_j w[t,j] * y[pos[t,j], n0 + lane], slot order
                a.out[(int64_t)t * a.H + n0 + lane] = f32_to_bf16_rne(combine_column(a, t, n0 + lane));
            }
        }
    }
}

}  // namespace moe
