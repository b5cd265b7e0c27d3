// prepack.hip -- one-time rearrangement of MXFP4 expert matrices from the
// row-major layout into the MFMA tile layout read by mfma.hip.
//
// Same bytes, different order: for every 64-row quad (four 16-row groups)
// and 128-column chunk (four MX blocks), the packed codes become
// [group rg][lane l][16 bytes] with lane l = r + 16 g holding block g of row
// r of the group, and the scale bytes become [lane l][group rg].  With
// gate_up_pairs, quad q takes gate rows 32q..32q+31 as groups 0, 1 and the
// up rows I+32q..I+32q+31 (I = rows / 2) as groups 2, 3.  Pure data
// movement: the codes and scales are copied bit for bit.
//
// MXFP8 matrices (one byte per element, 32 bytes per block) use the same
// quads, chunks, lanes and scale order with each group split in two
// halves: [group rg][half h][lane l][16 bytes], lane l = r + 16 g holding
// bytes 16h..16h+15 of block g of row r -- 8 KB per (quad, chunk).
#include "../../include/moe_mxfp4.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kPrepackThreads = 256;

__device__ inline int64_t source_row(int64_t quad, int rg, int r, int64_t rows, int pairs) {
    if (!pairs) return 64 * quad + 16 * rg + r;
    const int64_t half = rows / 2;
    return (rg < 2 ? 0 : half) + 32 * quad + 16 * (rg & 1) + r;
}

// one thread per 16-byte output granule; halves = 1 (MXFP4: a block is one
// granule) or 2 (MXFP8: a block is two)
__global__ void __launch_bounds__(kPrepackThreads)
prepack_codes_kernel(const uint8_t* __restrict__ packed, int64_t rows, int64_t cols, int pairs,
                     int halves, int64_t total, uint8_t* __restrict__ tiles) {
    const int64_t idx = (int64_t)blockIdx.x * kPrepackThreads + threadIdx.x;
    if (idx >= total) return;
    const int64_t chunks = cols / 128, quads = rows / 64;
    const int lane = (int)(idx % 64);
    int64_t rest = idx / 64;
    const int half = (int)(rest % halves);
    rest /= halves;
    const int rg = (int)(rest % 4);
    rest /= 4;
    const int64_t chunk = rest % chunks;
    rest /= chunks;
    const int64_t quad = rest % quads, mat = rest / quads;
    const int r = lane % 16, g = lane / 16;
    const int64_t row = source_row(quad, rg, r, rows, pairs);
    const int64_t row_bytes = cols / 2 * halves;
    const uint8_t* src = packed + (mat * rows + row) * row_bytes + (chunk * 4 + g) * 16 * halves + 16 * half;
    *reinterpret_cast<uint4*>(tiles + idx * 16) = *reinterpret_cast<const uint4*>(src);
}

// one thread per output dword (the four group scales of one lane)
__global__ void __launch_bounds__(kPrepackThreads)
prepack_scales_kernel(const uint8_t* __restrict__ scales, int64_t rows, int64_t cols, int pairs,
                      int64_t total, uint8_t* __restrict__ tscales) {
    const int64_t idx = (int64_t)blockIdx.x * kPrepackThreads + threadIdx.x;
    if (idx >= total) return;
    const int64_t chunks = cols / 128, quads = rows / 64;
    const int lane = (int)(idx % 64);
    const int64_t chunk = (idx / 64) % chunks;
    const int64_t quad = (idx / (64 * chunks)) % quads;
    const int64_t mat = idx / (64 * chunks * quads);
    const int r = lane % 16, g = lane / 16;
    uint32_t word = 0;
    for (int rg = 0; rg < 4; rg++) {
        const int64_t row = source_row(quad, rg, r, rows, pairs);
        word |= (uint32_t)scales[mat * rows * (cols / 32) + row * (cols / 32) + chunk * 4 + g]
                << (8 * rg);
    }
    *reinterpret_cast<uint32_t*>(tscales + idx * 4) = word;
}

}  // namespace
}  // namespace moe

namespace {

int prepack(const uint8_t* codes, const uint8_t* scales, int64_t num_matrices, int64_t rows,
            int64_t cols, int32_t gate_up_pairs, int halves, uint8_t* tiles, uint8_t* tile_scales,
            void* stream) {
    if (num_matrices < 0 || rows < 0 || cols < 0 || rows % 64 || cols % 128) return MOE_E_SHAPE;
    if (num_matrices == 0 || rows == 0 || cols == 0) return MOE_OK;
    if (!codes || !scales || !tiles || !tile_scales) return MOE_E_NULL;
    if (((uintptr_t)codes & 15u) || ((uintptr_t)tiles & 15u) || ((uintptr_t)tile_scales & 3u))
        return MOE_E_ALIGN;
    const int pairs = gate_up_pairs ? 1 : 0;
    hipStream_t st = (hipStream_t)stream;
    const int64_t n16 = num_matrices * rows * cols / 32 * halves;  // 16-byte granules
    const int64_t n4 = num_matrices * rows * cols / 128;           // scale dwords
    moe::prepack_codes_kernel<<<(unsigned)((n16 + moe::kPrepackThreads - 1) / moe::kPrepackThreads),
                                moe::kPrepackThreads, 0, st>>>(codes, rows, cols, pairs, halves, n16,
                                                               tiles);
    if (hipGetLastError() != hipSuccess) return MOE_E_HIP;
    moe::prepack_scales_kernel<<<(unsigned)((n4 + moe::kPrepackThreads - 1) / moe::kPrepackThreads),
                                 moe::kPrepackThreads, 0, st>>>(scales, rows, cols, pairs, n4,
                                                                tile_scales);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_E_HIP;
}

}  // namespace

extern "C" int moe_mxfp4_prepack(const uint8_t* packed, const uint8_t* scales,
                                 int64_t num_matrices, int64_t rows, int64_t cols,
                                 int32_t gate_up_pairs, uint8_t* tiles, uint8_t* tile_scales,
                                 void* stream) {
    return prepack(packed, scales, num_matrices, rows, cols, gate_up_pairs, 1, tiles, tile_scales,
                   stream);
}

extern "C" int moe_mxfp8_prepack(const uint8_t* codes, const uint8_t* scales,
                                 int64_t num_matrices, int64_t rows, int64_t cols,
                                 int32_t gate_up_pairs, uint8_t* tiles, uint8_t* tile_scales,
                                 void* stream) {
    return prepack(codes, scales, num_matrices, rows, cols, gate_up_pairs, 2, tiles, tile_scales,
                   stream);
}
