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

// one thread per 16-byte output granule
__global__ void __launch_bounds__(kPrepackThreads)
prepack_codes_kernel(const uint8_t* __restrict__ packed, int64_t rows, int64_t cols, int pairs,
                     int64_t total, uint8_t* __restrict__ tiles) {
    const int64_t idx = (int64_t)blockIdx.x * kPrepackThreads + threadIdx.x;
    if (idx >= total) return;
    const int64_t chunks = cols / 128, quads = rows / 64;
    const int lane = (int)(idx % 64), rg = (int)((idx / 64) % 4);
    const int64_t chunk = (idx / 256) % chunks;
    const int64_t quad = (idx / (256 * chunks)) % quads;
    const int64_t mat = idx / (256 * chunks * quads);
    const int r = lane % 16, g = lane / 16;
    const int64_t row = source_row(quad, rg, r, rows, pairs);
    const uint8_t* src = packed + mat * rows * (cols / 2) + row * (cols / 2) + (chunk * 4 + g) * 16;
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

extern "C" int moe_mxfp4_prepack(const uint8_t* packed, const uint8_t* scales,
                                 int64_t num_matrices, int64_t rows, int64_t cols,
                                 int32_t gate_up_pairs, uint8_t* tiles, uint8_t* tile_scales,
                                 void* stream) {
    if (num_matrices < 0 || rows < 0 || cols < 0 || rows % 64 || cols % 128) return MOE_E_SHAPE;
    if (num_matrices == 0 || rows == 0 || cols == 0) return MOE_OK;
    if (!packed || !scales || !tiles || !tile_scales) return MOE_E_NULL;
    if (((uintptr_t)packed & 15u) || ((uintptr_t)tiles & 15u) || ((uintptr_t)tile_scales & 3u))
        return MOE_E_ALIGN;
    const int pairs = gate_up_pairs ? 1 : 0;
    hipStream_t st = (hipStream_t)stream;
    const int64_t n16 = num_matrices * rows * cols / 32;  // 16-byte granules
    const int64_t n4 = num_matrices * rows * cols / 128;  // scale dwords
    moe::prepack_codes_kernel<<<(unsigned)((n16 + moe::kPrepackThreads - 1) / moe::kPrepackThreads),
                                moe::kPrepackThreads, 0, st>>>(packed, rows, cols, pairs, n16, tiles);
    if (hipGetLastError() != hipSuccess) return MOE_E_HIP;
    moe::prepack_scales_kernel<<<(unsigned)((n4 + moe::kPrepackThreads - 1) / moe::kPrepackThreads),
                                 moe::kPrepackThreads, 0, st>>>(scales, rows, cols, pairs, n4,
                                                                tile_scales);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_E_HIP;
}
