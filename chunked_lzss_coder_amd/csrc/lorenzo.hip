// lorenzo.hip -- the Lorenzo-quantizer front end (include/gpulz_lorenzo.h).
//
// A thread owns four consecutive cells of one row.  For each lower-neighbour
// row it needs (itself, y - 1, z - 1, both) it loads the five floats x0 - 1 ..
// x0 + 3, quantizes them once (q = round-half-even(f / 2eb) in double
// precision, the same operations as a plain per-cell evaluation, so every
// code is bit-identical to it) and adds their signed differences to the four
// cells' residuals: 2.5 divisions per cell in 2-D, 5 in 3-D, instead of the 4
// or 8 of a per-cell recomputation.  Codes are stored as u32; clamped cells
// are counted with one atomic per wave.
#include "gpulz_lorenzo.h"

#include <math.h>

#include "common.h"

namespace gpulz {
namespace {

constexpr uint32_t kCellsPerThread = 4;
constexpr int32_t kRadius = 32768;
constexpr int64_t kCodeMax = 65535;

__global__ void zero_counter_kernel(unsigned long long* c) { *c = 0ull; }

__device__ __forceinline__ int64_t quant(float f, double ebx2) {
  return (int64_t)__builtin_rint((double)f / ebx2);
}

__global__ __launch_bounds__(kBlock) void lorenzo_quant_kernel(const float* __restrict__ f, uint32_t nx,
                                                               uint32_t ny, uint32_t nz, uint32_t gx,
                                                               uint64_t threads, double ebx2,
                                                               uint32_t* __restrict__ codes,
                                                               unsigned long long* __restrict__ clamped) {
  const uint64_t t = (uint64_t)blockIdx.x * kBlock + threadIdx.x;
  uint32_t nclamp = 0;
  if (t < threads) {
    const uint32_t t32 = (uint32_t)t;            // threads < 2^32
    const uint32_t row = t32 / gx;               // z * ny + y
    const uint32_t x0 = (t32 % gx) * kCellsPerThread;
    const uint32_t y = row % ny, z = row / ny;
    int64_t d[kCellsPerThread] = {0, 0, 0, 0};
#pragma unroll
    for (uint32_t dz = 0; dz < 2u; ++dz) {
#pragma unroll
      for (uint32_t dy = 0; dy < 2u; ++dy) {
        if (z < dz || y < dy) continue;  // that row lies outside the grid: all 0
        const float* r = f + (uint64_t)((z - dz) * ny + (y - dy)) * nx;
        // q at x0 - 1 .. x0 + 3 (0 outside the row)
        int64_t q[kCellsPerThread + 1];
        q[0] = x0 > 0u ? quant(r[x0 - 1u], ebx2) : 0;
#pragma unroll
        for (uint32_t k = 0; k < kCellsPerThread; ++k) q[k + 1] = x0 + k < nx ? quant(r[x0 + k], ebx2) : 0;
        const bool neg = ((dz + dy) & 1u) != 0u;
#pragma unroll
        for (uint32_t k = 0; k < kCellsPerThread; ++k) {
          const int64_t v = q[k + 1] - q[k];  // the dx = 0 term minus the dx = 1 term
          d[k] += neg ? -v : v;
        }
      }
    }
    uint32_t* out = codes + (uint64_t)row * nx;
#pragma unroll
    for (uint32_t k = 0; k < kCellsPerThread; ++k) {
      if (x0 + k >= nx) continue;
      int64_t c = d[k] + kRadius;
      if (c < 0 || c > kCodeMax) {
        ++nclamp;
        c = c < 0 ? 0 : kCodeMax;
      }
      out[x0 + k] = (uint32_t)c;
    }
  }
  const uint32_t total = lane63(wave_incl_add(nclamp));
  if (total != 0u && (threadIdx.x & 63u) == 0u) atomicAdd(clamped, (unsigned long long)total);
}

}  // namespace
}  // namespace gpulz

using namespace gpulz;

extern "C" GPULZ_API int gpulz_lorenzo_quant(const float* d_field, uint32_t nx, uint32_t ny, uint32_t nz, double eb,
                                             uint32_t* d_codes, uint64_t* d_clamped, hipStream_t stream) {
  if (!d_field || !d_codes || !d_clamped || nx == 0u || ny == 0u || nz == 0u) return GPULZ_ERR_INVALID_ARG;
  if ((uint64_t)nx * ny * nz >= (1ull << 32)) return GPULZ_ERR_INVALID_ARG;
  if ((((uintptr_t)d_field) & 3u) || (((uintptr_t)d_codes) & 3u) || (((uintptr_t)d_clamped) & 7u))
    return GPULZ_ERR_INVALID_ARG;
  if (!(eb > 0.0) || !isfinite(eb) || !isfinite(2.0 * eb)) return GPULZ_ERR_INVALID_ARG;
  const uint32_t gx = (nx + kCellsPerThread - 1u) / kCellsPerThread;
  const uint64_t threads = (uint64_t)gx * ny * nz;
  const uint64_t blocks = (threads + kBlock - 1u) / kBlock;
  hipLaunchKernelGGL(zero_counter_kernel, dim3(1), dim3(1), 0, stream, (unsigned long long*)d_clamped);
  hipLaunchKernelGGL(lorenzo_quant_kernel, dim3((uint32_t)blocks), dim3(kBlock), 0, stream, d_field, nx, ny, nz, gx,
                     threads, 2.0 * eb, d_codes, (unsigned long long*)d_clamped);
  return hipGetLastError() == hipSuccess ? GPULZ_OK : GPULZ_ERR_HIP;
}
