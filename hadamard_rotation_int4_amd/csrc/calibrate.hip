// Measurement support for the W4A4 GEMM's roofline, not a step of the method:
// the rate the int8 matrix cores sustain on this chip when nothing else runs
// (qr_calibrate_mfma_i8).
//
// Every wavefront keeps its fragments in registers and issues four
// independent chains of v_mfma_i32_32x32x32_i8, the instruction the tiled GEMM
// uses, with no memory traffic inside the loop.  Each chain has its own B
// fragment, so no two chains compute the same product.  The operands are
// whatever the caller passes; 16 q with q uniform in -8..7 reproduces the
// values the GEMM feeds after unpacking INT4 codes.  Wavefront 0 of each
// workgroup can also record the shader clock counter and the 100 MHz constant
// counter around its loop, which gives the clock the loop ran at.
#include "common.hpp"

namespace qr {

constexpr int CALIB_CHAINS = 4;

__global__ __launch_bounds__(256) void k_calib_mfma_i8(const v4i* __restrict__ frag, int iters,
                                                       int32_t* __restrict__ checksum,
                                                       uint64_t* __restrict__ clocks) {
  const int lane = threadIdx.x & 63;
  const v4i a = frag[lane];
  v4i b[CALIB_CHAINS];
#pragma unroll
  for (int j = 0; j < CALIB_CHAINS; ++j) b[j] = frag[(lane + 7 + 16 * j) & 63];
  uint64_t c0 = 0, t0 = 0;
  if (clocks && threadIdx.x == 0) {
    c0 = clock64();
    t0 = wall_clock64();
  }
  v16i acc[CALIB_CHAINS];
#pragma unroll
  for (int j = 0; j < CALIB_CHAINS; ++j) acc[j] = v16i{};
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int j = 0; j < CALIB_CHAINS; ++j)
      acc[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b[j], acc[j], 0, 0, 0);
  uint32_t s = 0;
#pragma unroll
  for (int j = 0; j < CALIB_CHAINS; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += (uint32_t)acc[j][r];
  checksum[(int64_t)blockIdx.x * 256 + threadIdx.x] = (int32_t)s;
  if (clocks && threadIdx.x == 0) {
    const uint64_t c1 = clock64(), t1 = wall_clock64();
    uint64_t* o = clocks + (int64_t)blockIdx.x * 4;
    o[0] = c0;
    o[1] = c1;
    o[2] = t0;
    o[3] = t1;
  }
}

}  // namespace qr

extern "C" qr_status qr_calibrate_mfma_i8(const void* fragments_i8, int32_t grid, int32_t iters,
                                          int32_t* checksum_i32, uint64_t* clocks_u64,
                                          hipStream_t stream) {
  using namespace qr;
  if (grid < 1 || iters < 1) return QR_ERR_SHAPE;
  if (!fragments_i8 || !checksum_i32) return QR_ERR_NULL;
  if (!aligned(fragments_i8, 16) || !aligned(checksum_i32, 4) ||
      (clocks_u64 && !aligned(clocks_u64, 8)))
    return QR_ERR_ALIGN;
  hipLaunchKernelGGL(k_calib_mfma_i8, dim3(grid), dim3(256), 0, stream, (const v4i*)fragments_i8,
                     iters, checksum_i32, clocks_u64);
  return launch_status();
}
