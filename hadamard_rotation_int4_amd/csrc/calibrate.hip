// Measurement support for the rooflines, not steps of the method:
//  * qr_calibrate_mfma_i8: the rate the int8 matrix cores of the W4A4 GEMM
//    sustain on this chip when nothing else runs;
//  * qr_calibrate_stream: the rate of a plain stream with the rotate+quant
//    kernels' mix of traffic, 16 bytes read for every 4 written.
//
// The matrix-core loop: every wavefront keeps its fragments in registers and issues four
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

// Grid-stride stream: chunk i (16 bytes) of src is read once (non-temporal) and
// the XOR of its four dwords is written to dst[i] (non-temporal); each lane
// keeps two chunks in flight.
__global__ __launch_bounds__(256) void k_calib_stream(const v4u* __restrict__ src, int64_t n16,
                                                      uint32_t* __restrict__ dst) {
  const int64_t stride = (int64_t)gridDim.x * 512;
  for (int64_t i = (int64_t)blockIdx.x * 512 + threadIdx.x; i < n16; i += stride) {
    const int64_t i1 = i + 256;
    const v4u a = __builtin_nontemporal_load(src + i);
    const v4u b = i1 < n16 ? __builtin_nontemporal_load(src + i1) : v4u{0u, 0u, 0u, 0u};
    __builtin_nontemporal_store(a[0] ^ a[1] ^ a[2] ^ a[3], dst + i);
    if (i1 < n16) __builtin_nontemporal_store(b[0] ^ b[1] ^ b[2] ^ b[3], dst + i1);
  }
}

}  // namespace qr

extern "C" qr_status qr_calibrate_stream(const void* src, int64_t n16, void* dst_u32, int32_t grid,
                                         hipStream_t stream) {
  using namespace qr;
  if (n16 < 0 || grid < 1) return QR_ERR_SHAPE;
  if (n16 == 0) return QR_OK;
  if (!src || !dst_u32) return QR_ERR_NULL;
  if (!aligned(src, 16) || !aligned(dst_u32, 4)) return QR_ERR_ALIGN;
  hipLaunchKernelGGL(k_calib_stream, dim3(grid), dim3(256), 0, stream, (const v4u*)src, n16,
                     (uint32_t*)dst_u32);
  return launch_status();
}

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
