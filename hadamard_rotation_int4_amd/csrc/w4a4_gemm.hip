// W4A4 GEMM with fused dequantization epilogue (qr_w4a4_gemm), for gfx950.
//
// QuaRot paper (activation-quantization and performance paragraphs): the
// 4-bit GEMM accumulates in INT32; the output is the INT32 result times the
// row (token) scale times the column (channel) scale.  Here
//   acc[t, n] = sum_k A[t, k] W[n, k]   exactly, and
//   Y[t, n]   = fp16(fp32(fp32(acc) * a_scale[t]) * w_scale[n]).
//
// Design (MI355X first):
//  * Matrix cores: v_mfma_i32_32x32x32_i8 (int8 in, int32 accumulate).  INT4
//    operands stay packed in HBM and LDS; each lane expands its 8 packed bytes
//    (16 nibbles) into 16 int8 lanes holding 16 * q with two masks and a shift:
//      lo = (x << 4) & 0xF0F0F0F0  -> 16 * (even nibbles)
//      hi =  x       & 0xF0F0F0F0  -> 16 * (odd nibbles)
//    A and W use the same permutation of k, so the dot product is unchanged,
//    and the int32 accumulator holds 256 * acc exactly (|256 acc| <= 256 * 64 * K
//    < 2^31 for K <= 131008); the epilogue shifts it back.
//  * Tiles: 256 x 256 outputs per workgroup of 4 wavefronts, each owning a
//    128 x 128 block = 4 x 4 MFMA tiles (accumulators in the unified register
//    file), K advanced 128 at a time through double-buffered LDS (2 x 32 KB).
//  * LDS layout [kk][half][row][8 bytes]: a 32-lane half wavefront reads 32
//    consecutive rows x 8 bytes = 256 contiguous bytes, conflict-free.
//  * Tile order: workgroup ids are remapped so that the ids the hardware places
//    on one XCD (id % 8) are consecutive, then grouped 8 tile-rows at a time, so
//    the tiles running together on an XCD share A and W panels in its L2.
#include "common.hpp"

namespace qr {

constexpr int BM = 256, BN = 256, BK = 128;  // BK in int4 elements (64 bytes per row)
constexpr int GEMM_THREADS = 256;
constexpr int PANEL_BYTES = 256 * 64;  // one operand's tile per K step: 16 KB

__device__ __forceinline__ v4i unpack16(uint32_t d0, uint32_t d1) {
  v4i r;
  r[0] = (int)((d0 << 4) & 0xF0F0F0F0u);
  r[1] = (int)(d0 & 0xF0F0F0F0u);
  r[2] = (int)((d1 << 4) & 0xF0F0F0F0u);
  r[3] = (int)(d1 & 0xF0F0F0F0u);
  return r;
}

// LDS byte offset of the 8-byte half `hf` (0/1) of k-chunk `kk` (0..3) of row r.
__device__ __forceinline__ int lds_off(int kk, int hf, int r) {
  return ((kk * 2 + hf) * 256 + r) * 8;
}

template <bool DBG>
__global__ __launch_bounds__(GEMM_THREADS, 1) void k_w4a4_gemm(
    const uint8_t* __restrict__ A, const uint16_t* __restrict__ a_scale, int T,
    const uint8_t* __restrict__ W, const uint16_t* __restrict__ w_scale, int N, int K,
    uint16_t* __restrict__ Y, int32_t* __restrict__ acc_dbg, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2][2][PANEL_BYTES];  // [stage][A/W]

  // ---- tile assignment (XCD-aware, grouped) ----
  const int nblk = tiles_m * tiles_n;
  int bid = blockIdx.x;
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  constexpr int GM = 8;
  const int group = bid / (GM * tiles_n);
  const int first_m = group * GM;
  const int gm = min(tiles_m - first_m, GM);
  const int in_group = bid - group * GM * tiles_n;
  const int tm = first_m + in_group % gm;
  const int tn = in_group / gm;
  const int m0 = tm * BM, n0 = tn * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = (wave >> 1) * 128, wn = (wave & 1) * 128;  // wave's block inside the tile
  const int li = lane & 31, lg = lane >> 5;                  // MFMA row/col lane, k-half
  const int64_t rowbytes = K / 2;

  // ---- global -> register staging: 4 x 16 B of A and of W per thread ----
  // chunk id = tid + 256 j: row = id >> 2, kk = id & 3
  const uint8_t* a_src[4];
  const uint8_t* w_src[4];
  int st_row[4], st_kk[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int id = tid + 256 * j;
    st_row[j] = id >> 2;
    st_kk[j] = id & 3;
    const int ar = min(m0 + st_row[j], T - 1);
    const int wr = min(n0 + st_row[j], N - 1);
    a_src[j] = A + (int64_t)ar * rowbytes + st_kk[j] * 16;
    w_src[j] = W + (int64_t)wr * rowbytes + st_kk[j] * 16;
  }
  v4u ra[4], rw[4];
  auto gload = [&](int k0) {  // k0 in elements
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (k0 + st_kk[j] * 32 < K) {
        ra[j] = *(const v4u*)(a_src[j] + k0 / 2);
        rw[j] = *(const v4u*)(w_src[j] + k0 / 2);
      } else {
        ra[j] = v4u{0u, 0u, 0u, 0u};
        rw[j] = v4u{0u, 0u, 0u, 0u};
      }
    }
  };
  auto lstore = [&](int stage) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint8_t* pa = &smem[stage][0][0];
      uint8_t* pw = &smem[stage][1][0];
      *(uint2*)(pa + lds_off(st_kk[j], 0, st_row[j])) = make_uint2(ra[j][0], ra[j][1]);
      *(uint2*)(pa + lds_off(st_kk[j], 1, st_row[j])) = make_uint2(ra[j][2], ra[j][3]);
      *(uint2*)(pw + lds_off(st_kk[j], 0, st_row[j])) = make_uint2(rw[j][0], rw[j][1]);
      *(uint2*)(pw + lds_off(st_kk[j], 1, st_row[j])) = make_uint2(rw[j][2], rw[j][3]);
    }
  };

  v16i acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

  const int ksteps = (K + BK - 1) / BK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int ks = 0; ks < ksteps; ++ks) {
    const int stage = ks & 1;
    if (ks + 1 < ksteps) gload((ks + 1) * BK);
    const uint8_t* pa = &smem[stage][0][0];
    const uint8_t* pw = &smem[stage][1][0];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      v4i af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint2 v = *(const uint2*)(pa + lds_off(kk, lg, wm + i * 32 + li));
        af[i] = unpack16(v.x, v.y);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint2 v = *(const uint2*)(pw + lds_off(kk, lg, wn + j * 32 + li));
        bf[j] = unpack16(v.x, v.y);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    if (ks + 1 < ksteps) lstore(stage ^ 1);
    __syncthreads();
  }

  // ---- epilogue: 32x32 accumulator layout: lane (n = li, k-half lg), register r
  //      holds row 8 (r / 4) + 4 lg + (r % 4) ----
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = n0 + wn + j * 32 + li;
    if (n >= N) continue;
    const float ws = h2f(w_scale[n]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = m0 + wm + i * 32 + 8 * (r >> 2) + 4 * lg + (r & 3);
        if (t < T) {
          const int32_t a = acc[i][j][r] >> 8;  // exact: the accumulator is 256 * acc
          const float as = h2f(a_scale[t]);
          Y[(int64_t)t * N + n] = f2h(__fmul_rn(__fmul_rn((float)a, as), ws));
          if (DBG) acc_dbg[(int64_t)t * N + n] = a;
        }
      }
    }
  }
}

}  // namespace qr

using namespace qr;

extern "C" qr_status qr_w4a4_gemm(const void* a_q, const void* a_scale_f16, int64_t T,
                                  const void* w_q, const void* w_scale_f16, int64_t N, int64_t K,
                                  void* y_f16, int32_t* acc_dbg, hipStream_t stream) {
  if (T < 0 || N < 0 || K <= 0) return QR_ERR_SHAPE;
  if (K % 64 != 0 || K > 131008) return QR_ERR_UNSUPPORTED;
  if (T > INT32_MAX / 2 || N > INT32_MAX / 2) return QR_ERR_SHAPE;
  if (T == 0 || N == 0) return QR_OK;
  if (!a_q || !a_scale_f16 || !w_q || !w_scale_f16 || !y_f16) return QR_ERR_NULL;
  if (!aligned(a_q, 16) || !aligned(w_q, 16) || !aligned(y_f16, 4) || !aligned(a_scale_f16, 2) ||
      !aligned(w_scale_f16, 2) || (acc_dbg && !aligned(acc_dbg, 4)))
    return QR_ERR_ALIGN;
  const int tiles_m = (int)((T + BM - 1) / BM);
  const int tiles_n = (int)((N + BN - 1) / BN);
  const int64_t nblk = (int64_t)tiles_m * tiles_n;
  if (nblk > INT32_MAX) return QR_ERR_SHAPE;
  if (acc_dbg)
    hipLaunchKernelGGL((k_w4a4_gemm<true>), dim3((unsigned)nblk), dim3(GEMM_THREADS), 0, stream,
                       (const uint8_t*)a_q, (const uint16_t*)a_scale_f16, (int)T,
                       (const uint8_t*)w_q, (const uint16_t*)w_scale_f16, (int)N, (int)K,
                       (uint16_t*)y_f16, acc_dbg, tiles_m, tiles_n);
  else
    hipLaunchKernelGGL((k_w4a4_gemm<false>), dim3((unsigned)nblk), dim3(GEMM_THREADS), 0, stream,
                       (const uint8_t*)a_q, (const uint16_t*)a_scale_f16, (int)T,
                       (const uint8_t*)w_q, (const uint16_t*)w_scale_f16, (int)N, (int)K,
                       (uint16_t*)y_f16, (int32_t*)nullptr, tiles_m, tiles_n);
  return launch_status();
}
