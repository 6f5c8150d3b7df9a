// The other two online input quantizers of QuaRot's block, for gfx950:
//
//  * qr_rmsnorm_quant: RMSNorm without its scale, in fp32, fused with the
//    per-token symmetric INT4 quantizer (the QKV, gate and up inputs).  QuaRot
//    paper, method section (the RMSNorm scale is absorbed into the next
//    weights) and activation-quantization paragraph (RMSNorm without scaling
//    in FP32, then per-token quantization).
//  * qr_hadamard_heads_quant: the Hadamard-heads block Z <- Z (H_{n_h} (x) I)
//    in front of the O projection, fused with the same quantizer.  QuaRot
//    paper, attention-block paragraph on (H_{n_h} (x) I)(I (x) H_{d_h}) = H and
//    Figure 6.
//
// Both are HBM-bound streams (2 bytes in, half a byte out per element) with
// little arithmetic, so they run on the VALU: one pass over each row, the row
// held in registers, reductions across the lanes of the row, one store.  The
// _i8 entry points write b-bit codes one per byte instead (QuaRot paper, 6-
// and 8-bit round-to-nearest results).
#include "common.hpp"
#include "quant_common.hpp"

namespace qr {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// ===========================================================================
// k_rms_quant: one wavefront per row, lane l holds the 8-element chunks
// l, l + 64, ... (16-byte loads, 4-byte stores of packed codes).
// ===========================================================================
// Q8: b-bit codes one per byte (8-byte stores per chunk) instead of packed INT4.
template <int NCH, bool Q8>
__global__ __launch_bounds__(256) void k_rms_quant(const uint16_t* __restrict__ x, int64_t T,
                                                   int d, int64_t ld, float eps, float clip,
                                                   int bits, uint8_t* __restrict__ q,
                                                   uint16_t* __restrict__ scale,
                                                   float* __restrict__ rdbg) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= T) return;  // wave-uniform
  const int nch = d >> 3;
  const uint16_t* xr = x + row * ld;
  v4u raw[NCH];
#pragma unroll
  for (int k = 0; k < NCH; ++k) {
    const int c = lane + 64 * k;
    raw[k] = c < nch ? ld_stream(xr + 8 * c) : v4u{0u, 0u, 0u, 0u};
  }
  // sum of squares (each square is exact in fp32; the additions round) and max|x|
  float ss = 0.0f, am = 0.0f;
#pragma unroll
  for (int k = 0; k < NCH; ++k)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a = h2f((uint16_t)(raw[k][j] & 0xffffu)), b = h2f((uint16_t)(raw[k][j] >> 16));
      ss = fmaf(a, a, ss);
      ss = fmaf(b, b, ss);
      am = fmaxf(am, fmaxf(fabsf(a), fabsf(b)));
    }
  ss = wave_sum(ss);
  am = wave_max(am);
  // r = 1 / sqrt(ss / d + eps), each step rounded to fp32; r = 0 when the
  // mean square plus eps is 0 (an all-zero row with eps = 0)
  const float t = __fadd_rn(__fdiv_rn(ss, (float)d), eps);
  const float r = t > 0.0f ? __fdiv_rn(1.0f, __fsqrt_rn(t)) : 0.0f;
  const QRange rg = q_range(Q8 ? bits : 4);
  uint16_t sh;
  float m;
  sym_scale(am, r, clip, &sh, &m, rg.qmax);
  // |x m| <= qmax (1 + 2^-11) < qmax + 1/2 unless clip < 1 or the scale is subnormal
  const bool clamp = clip < 1.0f || (sh & 0x7fffu) < 0x0400u;
  uint8_t* qr_ = q + row * (Q8 ? d : d / 2);
#pragma unroll
  for (int k = 0; k < NCH; ++k) {
    const int c = lane + 64 * k;
    if (c < nch) {
      float v[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[2 * j] = h2f((uint16_t)(raw[k][j] & 0xffffu));
        v[2 * j + 1] = h2f((uint16_t)(raw[k][j] >> 16));
      }
      if constexpr (Q8) {
        if (clamp)
          st_stream8(qr_ + 8 * c, quant_pack4_i8<true>(v, m, rg.lo, rg.hi),
                     quant_pack4_i8<true>(v + 4, m, rg.lo, rg.hi));
        else
          st_stream8(qr_ + 8 * c, quant_pack4_i8<false>(v, m, rg.lo, rg.hi),
                     quant_pack4_i8<false>(v + 4, m, rg.lo, rg.hi));
      } else {
        st_stream((uint32_t*)(qr_ + 4 * c),
                  clamp ? quant_pack8<true>(v, m) : quant_pack8<false>(v, m));
      }
    }
  }
  if (lane == 0) {
    scale[row] = sh;
    if (rdbg) rdbg[row] = r;
  }
}

// ===========================================================================
// k_heads_quant: y = (H_NH (x) I_DH) x / sqrt(NH), then the quantizer.
// A lane holds J consecutive positions j of every head (NH * J = 128 values
// for NH >= 16), so all log2(NH) butterfly stages are between its own
// registers; LPR = DH / J lanes cover a row and a wavefront takes 64 / LPR
// rows.  Loads are J fp16 per head, stores J/2 bytes of packed codes per
// head (J bytes of b-bit codes).
// ===========================================================================
template <int J>
struct HeadsIO;
template <>
struct HeadsIO<2> {
  typedef uint32_t raw_t;
  static __device__ __forceinline__ raw_t load(const uint16_t* p) {
    return __builtin_nontemporal_load((const uint32_t*)p);
  }
  static __device__ __forceinline__ uint32_t word(const raw_t& r, int i) { return r; }
};
template <>
struct HeadsIO<4> {
  typedef uint32_t raw_t __attribute__((ext_vector_type(2)));
  static __device__ __forceinline__ raw_t load(const uint16_t* p) {
    return __builtin_nontemporal_load((const raw_t*)p);
  }
  static __device__ __forceinline__ uint32_t word(const raw_t& r, int i) { return r[i]; }
};
template <>
struct HeadsIO<8> {
  typedef v4u raw_t;
  static __device__ __forceinline__ raw_t load(const uint16_t* p) { return ld_stream(p); }
  static __device__ __forceinline__ uint32_t word(const raw_t& r, int i) { return r[i]; }
};

// J fp32 values times m -> J/2 bytes of two's-complement nibble pairs, in the
// low bytes of the result (same rounding as quant_pack8).
template <int J, bool CLAMP>
__device__ __forceinline__ uint32_t quant_packJ(const float* v, float m) {
  if constexpr (J == 8) {
    return quant_pack8<CLAMP>(v, m);
  } else {
    uint32_t f[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      float t = fmaf(v[j], m, kMagic + 8.0f);
      if (CLAMP) t = __builtin_amdgcn_fmed3f(t, kMagic, kMagic + 15.0f);
      f[j] = __float_as_uint(t);
    }
    const uint32_t p0 = (f[1] << 4) | f[0];
    if constexpr (J == 2) {
      return (p0 & 0xffu) ^ 0x88u;
    } else {
      const uint32_t p1 = (f[3] << 4) | f[2];
      return __builtin_amdgcn_perm(p1, p0, 0x0c0c0400u) ^ 0x8888u;
    }
  }
}

template <int NH, int J, int LPR, bool Q8>
__global__ __launch_bounds__(256) void k_heads_quant(const uint16_t* __restrict__ x, int64_t T,
                                                     int64_t ld, float c, float clip, int bits,
                                                     uint8_t* __restrict__ q,
                                                     uint16_t* __restrict__ scale,
                                                     float* __restrict__ zdbg) {
  constexpr int RPW = 64 / LPR;  // rows per wavefront
  constexpr int DH = J * LPR;    // head dimension
  constexpr int D = NH * DH;
  typedef HeadsIO<J> IO;
  const int lane = threadIdx.x & 63;
  const int sub = lane % LPR, rw = lane / LPR;
  const int64_t row0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW;
  if (row0 >= T) return;  // wave-uniform
  const int64_t row = row0 + rw;
  const bool valid = row < T;
  const int j0 = sub * J;
  const uint16_t* xr = x + (valid ? row : row0) * ld + j0;

  typename IO::raw_t raw[NH];
#pragma unroll
  for (int h = 0; h < NH; ++h) raw[h] = IO::load(xr + h * DH);
  float v[NH][J];
#pragma unroll
  for (int h = 0; h < NH; ++h)
#pragma unroll
    for (int i = 0; i < J / 2; ++i) {
      const uint32_t w = IO::word(raw[h], i);
      v[h][2 * i] = h2f((uint16_t)(w & 0xffffu));
      v[h][2 * i + 1] = h2f((uint16_t)(w >> 16));
    }
  // H_NH over the head index: Sylvester butterflies, natural order
#pragma unroll
  for (int s = 1; s < NH; s <<= 1)
#pragma unroll
    for (int h = 0; h < NH; ++h)
      if (!(h & s))
#pragma unroll
        for (int j = 0; j < J; ++j) {
          const float a = v[h][j], b = v[h + s][j];
          v[h][j] = a + b;
          v[h + s][j] = a - b;
        }
  if (zdbg && valid) {
    float* zr = zdbg + row * D + j0;
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int j = 0; j < J; ++j) zr[h * DH + j] = v[h][j];
  }
  float am = 0.0f;
#pragma unroll
  for (int h = 0; h < NH; ++h)
#pragma unroll
    for (int j = 0; j < J; ++j) am = fmaxf(am, fabsf(v[h][j]));
#pragma unroll
  for (int o = 1; o < LPR; o <<= 1) am = fmaxf(am, __shfl_xor(am, o));
  const QRange rg = q_range(Q8 ? bits : 4);
  uint16_t sh;
  float m;
  sym_scale(am, c, clip, &sh, &m, rg.qmax);
  if (!valid) return;
  const bool clamp = clip < 1.0f || (sh & 0x7fffu) < 0x0400u;
  if constexpr (Q8) {
    // J codes of one byte each per head
    uint8_t* q8 = q + row * D + j0;
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      uint8_t* dst = q8 + h * DH;
      if constexpr (J == 2) {
        const uint32_t p = clamp ? quant_pack2_i8<true>(v[h], m, rg.lo, rg.hi)
                                 : quant_pack2_i8<false>(v[h], m, rg.lo, rg.hi);
        __builtin_nontemporal_store((uint16_t)p, (uint16_t*)dst);
      } else if constexpr (J == 4) {
        const uint32_t p = clamp ? quant_pack4_i8<true>(v[h], m, rg.lo, rg.hi)
                                 : quant_pack4_i8<false>(v[h], m, rg.lo, rg.hi);
        st_stream((uint32_t*)dst, p);
      } else {
        if (clamp)
          st_stream8(dst, quant_pack4_i8<true>(v[h], m, rg.lo, rg.hi),
                     quant_pack4_i8<true>(v[h] + 4, m, rg.lo, rg.hi));
        else
          st_stream8(dst, quant_pack4_i8<false>(v[h], m, rg.lo, rg.hi),
                     quant_pack4_i8<false>(v[h] + 4, m, rg.lo, rg.hi));
      }
    }
    if (sub == 0) scale[row] = sh;
    return;
  }
  uint8_t* qr_ = q + row * (D / 2) + j0 / 2;
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    const uint32_t p = clamp ? quant_packJ<J, true>(v[h], m) : quant_packJ<J, false>(v[h], m);
    uint8_t* dst = qr_ + h * (DH / 2);
    if constexpr (J == 2) {
      __builtin_nontemporal_store((uint8_t)p, dst);
    } else if constexpr (J == 4) {
      __builtin_nontemporal_store((uint16_t)p, (uint16_t*)dst);
    } else {
      st_stream((uint32_t*)dst, p);
    }
  }
  if (sub == 0) scale[row] = sh;
}

static int blocks_for(int64_t rows, int rows_per_block) {
  return (int)((rows + rows_per_block - 1) / rows_per_block);
}

template <bool Q8>
static qr_status launch_rms(const uint16_t* x, int64_t T, int d, int64_t ld, float eps, float clip,
                            int bits, uint8_t* q, uint16_t* sc, float* r, hipStream_t st) {
  const int per_lane = (d / 8 + 63) / 64;
  const int grid = blocks_for(T, 4);
#define QR_RMS(N)                                                                              \
  hipLaunchKernelGGL((k_rms_quant<N, Q8>), dim3(grid), dim3(256), 0, st, x, T, d, ld, eps, clip, \
                     bits, q, sc, r)
  if (per_lane <= 1) QR_RMS(1);
  else if (per_lane <= 2) QR_RMS(2);
  else if (per_lane <= 4) QR_RMS(4);
  else if (per_lane <= 8) QR_RMS(8);
  else if (per_lane <= 16) QR_RMS(16);
  else if (per_lane <= 32) QR_RMS(32);
  else return QR_ERR_UNSUPPORTED;
#undef QR_RMS
  return launch_status();
}

// values per lane J = min(8, 128 / NH); lanes per row = head_dim / J
static int heads_j(int nh) { return nh >= 16 ? 128 / nh : 8; }

template <int NH, bool Q8>
static qr_status launch_heads_nh(int dh, const uint16_t* x, int64_t T, int64_t ld, float c,
                                 float clip, int bits, uint8_t* q, uint16_t* sc, float* z,
                                 hipStream_t st) {
  constexpr int J = NH >= 16 ? 128 / NH : 8;
  const int lpr = dh / J;
  const int grid = blocks_for(T, 4 * (64 / lpr));
  switch (lpr) {
#define QR_CASE(L)                                                                             \
  case L:                                                                                      \
    hipLaunchKernelGGL((k_heads_quant<NH, J, L, Q8>), dim3(grid), dim3(256), 0, st, x, T, ld, c, \
                       clip, bits, q, sc, z);                                                  \
    break;
    QR_CASE(4)
    QR_CASE(8)
    QR_CASE(16)
    QR_CASE(32)
    QR_CASE(64)
#undef QR_CASE
    default:
      return QR_ERR_UNSUPPORTED;
  }
  return launch_status();
}

static qr_status rmsnorm_entry(const void* x_f16, int64_t T, int32_t d, int64_t ld_x, float eps,
                               float clip_ratio, int bits, bool q8, void* q, void* scale_f16,
                               float* r_dbg, hipStream_t stream) {
  if (T < 0 || d <= 0 || ld_x < d) return QR_ERR_SHAPE;
  if (!valid_clip(clip_ratio) || !(eps >= 0.0f) || !(eps <= 1.0f)) return QR_ERR_ARG;
  if (q8 && (bits < 2 || bits > 8)) return QR_ERR_ARG;
  if (d % 8 != 0 || d > 16384) return QR_ERR_UNSUPPORTED;
  if (T == 0) return QR_OK;
  if (!x_f16 || !q || !scale_f16) return QR_ERR_NULL;
  if (ld_x % 8 != 0 || !aligned(x_f16, 16) || !aligned(q, q8 ? 8 : 4) || !aligned(scale_f16, 2) ||
      (r_dbg && !aligned(r_dbg, 4)))
    return QR_ERR_ALIGN;
  const uint16_t* x = (const uint16_t*)x_f16;
  return q8 ? launch_rms<true>(x, T, d, ld_x, eps, clip_ratio, bits, (uint8_t*)q,
                               (uint16_t*)scale_f16, r_dbg, stream)
            : launch_rms<false>(x, T, d, ld_x, eps, clip_ratio, 4, (uint8_t*)q,
                                (uint16_t*)scale_f16, r_dbg, stream);
}

template <bool Q8>
static qr_status heads_dispatch(int n_heads, int head_dim, const uint16_t* x, int64_t T, int64_t ld,
                                float c, float clip, int bits, uint8_t* q, uint16_t* sc, float* z,
                                hipStream_t st) {
  switch (n_heads) {
    case 2: return launch_heads_nh<2, Q8>(head_dim, x, T, ld, c, clip, bits, q, sc, z, st);
    case 4: return launch_heads_nh<4, Q8>(head_dim, x, T, ld, c, clip, bits, q, sc, z, st);
    case 8: return launch_heads_nh<8, Q8>(head_dim, x, T, ld, c, clip, bits, q, sc, z, st);
    case 16: return launch_heads_nh<16, Q8>(head_dim, x, T, ld, c, clip, bits, q, sc, z, st);
    case 32: return launch_heads_nh<32, Q8>(head_dim, x, T, ld, c, clip, bits, q, sc, z, st);
    default: return launch_heads_nh<64, Q8>(head_dim, x, T, ld, c, clip, bits, q, sc, z, st);
  }
}

static qr_status heads_entry(const void* x_f16, int64_t T, int32_t n_heads, int32_t head_dim,
                             int64_t ld_x, float clip_ratio, int bits, bool q8, void* q,
                             void* scale_f16, float* z_dbg, hipStream_t stream) {
  if (T < 0 || n_heads <= 0 || head_dim <= 0) return QR_ERR_SHAPE;
  const int64_t d = (int64_t)n_heads * head_dim;
  if (ld_x < d) return QR_ERR_SHAPE;
  if (!valid_clip(clip_ratio)) return QR_ERR_ARG;
  if (q8 && (bits < 2 || bits > 8)) return QR_ERR_ARG;
  const bool pow2 = !(n_heads & (n_heads - 1)) && !(head_dim & (head_dim - 1));
  if (!pow2 || n_heads < 2 || n_heads > 64) return QR_ERR_UNSUPPORTED;
  const int J = heads_j(n_heads);
  if (head_dim < 4 * J || head_dim > 64 * J) return QR_ERR_UNSUPPORTED;
  if (T == 0) return QR_OK;
  if (!x_f16 || !q || !scale_f16) return QR_ERR_NULL;
  if (ld_x % 8 != 0 || !aligned(x_f16, 16) || !aligned(q, q8 ? 8 : 4) || !aligned(scale_f16, 2) ||
      (z_dbg && !aligned(z_dbg, 16)))
    return QR_ERR_ALIGN;
  const float c = norm_constant(n_heads);
  const uint16_t* x = (const uint16_t*)x_f16;
  return q8 ? heads_dispatch<true>(n_heads, head_dim, x, T, ld_x, c, clip_ratio, bits,
                                   (uint8_t*)q, (uint16_t*)scale_f16, z_dbg, stream)
            : heads_dispatch<false>(n_heads, head_dim, x, T, ld_x, c, clip_ratio, 4, (uint8_t*)q,
                                    (uint16_t*)scale_f16, z_dbg, stream);
}

}  // namespace qr

using namespace qr;

extern "C" qr_status qr_rmsnorm_quant(const void* x_f16, int64_t T, int32_t d, int64_t ld_x,
                                      float eps, float clip_ratio, void* q_u8, void* scale_f16,
                                      float* r_dbg, hipStream_t stream) {
  return rmsnorm_entry(x_f16, T, d, ld_x, eps, clip_ratio, 4, false, q_u8, scale_f16, r_dbg,
                       stream);
}

extern "C" qr_status qr_rmsnorm_quant_i8(const void* x_f16, int64_t T, int32_t d, int64_t ld_x,
                                         float eps, float clip_ratio, int32_t bits, void* q_i8,
                                         void* scale_f16, float* r_dbg, hipStream_t stream) {
  return rmsnorm_entry(x_f16, T, d, ld_x, eps, clip_ratio, bits, true, q_i8, scale_f16, r_dbg,
                       stream);
}

extern "C" qr_status qr_hadamard_heads_quant(const void* x_f16, int64_t T, int32_t n_heads,
                                             int32_t head_dim, int64_t ld_x, float clip_ratio,
                                             void* q_u8, void* scale_f16, float* z_dbg,
                                             hipStream_t stream) {
  return heads_entry(x_f16, T, n_heads, head_dim, ld_x, clip_ratio, 4, false, q_u8, scale_f16,
                     z_dbg, stream);
}

extern "C" qr_status qr_hadamard_heads_quant_i8(const void* x_f16, int64_t T, int32_t n_heads,
                                                int32_t head_dim, int64_t ld_x, float clip_ratio,
                                                int32_t bits, void* q_i8, void* scale_f16,
                                                float* z_dbg, hipStream_t stream) {
  return heads_entry(x_f16, T, n_heads, head_dim, ld_x, clip_ratio, bits, true, q_i8, scale_f16,
                     z_dbg, stream);
}
