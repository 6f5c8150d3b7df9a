// Per-row symmetric INT4 quantizer pieces shared by the fused kernels of
// libquarot_hip.so (QuaRot paper, activation-quantization paragraph: scale =
// max|y| / 7, round to nearest, two codes per byte), and streaming accesses.
// The exact fp32 recipe is stated in include/qr.h.
#pragma once

#include "common.hpp"

namespace qr {

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Per-row scale recipe (identical for every kernel): returns the fp16 scale
// bits and the multiplier m = c * (1 / s_h) (0 if s_h == 0).  qmax is the
// largest code: 7 for INT4, 2^(b-1) - 1 for b-bit codes.
__device__ __forceinline__ void sym_scale(float amax_z, float c, float clip, uint16_t* sh_out,
                                          float* m_out, float qmax = 7.0f) {
  const float a = __fmul_rn(amax_z, c);
  const float s = __fdiv_rn(__fmul_rn(clip, a), qmax);
  const uint16_t sh = f2h(s);
  const float shf = h2f(sh);
  const float inv = shf > 0.0f ? __fdiv_rn(1.0f, shf) : 0.0f;
  *sh_out = sh;
  *m_out = __fmul_rn(c, inv);
}

// Eight fp32 values times m -> eight offset-binary nibbles (q + 8), packed
// into one little-endian dword and converted to two's complement.
template <bool CLAMP>
__device__ __forceinline__ uint32_t quant_pack8(const float* v, float m) {
  uint32_t f[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float t = fmaf(v[j], m, kMagic + 8.0f);  // kMagic + 8 + rne(v*m)
    if (CLAMP) t = __builtin_amdgcn_fmed3f(t, kMagic, kMagic + 15.0f);
    f[j] = __float_as_uint(t);
  }
  // low byte of each pair word: (q_odd + 8) << 4 | (q_even + 8)
  const uint32_t p0 = (f[1] << 4) | f[0];
  const uint32_t p1 = (f[3] << 4) | f[2];
  const uint32_t p2 = (f[5] << 4) | f[4];
  const uint32_t p3 = (f[7] << 4) | f[6];
  const uint32_t lo = __builtin_amdgcn_perm(p1, p0, 0x0c0c0400u);  // [p0.b0, p1.b0, 0, 0]
  const uint32_t hi = __builtin_amdgcn_perm(p3, p2, 0x04000c0cu);  // [0, 0, p2.b0, p3.b0]
  return lo ^ hi ^ 0x88888888u;  // offset binary -> two's complement nibbles
}

// b-bit codes stored one per byte (b <= 8; QuaRot paper, 6- and 8-bit RTN):
// fma(v, m, kMagic) = kMagic + rne(v m), whose low byte is the two's-complement
// code; the clamp to [lo, hi] = [-2^(b-1), 2^(b-1) - 1] is a med3 on the same
// biased values.  Four codes per dword, code j in byte j.
template <bool CLAMP>
__device__ __forceinline__ uint32_t q8_word(float v, float m, float lo, float hi) {
  float t = fmaf(v, m, kMagic);
  if (CLAMP) t = __builtin_amdgcn_fmed3f(t, kMagic + lo, kMagic + hi);
  return __float_as_uint(t);
}
template <bool CLAMP>
__device__ __forceinline__ uint32_t quant_pack4_i8(const float* v, float m, float lo, float hi) {
  const uint32_t f0 = q8_word<CLAMP>(v[0], m, lo, hi), f1 = q8_word<CLAMP>(v[1], m, lo, hi);
  const uint32_t f2 = q8_word<CLAMP>(v[2], m, lo, hi), f3 = q8_word<CLAMP>(v[3], m, lo, hi);
  return __builtin_amdgcn_perm(f1, f0, 0x0c0c0400u) | __builtin_amdgcn_perm(f3, f2, 0x04000c0cu);
}
template <bool CLAMP>
__device__ __forceinline__ uint32_t quant_pack2_i8(const float* v, float m, float lo, float hi) {
  const uint32_t f0 = q8_word<CLAMP>(v[0], m, lo, hi), f1 = q8_word<CLAMP>(v[1], m, lo, hi);
  return __builtin_amdgcn_perm(f1, f0, 0x0c0c0400u);
}
// Code range of b-bit symmetric codes as the floats the packers take.
struct QRange {
  float qmax, lo, hi;
};
__host__ __device__ inline QRange q_range(int bits) {
  const int h = 1 << (bits - 1);
  return QRange{(float)(h - 1), (float)(-h), (float)(h - 1)};
}

// Streaming accesses: every input row is read once and every output written
// once, so both bypass cache retention (non-temporal).
__device__ __forceinline__ v4u ld_stream(const uint16_t* p) {
  return __builtin_nontemporal_load((const v4u*)p);
}
__device__ __forceinline__ void st_stream(uint32_t* p, uint32_t v) {
  __builtin_nontemporal_store(v, p);
}
typedef uint32_t v2u __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void st_stream8(void* p, uint32_t lo, uint32_t hi) {
  const v2u v = {lo, hi};
  __builtin_nontemporal_store(v, (v2u*)p);
}

}  // namespace qr
