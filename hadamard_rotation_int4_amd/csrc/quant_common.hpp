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
// bits and the multiplier m = c * (1 / s_h) (0 if s_h == 0).
__device__ __forceinline__ void sym_scale(float amax_z, float c, float clip, uint16_t* sh_out,
                                          float* m_out) {
  const float a = __fmul_rn(amax_z, c);
  const float s = __fdiv_rn(__fmul_rn(clip, a), 7.0f);
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

// Streaming accesses: every input row is read once and every output written
// once, so both bypass cache retention (non-temporal).
#ifndef QR_NT
#define QR_NT 1
#endif
__device__ __forceinline__ v4u ld_stream(const uint16_t* p) {
  return QR_NT ? __builtin_nontemporal_load((const v4u*)p) : *(const v4u*)p;
}
__device__ __forceinline__ void st_stream(uint32_t* p, uint32_t v) {
  if (QR_NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

}  // namespace qr
