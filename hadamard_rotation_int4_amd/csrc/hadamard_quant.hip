// Online randomized Hadamard rotation fused with per-token symmetric INT4
// quantization and nibble packing (qr_hadamard_quant), and the rotation alone
// (qr_hadamard), for gfx950.
//
// What is computed (QuaRot paper, background on Hadamard matrices and the
// activation-quantization paragraph): z = H_d (s * x) with H_d = H_{2^n} (x) H_m,
// y = z / sqrt(d), scale = fp16(clip * max|y| / 7), q = clamp(rne(y / scale), -8, 7),
// two codes per byte.  The exact fp32 recipe is stated in include/qr.h.
//
// Kernel families:
//  * k_hq_pow2   d = 512 .. 8192 (powers of two), one wavefront per row, no LDS
//                traffic for data.  H_d = H_{d/(32K)} (x) H_K (x) H_32, K = min(4,
//                d/512): the H_K (x) H_32 factor runs on the matrix cores
//                (v_mfma_f32_16x16x32_f16, K chained products per output tile,
//                the H_K signs carried by negated A fragments) directly on the
//                fp16 input with the signs applied by flipping sign bits, which is
//                exact (the products are +-x and the accumulation is fp32).  The
//                remaining stages run in fp32 VALU: 4 across lanes through DPP
//                (one v_fmac_f32_dpp per element and stage, with a per-lane +-1
//                multiplier) and the rest between registers of a lane.  amax,
//                scale, rounding and packing follow in registers; the row makes
//                exactly one HBM round trip, and the next row's loads are in
//                flight while the current row is transformed.
//  * k_hq_small  d = 8 .. 256 (and the head-wise K/V path): d/8 lanes per row,
//                three in-register stages and the rest through lane shuffles.
//  * k_hq_k28    d = 1024 * 28: H_4 (x) H_28 on the matrix cores, H_256 in
//                registers, DPP and one LDS exchange across the workgroup.
//  * k_hq_k172   d = 64 * 172: H_172 on the matrix cores, H_64 in DPP/registers.
//  * k_hq_lds    other d = 2^n * m, m in {28, 172}, and quantization without
//                rotation: one workgroup per row, the row staged in LDS as fp32,
//                the dense +-1 H_m products on contiguous m-chunks followed by
//                radix-32 butterfly passes in LDS.
// MODE_QUANT8 (qr_hadamard_quant_i8: b-bit codes one per byte, QuaRot paper's
// 6- and 8-bit round-to-nearest results) is implemented by k_hq_k28, k_hq_k172
// and k_hq_lds, which then also serves d = 2^n.
#include <type_traits>

#include "common.hpp"
#include "dpp.hpp"
#include "quant_common.hpp"

namespace qr {

__constant__ HTable<28> g_h28 = make_h28();
__constant__ HTable<172> g_h172 = make_h172();

// MODE_QUANT8: b-bit codes stored one per byte.  MODE_QUANT_GROUPS: packed
// INT4 codes with one scale per group of consecutive elements (k_hq_lds only).
enum { MODE_QUANT = 0, MODE_ROT_F32 = 1, MODE_ROT_F16 = 2, MODE_QUANT8 = 3, MODE_QUANT_GROUPS = 4 };

// Sign-bit masks of 8 consecutive fp16 values from their 8 int8 signs (+1 or
// -1; the int8 sign bit decides): dword j gets bit 15 if sign 2j is negative
// and bit 31 if sign 2j + 1 is.  Two dword loads; `s` is 4-byte aligned.
__device__ __forceinline__ v4u sign_masks8(const int8_t* s, bool second_half = true) {
  const uint32_t w0 = *(const uint32_t*)s;
  const uint32_t w1 = second_half ? *(const uint32_t*)(s + 4) : 0u;
  v4u m;
  m[0] = ((w0 << 8) & 0x8000u) | ((w0 << 16) & 0x80000000u);
  m[1] = ((w0 >> 8) & 0x8000u) | (w0 & 0x80000000u);
  m[2] = ((w1 << 8) & 0x8000u) | ((w1 << 16) & 0x80000000u);
  m[3] = ((w1 >> 8) & 0x8000u) | (w1 & 0x80000000u);
  return m;
}
// The same eight signs as one word: bit 15 - j / 31 - j for elements 2j / 2j + 1,
// so that (E << j) & 0x80008000 is the mask of dword j.
__device__ __forceinline__ uint32_t sign_word8(const int8_t* s, bool second_half = true) {
  const v4u m = sign_masks8(s, second_half);
  return m[0] | (m[1] >> 1) | (m[2] >> 2) | (m[3] >> 3);
}

// ===========================================================================
// k_hq_pow2: d = NB * 512
// ===========================================================================


// Launch shapes and pipeline depths of the rotate+quant kernels (each the
// fastest of the values measured at the Llama-2 shapes):
//  * k_hq_pow2 holds a row in 128 + 64 VGPRs: two wavefronts per SIMD;
//  * POW2_KM blocks are combined on the matrix cores (H_4 (x) H_32); 8 moves
//    one more butterfly stage onto them but was slower at d = 8192;
//  * POW2_PF_EARLY of the 16 blocks of the next 8192-wide row are fetched
//    right after the MFMAs, the rest during quantization (4 or 16: slower);
//  * k_hq_small works on one group of rows per wavefront at a time.
constexpr int POW2_WAVES_PER_SIMD = 2;
constexpr int POW2_KM = 4;
constexpr int POW2_PF_EARLY = 8;
constexpr int SMALL_UNROLL = 1;
constexpr int K28_WAVES_PER_SIMD = 2;

// Buffer-resource cache policy of the streaming accesses (gfx9 "nt" bit).
constexpr int BUF_POLICY_NT = 2;

template <int NB, int MODE, bool CLAMP, bool DBG>
__global__ __launch_bounds__(256, POW2_WAVES_PER_SIMD) void k_hq_pow2(const uint16_t* __restrict__ x, int64_t T,
                                                 int64_t ld, const int8_t* __restrict__ signs,
                                                 float c, float clip, uint8_t* __restrict__ q,
                                                 uint16_t* __restrict__ scale,
                                                 float* __restrict__ zdbg,
                                                 void* __restrict__ yout) {
  constexpr int D = NB * 512;
  // Blocks of the next row fetched right after the MFMAs; the others are
  // fetched during quantization, as the registers of the current row free up
  // (quantization-only kernels: there is no later point, all are early).
  constexpr int PF_EARLY = (MODE == MODE_QUANT && NB == 16) ? POW2_PF_EARLY : NB;
  // Blocks combined on the matrix cores (the rest by butterflies in the lane).
  constexpr int KM = NB < POW2_KM ? NB : POW2_KM;
  __shared__ v4u s_mask[NB * 64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int cl = lane & 15, g = lane >> 4;
  const int gc = gmap(cl);
  const int lane_off = gc * 32 + g * 8;  // first of the lane's 8 elements in a 512-block

  // Sign-bit masks for the lane's 8 fp16 values of every block (same for all rows).
  for (int i = tid; i < NB * 64; i += 256) {
    const int b = i >> 6, ln = i & 63;
    const int e = b * 512 + gmap(ln & 15) * 32 + (ln >> 4) * 8;
    s_mask[i] = signs ? sign_masks8(signs + e) : v4u{0u, 0u, 0u, 0u};
  }
  __syncthreads();

  // A operands: rows of H_32 permuted so that MFMA m, row i produces output
  // element o = 8 (i >> 2) + 4 m + (i & 3) of the chunk; with the 16x16 output
  // layout (lane = n + 16 (i >> 2), register i & 3) each lane then holds the
  // 8 consecutive outputs at the same offsets it loaded.
  v8h a0, a1;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int k = 8 * g + j;
    const int o0 = 8 * (cl >> 2) + (cl & 3);
    const int o1 = o0 + 4;
    a0[j] = (__builtin_popcount(o0 & k) & 1) ? (_Float16)-1.0f : (_Float16)1.0f;
    a1[j] = (__builtin_popcount(o1 & k) & 1) ? (_Float16)-1.0f : (_Float16)1.0f;
  }
  const v8h a0n = -a0, a1n = -a1;
  // DPP stage multipliers: +1 on the lane holding the lower chunk of the pair.
  const float s0 = (gc & 1) ? -1.0f : 1.0f;
  const float s1 = (gc & 2) ? -1.0f : 1.0f;
  const float s2 = (gc & 4) ? -1.0f : 1.0f;
  const float s3 = (gc & 8) ? -1.0f : 1.0f;
  // After the four DPP stages the lane holds sigma * z.
  const float sigma = (__builtin_popcount(gc) & 1) ? -1.0f : 1.0f;

  // Rows are addressed through one buffer resource per row (a wave-uniform
  // base in scalar registers) plus the lane's fixed byte offset, so no 64-bit
  // per-lane pointers stay live.  Block b of a row sits at scalar offset
  // 1024 b.  A resource with zero records returns zeros without a fetch.
  const int voff = lane_off * 2;
  auto row_rsrc = [&](int64_t r, bool valid) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)(x + r * ld), 0, valid ? D * 2 : 0, 0x00020000);
  };

  // The next row's input is fetched into the same registers block by block as
  // soon as the MFMAs have consumed the current one, so its latency overlaps
  // this row's butterflies and quantization.
  const int64_t rstride = (int64_t)gridDim.x * 4;
  int64_t row = (int64_t)blockIdx.x * 4 + wave;
  v4u raw[NB];
  {
    const __amdgpu_buffer_rsrc_t rs = row_rsrc(row < T ? row : 0, row < T);
#pragma unroll
    for (int b = 0; b < NB; ++b)
      raw[b] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, b * 1024, BUF_POLICY_NT));
  }
  for (; row < T; row += rstride) {
    const bool more = row + rstride < T;
    const __amdgpu_buffer_rsrc_t rsn = row_rsrc(more ? row + rstride : row, more);
    // Matrix-core stage over element bits 0..4 and the low log2(KM) block
    // bits: H_KM (x) H_32 as KM chained MFMAs per output tile, the H_KM signs
    // carried by the negated A fragments.
    float w[NB][8];
#pragma unroll
    for (int grp = 0; grp < NB / KM; ++grp) {
      v8h bop[KM];
#pragma unroll
      for (int kb = 0; kb < KM; ++kb) {
        const int b = grp * KM + kb;
        bop[kb] = __builtin_bit_cast(v8h, raw[b] ^ s_mask[b * 64 + lane]);
        if (b < PF_EARLY)
          raw[b] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(rsn, voff, b * 1024, BUF_POLICY_NT));
      }
#pragma unroll
      for (int h = 0; h < KM; ++h) {
        v4f r0 = {0.0f, 0.0f, 0.0f, 0.0f}, r1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kb = 0; kb < KM; ++kb) {
          const bool neg = __builtin_popcount(h & kb) & 1;
          r0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(neg ? a0n : a0, bop[kb], r0, 0, 0, 0);
          r1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(neg ? a1n : a1, bop[kb], r1, 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          w[grp * KM + h][j] = r0[j];
          w[grp * KM + h][4 + j] = r1[j];
        }
      }
    }
    // Butterflies over the remaining block bits, inside the lane.
#pragma unroll
    for (int h = KM; h < NB; h <<= 1)
#pragma unroll
      for (int b = 0; b < NB; ++b)
        if (!(b & h))
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float u = w[b][j], v = w[b + h][j];
            w[b][j] = u + v;
            w[b + h][j] = u - v;
          }
    if (NB == KM) {
      // No register butterfly ran, so the DPP asm below would read MFMA results
      // directly, and the compiler inserts no MFMA-to-VALU wait states in front
      // of inline asm: pass every result through a compiler-visible VALU op.
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int j = 0; j < 8; ++j) w[b][j] = __fadd_rn(w[b][j], 0.0f);
    }
    // Butterflies over the chunk index (element bits 5..8), across lanes.
#pragma unroll
    for (int b = 0; b < NB; ++b) QR_DPP8("quad_perm:[1,0,3,2]", w[b], s0);
#pragma unroll
    for (int b = 0; b < NB; ++b) QR_DPP8("quad_perm:[2,3,0,1]", w[b], s1);
#pragma unroll
    for (int b = 0; b < NB; ++b) QR_DPP8("row_half_mirror", w[b], s2);
#pragma unroll
    for (int b = 0; b < NB; ++b) QR_DPP8("row_mirror", w[b], s3);

    if constexpr (DBG) {
      float* zr = zdbg + row * D + lane_off;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        v4f lo = {w[b][0] * sigma, w[b][1] * sigma, w[b][2] * sigma, w[b][3] * sigma};
        v4f hi = {w[b][4] * sigma, w[b][5] * sigma, w[b][6] * sigma, w[b][7] * sigma};
        *(v4f*)(zr + b * 512) = lo;
        *(v4f*)(zr + b * 512 + 4) = hi;
      }
    }

    if constexpr (MODE == MODE_QUANT) {
      float am = 0.0f;
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int j = 0; j < 8; ++j) am = fmaxf(am, fabsf(w[b][j]));
      am = wave_max(am);
      uint16_t sh;
      float m;
      sym_scale(am, c, clip, &sh, &m);
      sh = (uint16_t)__builtin_amdgcn_readfirstlane(sh);  // the same on every lane
      const float ml = m * sigma;  // w * ml = z * m exactly
      const __amdgpu_buffer_rsrc_t rsq =
          __builtin_amdgcn_make_buffer_rsrc((void*)(q + row * (D / 2)), 0, D / 2, 0x00020000);
      const int qoff = lane_off / 2;
      // Without clipping |z m| <= 7 (1 + 2^-10) < 7.5 whenever s_h is a normal
      // fp16, so the clamp can be skipped; a subnormal s_h carries a larger
      // relative rounding error and takes the clamped path (wave-uniform branch).
      // The blocks not fetched early are fetched as their registers free up.
      if (CLAMP || (sh & 0x7fffu) < 0x0400u) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          __builtin_amdgcn_raw_buffer_store_b32(quant_pack8<true>(w[b], ml), rsq, qoff, b * 256, BUF_POLICY_NT);
          if (b >= PF_EARLY)
            raw[b] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(rsn, voff, b * 1024, BUF_POLICY_NT));
        }
      } else {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          __builtin_amdgcn_raw_buffer_store_b32(quant_pack8<false>(w[b], ml), rsq, qoff, b * 256, BUF_POLICY_NT);
          if (b >= PF_EARLY)
            raw[b] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(rsn, voff, b * 1024, BUF_POLICY_NT));
        }
      }
      if (lane == 0) scale[row] = sh;
    } else {
      const float cs = c * sigma;
      if (MODE == MODE_ROT_F32) {
        float* yr = (float*)yout + row * D + lane_off;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          v4f lo = {__fmul_rn(w[b][0], cs), __fmul_rn(w[b][1], cs), __fmul_rn(w[b][2], cs),
                    __fmul_rn(w[b][3], cs)};
          v4f hi = {__fmul_rn(w[b][4], cs), __fmul_rn(w[b][5], cs), __fmul_rn(w[b][6], cs),
                    __fmul_rn(w[b][7], cs)};
          *(v4f*)(yr + b * 512) = lo;
          *(v4f*)(yr + b * 512 + 4) = hi;
        }
      } else {
        uint16_t* yr = (uint16_t*)yout + row * D + lane_off;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          v4u o;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            o[j] = (uint32_t)f2h(__fmul_rn(w[b][2 * j], cs)) |
                   ((uint32_t)f2h(__fmul_rn(w[b][2 * j + 1], cs)) << 16);
          *(v4u*)(yr + b * 512) = o;
        }
      }
    }
  }
}

// ===========================================================================
// k_hq_small: d = 8 .. 256 (powers of two), d/8 lanes per row
// ===========================================================================
template <int LPR, int MODE, bool CLAMP>
__global__ __launch_bounds__(256) void k_hq_small(const uint16_t* __restrict__ x, int64_t T,
                                                  int64_t ld, const int8_t* __restrict__ signs,
                                                  int rot, float c, float clip,
                                                  uint8_t* __restrict__ q,
                                                  uint16_t* __restrict__ scale,
                                                  float* __restrict__ zdbg,
                                                  void* __restrict__ yout) {
  constexpr int D = LPR * 8;
  constexpr int RPW = 64 / LPR;  // rows per wavefront
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int sub = lane % LPR;  // lane within the row
  const int rw = lane / LPR;   // row within the wavefront
  // With 16 lanes per row (one DPP row), the lane holds chunk gmap(sub) and
  // the cross-lane stages run through DPP as in k_hq_pow2; the lane then ends
  // with sigma * z.  Otherwise chunk sub and lane shuffles.
  constexpr bool DPP = LPR == 16;
  const int gc = DPP ? gmap(sub) : sub;
  const int coff = gc * 8;     // first element of the lane's chunk
  const float sigma = (DPP && (__builtin_popcount(gc) & 1)) ? -1.0f : 1.0f;
  float sg[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) sg[j] = 1.0f;
  if (rot && signs) {
    const uint32_t w0 = *(const uint32_t*)(signs + coff), w1 = *(const uint32_t*)(signs + coff + 4);
#pragma unroll
    for (int j = 0; j < 8; ++j) sg[j] = (((j < 4 ? w0 : w1) >> (8 * (j & 3) + 7)) & 1u) ? -1.0f : 1.0f;
  }

  // Grid-stride over groups of RPW rows per wavefront; SMALL_UNROLL groups
  // are loaded before any is processed, so that many loads are in flight.
  constexpr int U = SMALL_UNROLL;
  const int64_t gstride = (int64_t)gridDim.x * 4 * RPW;
  for (int64_t base0 = ((int64_t)blockIdx.x * 4 + wave) * RPW; base0 < T; base0 += U * gstride) {
  v4u raws[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t r = base0 + u * gstride + rw;
    raws[u] = r < T ? ld_stream(x + r * ld + coff) : v4u{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t row = base0 + u * gstride + rw;
    const bool valid = row < T;
    float v[8];
    {
      const v4u raw = raws[u];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[2 * j] = h2f((uint16_t)(raw[j] & 0xffffu)) * sg[2 * j];
        v[2 * j + 1] = h2f((uint16_t)(raw[j] >> 16)) * sg[2 * j + 1];
      }
    }
    if (rot) {
#pragma unroll
      for (int h = 1; h < 8; h <<= 1)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (!(j & h)) {
            const float a = v[j], b = v[j + h];
            v[j] = a + b;
            v[j + h] = a - b;
          }
      if constexpr (DPP) {
        const float s0 = (gc & 1) ? -1.0f : 1.0f, s1 = (gc & 2) ? -1.0f : 1.0f;
        const float s2 = (gc & 4) ? -1.0f : 1.0f, s3 = (gc & 8) ? -1.0f : 1.0f;
        QR_DPP8("quad_perm:[1,0,3,2]", v, s0);
        QR_DPP8("quad_perm:[2,3,0,1]", v, s1);
        QR_DPP8("row_half_mirror", v, s2);
        QR_DPP8("row_mirror", v, s3);
      } else {
#pragma unroll
        for (int h = 1; h < LPR; h <<= 1) {
          const float s = (sub & h) ? -1.0f : 1.0f;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float p = __shfl_xor(v[j], h);
            v[j] = fmaf(v[j], s, p);  // low lane: mine + partner; high lane: partner - mine
          }
        }
      }
    }
    if (valid && zdbg) {
      float* zr = zdbg + row * D + coff;
      *(v4f*)zr = v4f{v[0] * sigma, v[1] * sigma, v[2] * sigma, v[3] * sigma};
      *(v4f*)(zr + 4) = v4f{v[4] * sigma, v[5] * sigma, v[6] * sigma, v[7] * sigma};
    }
    if (MODE == MODE_QUANT) {
      float am = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) am = fmaxf(am, fabsf(v[j]));
#pragma unroll
      for (int h = 1; h < LPR; h <<= 1) am = fmaxf(am, __shfl_xor(am, h));
      uint16_t sh;
      float m;
      sym_scale(am, c, clip, &sh, &m);
      const float ml = m * sigma;  // v * ml = z * m exactly
      if (valid) {
        *(uint32_t*)(q + row * (D / 2) + coff / 2) = (CLAMP || (sh & 0x7fffu) < 0x0400u)
                                                         ? quant_pack8<true>(v, ml)
                                                         : quant_pack8<false>(v, ml);
        if (sub == 0) scale[row] = sh;
      }
    } else if (valid) {
      const float cs = c * sigma;
      if (MODE == MODE_ROT_F32) {
        float* yr = (float*)yout + row * D + coff;
        *(v4f*)yr = v4f{__fmul_rn(v[0], cs), __fmul_rn(v[1], cs), __fmul_rn(v[2], cs),
                        __fmul_rn(v[3], cs)};
        *(v4f*)(yr + 4) = v4f{__fmul_rn(v[4], cs), __fmul_rn(v[5], cs), __fmul_rn(v[6], cs),
                              __fmul_rn(v[7], cs)};
      } else {
        v4u o;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          o[j] = (uint32_t)f2h(__fmul_rn(v[2 * j], cs)) |
                 ((uint32_t)f2h(__fmul_rn(v[2 * j + 1], cs)) << 16);
        *(v4u*)((uint16_t*)yout + row * D + coff) = o;
      }
    }
  }
  }
}

// ===========================================================================
// k_hq_lds: d = 2^n * M (M in {28, 172}), or quantization without rotation
// ===========================================================================
__device__ __forceinline__ int pad(int e) { return e + (e >> 5); }

// R in-register butterfly stages on 2^R values at LDS stride `stride`.
template <int R, int M>
__device__ __forceinline__ void lds_pass(float* buf, int d, int b0, int tid) {
  constexpr int G = 1 << R;
  const int groups = d >> R;
  const int stride = M << b0;
  for (int gi = tid; gi < groups; gi += 256) {
    const int mi = gi % M;
    const int rest = gi / M;
    const int alow = rest & ((1 << b0) - 1);
    const int ahigh = rest >> b0;
    const int base = ((ahigh << (b0 + R)) | alow) * M + mi;
    float v[G];
#pragma unroll
    for (int j = 0; j < G; ++j) v[j] = buf[pad(base + j * stride)];
#pragma unroll
    for (int h = 1; h < G; h <<= 1)
#pragma unroll
      for (int j = 0; j < G; ++j)
        if (!(j & h)) {
          const float a = v[j], b = v[j + h];
          v[j] = a + b;
          v[j + h] = a - b;
        }
#pragma unroll
    for (int j = 0; j < G; ++j) buf[pad(base + j * stride)] = v[j];
  }
}

// Dense +-1 product of one MB-block of H_M with one MB-block of a chunk:
// acc[o] += H[ob*MB + o][ib*MB + k] * xin[k].  H comes from constant memory
// with wave-uniform indices (scalar loads).
template <int M, int MB>
__device__ __forceinline__ void hm_block(const float* __restrict__ H, int ob, int ib,
                                         const float* xin, float* acc) {
#pragma unroll
  for (int o = 0; o < MB; ++o) {
    const float* hr = H + (ob * MB + o) * M + ib * MB;
#pragma unroll
    for (int k = 0; k < MB; ++k) acc[o] = fmaf(hr[k], xin[k], acc[o]);
  }
}

template <int M, int MODE, bool CLAMP, bool ROT>
__global__ __launch_bounds__(256) void k_hq_lds(const uint16_t* __restrict__ x, int64_t T, int d,
                                                int n, int64_t ld,
                                                const int8_t* __restrict__ signs, float c,
                                                float clip, int bits, int group,
                                                uint8_t* __restrict__ q,
                                                uint16_t* __restrict__ scale,
                                                float* __restrict__ zdbg,
                                                void* __restrict__ yout) {
  extern __shared__ float smem[];
  constexpr int NOB = (M == 172) ? 4 : 1;  // output blocks per chunk
  constexpr int MB = M / NOB;
  constexpr bool DOUBLE = (M == 172);  // H_172 writes into a second buffer
  const int tid = threadIdx.x;
  const int plen = pad(d) + 1;
  float* buf0 = smem;
  float* buf1 = DOUBLE ? smem + plen : smem;
  float* red = smem + (DOUBLE ? 2 : 1) * plen;  // 8 floats of reduction scratch
  const float* H = (M == 28) ? &g_h28.v[0][0] : (M == 172 ? &g_h172.v[0][0] : nullptr);

  for (int64_t row = blockIdx.x; row < T; row += gridDim.x) {
    // 1. fp16 -> fp32 (signs applied) into LDS
    for (int i = tid * 8; i < d; i += 256 * 8) {
      const v4u raw = *(const v4u*)(x + row * ld + i);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float f = h2f((uint16_t)((raw[j >> 1] >> (16 * (j & 1))) & 0xffffu));
        if (ROT && signs && signs[i + j] < 0) f = -f;
        buf0[pad(i + j)] = f;
      }
    }
    __syncthreads();
    float* buf = buf0;
    if (ROT) {
      // 2. H_M on every contiguous M-chunk
      if (M > 1) {
        const int chunks = d / M;
        constexpr int CPR = 256 / NOB;  // chunks per round (all NOB blocks of a chunk together)
        const int ob = __builtin_amdgcn_readfirstlane(tid / CPR);
        for (int c0 = 0; c0 < chunks; c0 += CPR) {
          const int ch = c0 + tid % CPR;
          const bool active = ch < chunks;
          float acc[MB];
#pragma unroll
          for (int o = 0; o < MB; ++o) acc[o] = 0.0f;
          if (active) {
#pragma unroll
            for (int ib = 0; ib < NOB; ++ib) {
              float xin[MB];
#pragma unroll
              for (int k = 0; k < MB; ++k) xin[k] = buf0[pad(ch * M + ib * MB + k)];
              hm_block<M, MB>(H, ob, ib, xin, acc);
            }
          }
          if (!DOUBLE) __syncthreads();
          if (active) {
#pragma unroll
            for (int o = 0; o < MB; ++o) buf1[pad(ch * M + ob * MB + o)] = acc[o];
          }
          if (!DOUBLE) __syncthreads();
        }
        if (DOUBLE) __syncthreads();
        buf = buf1;
      }
      // 3. butterflies over the 2^n index (stride M), five stages per LDS pass
      for (int b0 = 0; b0 < n; b0 += 5) {
        const int r = min(5, n - b0);
        switch (r) {
          case 1: lds_pass<1, M>(buf, d, b0, tid); break;
          case 2: lds_pass<2, M>(buf, d, b0, tid); break;
          case 3: lds_pass<3, M>(buf, d, b0, tid); break;
          case 4: lds_pass<4, M>(buf, d, b0, tid); break;
          default: lds_pass<5, M>(buf, d, b0, tid); break;
        }
        __syncthreads();
      }
    }
    if (zdbg) {
      for (int i = tid; i < d; i += 256) zdbg[row * d + i] = buf[pad(i)];
    }
    if (MODE == MODE_QUANT_GROUPS) {
      // 4'. one scale per group of `group` elements: a group is group / 8
      // consecutive threads of one wavefront (group <= 512 and aligned), which
      // reduce its amax among themselves; the group's first thread writes the scale
      const int lpg = group >> 3;
      for (int i = tid * 8; i < d; i += 256 * 8) {
        float v[8];
        float am = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          v[j] = buf[pad(i + j)];
          am = fmaxf(am, fabsf(v[j]));
        }
        for (int o = 1; o < lpg; o <<= 1) am = fmaxf(am, __shfl_xor(am, o));
        uint16_t sh;
        float m;
        sym_scale(am, c, clip, &sh, &m);
        *(uint32_t*)(q + row * (d / 2) + i / 2) = (CLAMP || (sh & 0x7fffu) < 0x0400u)
                                                      ? quant_pack8<true>(v, m)
                                                      : quant_pack8<false>(v, m);
        if ((i & (group - 1)) == 0) scale[row * (d / group) + i / group] = sh;
      }
    } else if (MODE == MODE_QUANT || MODE == MODE_QUANT8) {
      // 4. amax over the row
      float am = 0.0f;
      for (int i = tid; i < d; i += 256) am = fmaxf(am, fabsf(buf[pad(i)]));
      am = wave_max(am);
      if ((tid & 63) == 0) red[tid >> 6] = am;
      __syncthreads();
      am = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
      const QRange rg = q_range(MODE == MODE_QUANT8 ? bits : 4);
      uint16_t sh;
      float m;
      sym_scale(am, c, clip, &sh, &m, rg.qmax);
      sh = (uint16_t)__builtin_amdgcn_readfirstlane(sh);  // the same on every lane
      // 5. quantize + pack, 8 elements per thread and step
      const bool clamp = CLAMP || (sh & 0x7fffu) < 0x0400u;  // block-uniform
      for (int i = tid * 8; i < d; i += 256 * 8) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = buf[pad(i + j)];
        if (MODE == MODE_QUANT8) {
          *(uint2*)(q + row * d + i) =
              clamp ? make_uint2(quant_pack4_i8<true>(v, m, rg.lo, rg.hi),
                                 quant_pack4_i8<true>(v + 4, m, rg.lo, rg.hi))
                    : make_uint2(quant_pack4_i8<false>(v, m, rg.lo, rg.hi),
                                 quant_pack4_i8<false>(v + 4, m, rg.lo, rg.hi));
        } else {
          *(uint32_t*)(q + row * (d / 2) + i / 2) =
              clamp ? quant_pack8<true>(v, m) : quant_pack8<false>(v, m);
        }
      }
      if (tid == 0) scale[row] = sh;
    } else if (MODE == MODE_ROT_F32) {
      for (int i = tid; i < d; i += 256) ((float*)yout)[row * d + i] = __fmul_rn(buf[pad(i)], c);
    } else {
      for (int i = tid; i < d; i += 256)
        ((uint16_t*)yout)[row * d + i] = f2h(__fmul_rn(buf[pad(i)], c));
    }
    __syncthreads();  // the LDS row is reused by the next iteration
  }
}

// ===========================================================================
// k_hq_k28: d = 1024 * 28 = 28672, one workgroup of 4 wavefronts per row
// ===========================================================================
// The row is a [1024 chunks x 28] matrix; z = (H_1024 (x) H_28) (s * x).  With
// H_1024 = H_256 (x) H_4 the factor H_112 = H_4 (x) H_28 acts on 4 consecutive
// chunks ("group" G = 0..255, 112 contiguous elements) and is a dense +-1
// contraction: it runs on the matrix cores (v_mfma_f32_16x16x32_f16) straight
// on the fp16 input with the signs XORed into the sign bits, which is exact
// (products are +-x, accumulation fp32).  B column n of an MFMA is one group,
// K = 112 padded to 4 blocks of 32, M = 112 = 7 tiles of 16.  The A rows are
// permuted so that lane (n, g) receives all 28 outputs of chunk 4G + g.
// H_256 over G remains, in fp32 VALU: G = 64 w + 16 ct + gmap(n) with w the
// wavefront, ct the lane's column tile (4 per wavefront): four stages through
// DPP across lanes, two between registers, and a radix-4 stage across the
// wavefronts through LDS (rounds of 8, 8, 8 and 4 chunk positions).  After it
// each wavefront owns column tile ct = w of all four w'' and so whole chunks;
// amax is reduced through LDS, and each lane stores its chunks' 14 bytes of
// packed codes directly (two-byte stores: measured faster than staging the row
// in LDS for 16-byte stores, which costs two more barriers per row).
// The exchange moves each lane's values as 16-byte blocks [w][ct][kb][lane]
// (four positions per block, two blocks per round); its LDS buffer holds one
// round: more would not leave room for two workgroups per CU.
constexpr int K28_XBLK = 2;                           // 16-byte blocks per (w, ct) and round
constexpr int K28_XROUND = 4 * 4 * K28_XBLK * 4 * 64;  // floats per round
constexpr int K28_AFRAG = 7 * 4 * 64;                 // A fragments: [mt][kb][lane]

// H_112 = H_4 (x) H_28 in MFMA A-fragment layout, built at compile time: tile
// mt row i -> output 28 (i >> 2) + 4 mt + (i & 3), block kb lane (i, g) ->
// columns 32 kb + 8 g .. + 7 (zero past 111); +-1 as fp16 bit patterns.
struct H112Frags {
  uint16_t v[K28_AFRAG][8];
};
constexpr H112Frags make_h112_frags() {
  H112Frags f{};
  const HTable<28> h = make_h28();
  for (int idx = 0; idx < K28_AFRAG; ++idx) {
    const int fl = idx & 63, mk = idx >> 6;
    const int mt = mk >> 2, kb = mk & 3;
    const int i = fl & 15, gg = fl >> 4;
    const int o = 28 * (i >> 2) + 4 * mt + (i & 3);
    for (int j = 0; j < 8; ++j) {
      const int col = 32 * kb + 8 * gg + j;
      uint16_t bits = 0;
      if (col < 112) {
        int par = 0;
        for (int b = (o / 28) & (col / 28); b; b >>= 1) par ^= b & 1;
        const bool neg = (h.v[o % 28][col % 28] < 0.0f) != (par == 1);
        bits = neg ? 0xBC00u : 0x3C00u;
      }
      f.v[idx][j] = bits;
    }
  }
  return f;
}
__device__ const H112Frags g_h112_frags = make_h112_frags();

// ---- fp16 variant of the transform after the matrix-core stage ----
// QuaRot paper, appendix on the FP16 Hadamard transformation (Table 10): the
// online transform may run in fp16 without changing accuracy.  Here every
// stage after the exact H_112 products rounds to fp16 (round to nearest
// even), two values per register: v_pk_add_f16 between registers and
// v_pk_fmac_f16 with DPP across lanes (one instruction per two values where
// the fp32 path needs one per value).  The stages carry z / 128 (the A
// fragments are +-2^-7), and z_dbg reports 128 times the fp16 values.

typedef _Float16 h2v __attribute__((ext_vector_type(2)));

// One fp16 butterfly stage across lanes for eight packed registers: r += dpp(r) * s.
#define QR_DPP8H(CTRL, r, s)                                                           \
  asm volatile(                                                                        \
      "s_nop 1\n\t"                                                                    \
      "v_pk_fmac_f16_dpp %0, %0, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"           \
      "v_pk_fmac_f16_dpp %1, %1, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"           \
      "v_pk_fmac_f16_dpp %2, %2, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"           \
      "v_pk_fmac_f16_dpp %3, %3, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"           \
      "v_pk_fmac_f16_dpp %4, %4, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"           \
      "v_pk_fmac_f16_dpp %5, %5, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"           \
      "v_pk_fmac_f16_dpp %6, %6, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"           \
      "v_pk_fmac_f16_dpp %7, %7, %8 " CTRL " row_mask:0xf bank_mask:0xf"               \
      : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]), "+v"(r[4]), "+v"(r[5]), "+v"(r[6]), \
        "+v"(r[7])                                                                     \
      : "v"(s))

__device__ __forceinline__ uint32_t pk_f16(float a, float b) {  // v_cvt_pk_f16_f32 (RNE)
  return __builtin_bit_cast(uint32_t, h2v{(_Float16)a, (_Float16)b});
}
__device__ __forceinline__ uint32_t hadd2(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2v, a) + __builtin_bit_cast(h2v, b));
}
__device__ __forceinline__ uint32_t hsub2(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2v, a) - __builtin_bit_cast(h2v, b));
}
// max(acc, |h.lo|, |h.hi|) on the low half of acc (fp16)
__device__ __forceinline__ uint32_t hmax3abs(uint32_t acc, uint32_t h) {
  asm("v_max3_f16 %0, |%1|, |%1|, %0 op_sel:[0,1,0,0]" : "+v"(acc) : "v"(h));
  return acc;
}
__device__ __forceinline__ float hlo(uint32_t h) { return (float)__builtin_bit_cast(h2v, h)[0]; }
__device__ __forceinline__ float hhi(uint32_t h) { return (float)__builtin_bit_cast(h2v, h)[1]; }
// Eight fp16 values (four packed words) times m -> packed nibbles, as quant_pack8.
template <bool CLAMP>
__device__ __forceinline__ uint32_t quant_pack8h(const uint32_t* h, float m) {
  float f[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[2 * j] = hlo(h[j]);
    f[2 * j + 1] = hhi(h[j]);
  }
  return quant_pack8<CLAMP>(f, m);
}

// Rest of a k_hq_k28 row in fp16 (quantizer only): v holds the fp32 products
// of H_112 (scaled by 2^-7) for the lane's four column tiles.
template <bool CLAMP>
__device__ __forceinline__ void k28_finish_f16(const float (&v)[4][28], int64_t row, int tid,
                                               int lane, int w, int gc, float s0, float s1,
                                               float s2, float s3, float sigma, float c,
                                               float clip, float* s_x, float* s_red,
                                               uint8_t* __restrict__ q,
                                               uint16_t* __restrict__ scale,
                                               float* __restrict__ zdbg) {
  constexpr int D = 28672;
  uint32_t hv[4][14];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int k = 0; k < 14; ++k) hv[ct][k] = pk_f16(v[ct][2 * k], v[ct][2 * k + 1]);
  // H_4 over ct between registers
#pragma unroll
  for (int hb = 1; hb < 4; hb <<= 1)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
      if (!(ct & hb))
#pragma unroll
        for (int k = 0; k < 14; ++k) {
          const uint32_t a = hv[ct][k], b = hv[ct + hb][k];
          hv[ct][k] = hadd2(a, b);
          hv[ct + hb][k] = hsub2(a, b);
        }
  // H_16 over gmap(n) through DPP: 56 packed registers in 7 blocks of 8
  auto pk_sign = [](float sv) { return sv < 0.0f ? 0xBC00BC00u : 0x3C003C00u; };
  const uint32_t h0 = pk_sign(s0), h1 = pk_sign(s1), h2s = pk_sign(s2), h3 = pk_sign(s3);
  uint32_t* hf = &hv[0][0];
#pragma unroll
  for (int b = 0; b < 56; b += 8) QR_DPP8H("quad_perm:[1,0,3,2]", (hf + b), h0);
#pragma unroll
  for (int b = 0; b < 56; b += 8) QR_DPP8H("quad_perm:[2,3,0,1]", (hf + b), h1);
#pragma unroll
  for (int b = 0; b < 56; b += 8) QR_DPP8H("row_half_mirror", (hf + b), h2s);
#pragma unroll
  for (int b = 0; b < 56; b += 8) QR_DPP8H("row_mirror", (hf + b), h3);
  // H_4 over the wavefront index through LDS, two rounds of 7 packed positions
  uint32_t* s_xu = (uint32_t*)s_x;
  uint32_t o[4][14];
#pragma unroll
  for (int rnd = 0; rnd < 2; ++rnd) {
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int k = 0; k < 7; ++k) s_xu[((w * 4 + ct) * 7 + k) * 64 + lane] = hv[ct][7 * rnd + k];
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 7; ++k) {
      const uint32_t a0 = s_xu[((0 * 4 + w) * 7 + k) * 64 + lane];
      const uint32_t a1 = s_xu[((1 * 4 + w) * 7 + k) * 64 + lane];
      const uint32_t a2 = s_xu[((2 * 4 + w) * 7 + k) * 64 + lane];
      const uint32_t a3 = s_xu[((3 * 4 + w) * 7 + k) * 64 + lane];
      const uint32_t p01 = hadd2(a0, a1), m01 = hsub2(a0, a1);
      const uint32_t p23 = hadd2(a2, a3), m23 = hsub2(a2, a3);
      o[0][7 * rnd + k] = hadd2(p01, p23);
      o[1][7 * rnd + k] = hadd2(m01, m23);
      o[2][7 * rnd + k] = hsub2(p01, p23);
      o[3][7 * rnd + k] = hsub2(m01, m23);
    }
    __syncthreads();
  }
  // o[w2][k] = sigma * z / 128 (fp16 pair) at chunk 4 ((4 w2 + w) 16 + gc) + g, positions 2k, 2k + 1
  const int g = lane >> 4;
  auto chunk_of = [&](int w2) { return 4 * ((4 * w2 + w) * 16 + gc) + g; };
  if (zdbg) {
    const float zs = 128.0f * sigma;
#pragma unroll
    for (int w2 = 0; w2 < 4; ++w2) {
      float* zr = zdbg + row * D + chunk_of(w2) * 28;
#pragma unroll
      for (int k = 0; k < 14; k += 2)
        *(v4f*)(zr + 2 * k) = v4f{hlo(o[w2][k]) * zs, hhi(o[w2][k]) * zs,
                                  hlo(o[w2][k + 1]) * zs, hhi(o[w2][k + 1]) * zs};
    }
  }
  uint32_t amh = 0;
#pragma unroll
  for (int w2 = 0; w2 < 4; ++w2)
#pragma unroll
    for (int k = 0; k < 14; ++k) amh = hmax3abs(amh, o[w2][k]);
  float am = wave_max(hlo(amh));
  if (lane == 0) s_red[w] = am;
  __syncthreads();
  am = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  uint16_t sh;
  float m;
  // the fp16 stages carry z / 128: the same recipe with c * 128 (exact scaling)
  sym_scale(am, c * 128.0f, clip, &sh, &m);
  sh = (uint16_t)__builtin_amdgcn_readfirstlane(sh);
  const float ml = m * sigma;
  uint16_t* qrow = (uint16_t*)(q + row * (D / 2));
  auto emit = [&](auto clamp_tag) {
    constexpr bool CL = decltype(clamp_tag)::value;
#pragma unroll
    for (int w2 = 0; w2 < 4; ++w2) {
      uint32_t words[4];
#pragma unroll
      for (int k8 = 0; k8 < 3; ++k8) words[k8] = quant_pack8h<CL>(&o[w2][4 * k8], ml);
      const uint32_t tail[4] = {o[w2][12], o[w2][13], 0u, 0u};
      words[3] = quant_pack8h<CL>(tail, ml);
      uint16_t* qc = qrow + chunk_of(w2) * 7;  // 14 bytes of packed codes per chunk
#pragma unroll
      for (int k = 0; k < 7; ++k)
        __builtin_nontemporal_store(
            (uint16_t)((k & 1) ? (words[k >> 1] >> 16) : (words[k >> 1] & 0xffffu)), qc + k);
    }
  };
  if (CLAMP || (sh & 0x7fffu) < 0x0400u)
    emit(std::true_type{});
  else
    emit(std::false_type{});
  if (tid == 0) scale[row] = sh;
}

template <int MODE, bool CLAMP, bool F16>
__global__ __launch_bounds__(256, K28_WAVES_PER_SIMD) void k_hq_k28(const uint16_t* __restrict__ x, int64_t T,
                                                   int64_t ld, const int8_t* __restrict__ signs,
                                                   float c, float clip, int bits,
                                                   uint8_t* __restrict__ q,
                                                   uint16_t* __restrict__ scale,
                                                   float* __restrict__ zdbg,
                                                   void* __restrict__ yout) {
  constexpr int D = 28672;
  __shared__ v8h s_afrag[K28_AFRAG];           // 28 KB
  __shared__ __attribute__((aligned(16))) float s_x[K28_XROUND];  // exchange rounds
  __shared__ v4u s_sbits[4 * 4 * 64];         // 16 KB
  __shared__ float s_red[4];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int gc = gmap(n);

  // A fragments of H_112 = H_4 (x) H_28: tile mt row i -> output 28 (i >> 2) + 4 mt + (i & 3),
  // block kb lane (i, g) holds columns 32 kb + 8 g + j (zero past 112).
  // (reading them through the caches on every row instead was measured slower)
  static_assert(!F16 || MODE == MODE_QUANT, "the fp16 transform is a quantizer variant");
  const v8h* afrag_g = (const v8h*)&g_h112_frags.v[0][0];
  for (int f = tid; f < K28_AFRAG; f += 256) {
    v4u a = __builtin_bit_cast(v4u, afrag_g[f]);
    // fp16 transform: +-1 (0x3C00, 0xBC00) -> +-2^-7 (0x2000, 0xA000) by masking;
    // the fp16 stages then carry z / 128, which keeps the first stage's sums
    // of 112 fp16 inputs inside the fp16 range
    if (F16) a &= 0xA000A000u;
    s_afrag[f] = __builtin_bit_cast(v8h, a);
  }
  const v8h* afrag = s_afrag;
  // Signs of the lane's B fragments (the same for every row), one dword per
  // fragment: bit 15 - j holds the sign of element 2 j, bit 31 - j that of
  // element 2 j + 1, so (E << j) & 0x80008000 is the sign-bit mask of dword j.
  // Kept in LDS ([w][ct][lane][kb]) and read once per row: held in registers
  // they would be recomputed from the sign vector on every row.
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    v4u ev;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int G = (w * 4 + ct) * 16 + gc;
      const int e0 = G * 112 + 32 * kb + 8 * g;
      ev[kb] = (signs && 32 * kb + 8 * g < 112) ? sign_word8(signs + e0) : 0u;
    }
    s_sbits[(w * 4 + ct) * 64 + lane] = ev;
  }
  const float s0 = (gc & 1) ? -1.0f : 1.0f;
  const float s1 = (gc & 2) ? -1.0f : 1.0f;
  const float s2 = (gc & 4) ? -1.0f : 1.0f;
  const float s3 = (gc & 8) ? -1.0f : 1.0f;
  const float sigma = (__builtin_popcount(gc) & 1) ? -1.0f : 1.0f;  // lane holds sigma * z
  __syncthreads();

  // ---- B fragments: group G, elements 32 kb + 8 g .. + 7 (16 bytes) ----
  v4u braw[4][4];
  auto load_b = [&](int64_t r) {
    const uint16_t* xr = x + r * ld;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const int G = (w * 4 + ct) * 16 + gc;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        braw[ct][kb] = (kb < 3 || g < 2) ? ld_stream(xr + G * 112 + 32 * kb + 8 * g)
                                         : v4u{0u, 0u, 0u, 0u};
    }
  };
  for (int64_t row = blockIdx.x; row < T; row += gridDim.x) {
    load_b(row);
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const v4u ev = s_sbits[(w * 4 + ct) * 64 + lane];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int j = 0; j < 4; ++j) braw[ct][kb][j] ^= (ev[kb] << j) & 0x80008000u;
    }
    // ---- H_112 on the matrix cores ----
    float v[4][28];
#pragma unroll
    for (int mt = 0; mt < 7; ++mt) {
      v4f accm[4];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) accm[ct] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const v8h a = afrag[(mt * 4 + kb) * 64 + lane];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          const v8h b = __builtin_bit_cast(v8h, braw[ct][kb]);
          accm[ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, accm[ct], 0, 0, 0);
        }
      }
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) v[ct][4 * mt + r] = accm[ct][r];
    }
    if constexpr (F16) {
      k28_finish_f16<CLAMP>(v, row, tid, lane, w, gc, s0, s1, s2, s3, sigma, c, clip, s_x, s_red,
                            q, scale, zdbg);
      continue;
    }
    // ---- H_4 over ct: butterflies between registers (first, so that plain VALU
    //      ops and not the DPP asm consume the MFMA results) ----
#pragma unroll
    for (int hb = 1; hb < 4; hb <<= 1)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
        if (!(ct & hb))
#pragma unroll
          for (int k = 0; k < 28; ++k) {
            const float a = v[ct][k], b = v[ct + hb][k];
            v[ct][k] = a + b;
            v[ct + hb][k] = a - b;
          }
    // ---- H_16 over gmap(n): DPP butterflies across lanes ----
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
#pragma unroll
      for (int k = 0; k < 24; k += 8) QR_DPP8("quad_perm:[1,0,3,2]", (&v[ct][k]), s0);
    }
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
#pragma unroll
      for (int k = 0; k < 24; k += 8) QR_DPP8("quad_perm:[2,3,0,1]", (&v[ct][k]), s1);
    }
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
#pragma unroll
      for (int k = 0; k < 24; k += 8) QR_DPP8("row_half_mirror", (&v[ct][k]), s2);
    }
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
#pragma unroll
      for (int k = 0; k < 24; k += 8) QR_DPP8("row_mirror", (&v[ct][k]), s3);
    }
    {
      // positions 24..27 of the four column tiles, eight registers per call
      float t8[8];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          t8[k] = v[2 * h][24 + k];
          t8[4 + k] = v[2 * h + 1][24 + k];
        }
        QR_DPP8("quad_perm:[1,0,3,2]", t8, s0);
        QR_DPP8("quad_perm:[2,3,0,1]", t8, s1);
        QR_DPP8("row_half_mirror", t8, s2);
        QR_DPP8("row_mirror", t8, s3);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          v[2 * h][24 + k] = t8[k];
          v[2 * h + 1][24 + k] = t8[4 + k];
        }
      }
    }
    // ---- H_4 over the wavefront index through LDS; afterwards v[w''][k] holds
    //      chunk 4 G + g, G = (4 w'' + w) 16 + gmap(n), position k ----
    float o[4][28];
    v4f* s_x4 = (v4f*)s_x;
#pragma unroll
    for (int rnd = 0; rnd < 4; ++rnd) {
      const int nb = rnd < 3 ? K28_XBLK : 1;  // blocks of 4 positions: 8, 8, 8, then 4
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int kb = 0; kb < nb; ++kb) {
          const int k0 = 8 * rnd + 4 * kb;
          s_x4[((w * 4 + ct) * K28_XBLK + kb) * 64 + lane] =
              v4f{v[ct][k0], v[ct][k0 + 1], v[ct][k0 + 2], v[ct][k0 + 3]};
        }
      __syncthreads();
#pragma unroll
      for (int kb = 0; kb < nb; ++kb) {
        const int k0 = 8 * rnd + 4 * kb;
        const v4f a0 = s_x4[((0 * 4 + w) * K28_XBLK + kb) * 64 + lane];
        const v4f a1 = s_x4[((1 * 4 + w) * K28_XBLK + kb) * 64 + lane];
        const v4f a2 = s_x4[((2 * 4 + w) * K28_XBLK + kb) * 64 + lane];
        const v4f a3 = s_x4[((3 * 4 + w) * K28_XBLK + kb) * 64 + lane];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p01 = a0[j] + a1[j], m01 = a0[j] - a1[j];
          const float p23 = a2[j] + a3[j], m23 = a2[j] - a3[j];
          o[0][k0 + j] = p01 + p23;
          o[1][k0 + j] = m01 + m23;
          o[2][k0 + j] = p01 - p23;
          o[3][k0 + j] = m01 - m23;
        }
      }
      __syncthreads();
    }
    // chunk index of o[w2] for this lane
    auto chunk_of = [&](int w2) { return 4 * ((4 * w2 + w) * 16 + gc) + g; };

    if (zdbg) {
#pragma unroll
      for (int w2 = 0; w2 < 4; ++w2) {
        float* zr = zdbg + row * D + chunk_of(w2) * 28;
#pragma unroll
        for (int k = 0; k < 28; k += 4)
          *(v4f*)(zr + k) = v4f{o[w2][k] * sigma, o[w2][k + 1] * sigma, o[w2][k + 2] * sigma,
                                o[w2][k + 3] * sigma};
      }
    }
    if (MODE == MODE_QUANT || MODE == MODE_QUANT8) {
      float am = 0.0f;
#pragma unroll
      for (int w2 = 0; w2 < 4; ++w2)
#pragma unroll
        for (int k = 0; k < 28; ++k) am = fmaxf(am, fabsf(o[w2][k]));
      am = wave_max(am);
      if (lane == 0) s_red[w] = am;
      __syncthreads();
      am = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
      const QRange rg = q_range(MODE == MODE_QUANT8 ? bits : 4);
      uint16_t sh;
      float m;
      sym_scale(am, c, clip, &sh, &m, rg.qmax);
      // The scale is the same on every lane: make that visible, so that the
      // clamp decision below is one scalar branch and not a per-lane mask.
      sh = (uint16_t)__builtin_amdgcn_readfirstlane(sh);
      const float ml = m * sigma;
      uint16_t* qrow = (uint16_t*)(q + row * (D / 2));
      auto emit = [&](auto clamp_tag) {
        constexpr bool CL = decltype(clamp_tag)::value;
        if constexpr (MODE == MODE_QUANT8) {
          // 28 codes of one byte per chunk: seven dwords
#pragma unroll
          for (int w2 = 0; w2 < 4; ++w2) {
            uint32_t* qc = (uint32_t*)(q + row * D + chunk_of(w2) * 28);
#pragma unroll
            for (int k = 0; k < 7; ++k)
              st_stream(qc + k, quant_pack4_i8<CL>(&o[w2][4 * k], ml, rg.lo, rg.hi));
          }
          return;
        }
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2) {
          uint32_t words[4];
#pragma unroll
          for (int k8 = 0; k8 < 3; ++k8) words[k8] = quant_pack8<CL>(&o[w2][8 * k8], ml);
          float tail[8] = {o[w2][24], o[w2][25], o[w2][26], o[w2][27], 0.0f, 0.0f, 0.0f, 0.0f};
          words[3] = quant_pack8<CL>(tail, ml);
          uint16_t* qc = qrow + chunk_of(w2) * 7;  // 14 bytes of packed codes per chunk
#pragma unroll
          for (int k = 0; k < 7; ++k)
            __builtin_nontemporal_store(
                (uint16_t)((k & 1) ? (words[k >> 1] >> 16) : (words[k >> 1] & 0xffffu)), qc + k);
        }
      };
      if (CLAMP || (sh & 0x7fffu) < 0x0400u)
        emit(std::true_type{});
      else
        emit(std::false_type{});
      if (tid == 0) scale[row] = sh;
    } else {
      const float cs = c * sigma;
#pragma unroll
      for (int w2 = 0; w2 < 4; ++w2) {
        const int e0 = chunk_of(w2) * 28;
        if (MODE == MODE_ROT_F32) {
          float* yr = (float*)yout + row * D + e0;
#pragma unroll
          for (int k = 0; k < 28; k += 4)
            *(v4f*)(yr + k) = v4f{__fmul_rn(o[w2][k], cs), __fmul_rn(o[w2][k + 1], cs),
                                  __fmul_rn(o[w2][k + 2], cs), __fmul_rn(o[w2][k + 3], cs)};
        } else {
          uint32_t* yr = (uint32_t*)((uint16_t*)yout + row * D + e0);
#pragma unroll
          for (int k = 0; k < 28; k += 2)
            yr[k / 2] = (uint32_t)f2h(__fmul_rn(o[w2][k], cs)) |
                        ((uint32_t)f2h(__fmul_rn(o[w2][k + 1], cs)) << 16);
        }
      }
    }
  }
}

// ===========================================================================
// k_hq_k172: d = 64 * 172 = 11008, one workgroup of 4 wavefronts per row
// ===========================================================================
// The row is a [64 chunks x 172] matrix; z = (H_64 (x) H_172) (s * x).  H_172,
// a dense +-1 contraction on every chunk, runs on the matrix cores
// (v_mfma_f32_16x16x32_f16) on the sign-flipped fp16 input: B column n is
// chunk a = 16 ct + gmap(n), K = 172 padded to 6 blocks of 32, and the 11
// output tiles of 16 rows (172 padded to 176) are split over the wavefronts
// (tiles w, w + 4, w + 8).  Every wavefront therefore sees every chunk, so
// H_64 over the chunk index stays inside it: four DPP stages across lanes and
// two between its column-tile registers.  Lane (n, g) of tile mt holds chunk
// positions 16 mt + 4 g .. + 3, i.e. two bytes of packed codes per (mt, ct),
// staged in LDS for coalesced row stores.
// The workgroup reads each row from HBM once: every thread fetches its six
// 16-byte chunks of the next row while the current one is transformed, then
// writes them, sign-flipped, into one of two LDS row buffers, from which the
// wavefronts read their B fragments.  The A fragments of a wavefront's three
// output tiles stay in registers for the whole kernel.
constexpr int K172_AFRAG = 11 * 6 * 64;  // A fragments [mt][kb][lane], 8 fp16 each: 66 KB

// H_172 in MFMA A-fragment layout, built at compile time: tile mt row i ->
// output 16 mt + i, block kb lane (i, g) -> columns 32 kb + 8 g .. + 7; +-1 as
// fp16 bit patterns, zero past 171 in either index.
struct H172Frags {
  uint16_t v[K172_AFRAG][8];
};
constexpr H172Frags make_h172_frags(uint16_t one, uint16_t minus_one) {
  H172Frags f{};
  const HTable<172> h = make_h172();
  for (int idx = 0; idx < K172_AFRAG; ++idx) {
    const int fl = idx & 63, mk = idx >> 6;
    const int mt = mk / 6, kb = mk % 6;
    const int o = 16 * mt + (fl & 15), gg = fl >> 4;
    for (int j = 0; j < 8; ++j) {
      const int col = 32 * kb + 8 * gg + j;
      uint16_t bits = 0;
      if (o < 172 && col < 172) bits = h.v[o][col] > 0.0f ? one : minus_one;
      f.v[idx][j] = bits;
    }
  }
  return f;
}
__device__ const H172Frags g_h172_frags = make_h172_frags(0x3C00u, 0xBC00u);
// +-2^-8 for the fp16 transform: the fp16 stages carry z / 256, which keeps
// the first stage's sums of 172 fp16 inputs inside the fp16 range
__device__ const H172Frags g_h172_frags16 = make_h172_frags(0x1C00u, 0x9C00u);

template <int MODE, bool CLAMP, bool F16>
__global__ __launch_bounds__(256, 2) void k_hq_k172(const uint16_t* __restrict__ x, int64_t T,
                                                    int64_t ld, const int8_t* __restrict__ signs,
                                                    float c, float clip, int bits,
                                                    uint8_t* __restrict__ q,
                                                    uint16_t* __restrict__ scale,
                                                    float* __restrict__ zdbg,
                                                    void* __restrict__ yout) {
  constexpr int D = 11008;
  constexpr int NCH = D / 8;                // 16-byte chunks per row: 1376
  constexpr int SPT = (NCH + 255) / 256;    // chunks staged per thread: 6 (the last for tid < 96)
  // The row, sign-flipped, double buffered: rows alternate between the two
  // buffers, so the staging barrier of one row also orders every wavefront's
  // last read of the buffer the row after next overwrites.
  __shared__ __attribute__((aligned(16))) uint16_t s_row[2][D];  // 43 KB
  __shared__ uint16_t s_stage[D / 4];        // packed row: 5504 bytes
  __shared__ float s_red[4];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int gc = gmap(n);
  static_assert(!F16 || MODE == MODE_QUANT, "the fp16 transform is a quantizer variant");

  // Sign-bit masks of the chunks this thread stages (the same for every row).
  v4u smask[SPT];
#pragma unroll
  for (int i = 0; i < SPT; ++i) {
    const int ch = tid + 256 * i;
    smask[i] = (signs && ch < NCH) ? sign_masks8(signs + 8 * ch) : v4u{0u, 0u, 0u, 0u};
  }
  const float s0 = (gc & 1) ? -1.0f : 1.0f;
  const float s1 = (gc & 2) ? -1.0f : 1.0f;
  const float s2 = (gc & 4) ? -1.0f : 1.0f;
  const float s3 = (gc & 8) ? -1.0f : 1.0f;
  const float sigma = (__builtin_popcount(gc) & 1) ? -1.0f : 1.0f;  // lane holds sigma * z
  const int nmt = (w < 3) ? 3 : 2;  // tiles w, w + 4, w + 8 (< 11)
  // A fragments of this wavefront's output tiles, held in registers for the
  // whole kernel (zero for the fourth wavefront's missing third tile).
  v8h areg[3][6];
  {
    const v8h* afrag = (const v8h*)&(F16 ? g_h172_frags16 : g_h172_frags).v[0][0];
#pragma unroll
    for (int t = 0; t < 3; ++t)
#pragma unroll
      for (int kb = 0; kb < 6; ++kb)
        areg[t][kb] = t < nmt ? afrag[((w + 4 * t) * 6 + kb) * 64 + lane] : v8h{};
  }

  // The next row's chunks, in flight while the current row is transformed.
  v4u pre[SPT];
  auto fetch = [&](int64_t r) {
    const uint16_t* xr = x + r * ld;
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const int ch = tid + 256 * i;
      pre[i] = ch < NCH ? ld_stream(xr + 8 * ch) : v4u{0u, 0u, 0u, 0u};
    }
  };
  if ((int64_t)blockIdx.x < T) fetch(blockIdx.x);

  int buf = 0;
  for (int64_t row = blockIdx.x; row < T; row += gridDim.x, buf ^= 1) {
    uint16_t* srow = s_row[buf];
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const int ch = tid + 256 * i;
      if (ch < NCH) *(v4u*)(srow + 8 * ch) = pre[i] ^ smask[i];
    }
    __syncthreads();
    if (row + gridDim.x < T) fetch(row + gridDim.x);

    // ---- H_172 on the matrix cores: B column n of block kb is chunk
    //      a = 16 ct + gc, elements 32 kb + 8 g .. + 7 (zero past 171);
    //      v[t][ct][r] = output 16 (w + 4 t) + 4 g + r ----
    v4f acc[3][4];
#pragma unroll
    for (int t = 0; t < 3; ++t)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) acc[t][ct] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kb = 0; kb < 6; ++kb) {
      const int col = 32 * kb + 8 * g;
      v8h bq[4];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        // chunk starts are 8-byte aligned in LDS (172 elements = 344 bytes)
        const uint2* p = (const uint2*)(srow + (16 * ct + gc) * 172 + col);
        v4u raw = {0u, 0u, 0u, 0u};
        if (col + 8 <= 172) {
          const uint2 lo = p[0], hi = p[1];
          raw = v4u{lo.x, lo.y, hi.x, hi.y};
        } else if (col < 172) {  // 168 .. 171
          const uint2 lo = p[0];
          raw[0] = lo.x;
          raw[1] = lo.y;
        }
        bq[ct] = __builtin_bit_cast(v8h, raw);
      }
#pragma unroll
      for (int t = 0; t < 3; ++t)
        if (t < nmt)
#pragma unroll
          for (int ct = 0; ct < 4; ++ct)
            acc[t][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(areg[t][kb], bq[ct], acc[t][ct],
                                                                0, 0, 0);
    }
    float v[3][4][4];
#pragma unroll
    for (int t = 0; t < 3; ++t)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) v[t][ct][r] = acc[t][ct][r];
    // element index of v[t][ct][0]: chunk 16 ct + gc, position 16 (w + 4 t) + 4 g
    auto elem_of = [&](int t, int ct) { return (16 * ct + gc) * 172 + 16 * (w + 4 * t) + 4 * g; };
    auto valid = [&](int t) { return t < nmt && 16 * (w + 4 * t) + 4 * g < 172; };
    if constexpr (F16) {
      // fp16 transform (QR_ROT_HADAMARD_F16): the remaining six stages on
      // packed fp16 pairs, as in k28_finish_f16
      uint32_t hv[3][4][2];
#pragma unroll
      for (int t = 0; t < 3; ++t)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          hv[t][ct][0] = pk_f16(v[t][ct][0], v[t][ct][1]);
          hv[t][ct][1] = pk_f16(v[t][ct][2], v[t][ct][3]);
        }
#pragma unroll
      for (int hb = 1; hb < 4; hb <<= 1)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
          if (!(ct & hb))
#pragma unroll
            for (int t = 0; t < 3; ++t)
#pragma unroll
              for (int j = 0; j < 2; ++j) {
                const uint32_t p = hv[t][ct][j], m = hv[t][ct + hb][j];
                hv[t][ct][j] = hadd2(p, m);
                hv[t][ct + hb][j] = hsub2(p, m);
              }
      auto pk_sign = [](float sv) { return sv < 0.0f ? 0xBC00BC00u : 0x3C003C00u; };
      const uint32_t h0 = pk_sign(s0), h1 = pk_sign(s1), h2s = pk_sign(s2), h3 = pk_sign(s3);
#pragma unroll
      for (int t = 0; t < 3; ++t) {
        uint32_t* r8 = &hv[t][0][0];
        QR_DPP8H("quad_perm:[1,0,3,2]", r8, h0);
        QR_DPP8H("quad_perm:[2,3,0,1]", r8, h1);
        QR_DPP8H("row_half_mirror", r8, h2s);
        QR_DPP8H("row_mirror", r8, h3);
      }
      if (zdbg) {
        const float zs = 256.0f * sigma;
#pragma unroll
        for (int t = 0; t < 3; ++t)
          if (valid(t))
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
              *(v4f*)(zdbg + row * D + elem_of(t, ct)) =
                  v4f{hlo(hv[t][ct][0]) * zs, hhi(hv[t][ct][0]) * zs, hlo(hv[t][ct][1]) * zs,
                      hhi(hv[t][ct][1]) * zs};
      }
      uint32_t amh = 0;
#pragma unroll
      for (int t = 0; t < 3; ++t)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
#pragma unroll
          for (int j = 0; j < 2; ++j) amh = hmax3abs(amh, hv[t][ct][j]);
      float am = wave_max(hlo(amh));
      if (lane == 0) s_red[w] = am;
      __syncthreads();
      am = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
      uint16_t sh;
      float m;
      sym_scale(am, c * 256.0f, clip, &sh, &m);  // the stages carry z / 256
      sh = (uint16_t)__builtin_amdgcn_readfirstlane(sh);
      const float ml = m * sigma;
      const bool clamp = CLAMP || (sh & 0x7fffu) < 0x0400u;  // block-uniform
#pragma unroll
      for (int t = 0; t < 3; ++t)
        if (valid(t))
#pragma unroll
          for (int ct = 0; ct < 4; ct += 2) {
            const uint32_t h4[4] = {hv[t][ct][0], hv[t][ct][1], hv[t][ct + 1][0], hv[t][ct + 1][1]};
            const uint32_t word = clamp ? quant_pack8h<true>(h4, ml) : quant_pack8h<false>(h4, ml);
            s_stage[elem_of(t, ct) / 4] = (uint16_t)(word & 0xffffu);
            s_stage[elem_of(t, ct + 1) / 4] = (uint16_t)(word >> 16);
          }
      __syncthreads();
      const uint32_t* st32 = (const uint32_t*)s_stage;
      uint32_t* qr32 = (uint32_t*)(q + row * (D / 2));
      for (int i = tid; i < D / 8; i += 256) st_stream(qr32 + i, st32[i]);
      if (tid == 0) scale[row] = sh;
      __syncthreads();  // stage and s_red are reused by the next row
      continue;
    }
    // ---- H_4 over ct between registers (plain VALU consumes the MFMA results) ----
#pragma unroll
    for (int hb = 1; hb < 4; hb <<= 1)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
        if (!(ct & hb))
#pragma unroll
          for (int t = 0; t < 3; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float p = v[t][ct][r], m = v[t][ct + hb][r];
              v[t][ct][r] = p + m;
              v[t][ct + hb][r] = p - m;
            }
    // ---- H_16 over gmap(n): DPP butterflies across lanes, 8 registers per call ----
#pragma unroll
    for (int t = 0; t < 3; ++t)
#pragma unroll
      for (int c2 = 0; c2 < 4; c2 += 2) {
        float r8[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          r8[r] = v[t][c2][r];
          r8[4 + r] = v[t][c2 + 1][r];
        }
        QR_DPP8("quad_perm:[1,0,3,2]", r8, s0);
        QR_DPP8("quad_perm:[2,3,0,1]", r8, s1);
        QR_DPP8("row_half_mirror", r8, s2);
        QR_DPP8("row_mirror", r8, s3);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          v[t][c2][r] = r8[r];
          v[t][c2 + 1][r] = r8[4 + r];
        }
      }
    if (zdbg) {
#pragma unroll
      for (int t = 0; t < 3; ++t)
        if (valid(t))
#pragma unroll
          for (int ct = 0; ct < 4; ++ct)
            *(v4f*)(zdbg + row * D + elem_of(t, ct)) =
                v4f{v[t][ct][0] * sigma, v[t][ct][1] * sigma, v[t][ct][2] * sigma, v[t][ct][3] * sigma};
    }
    if (MODE == MODE_QUANT || MODE == MODE_QUANT8) {
      float am = 0.0f;
#pragma unroll
      for (int t = 0; t < 3; ++t)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
#pragma unroll
          for (int r = 0; r < 4; ++r) am = fmaxf(am, fabsf(v[t][ct][r]));
      am = wave_max(am);
      if (lane == 0) s_red[w] = am;
      __syncthreads();
      am = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
      const QRange rg = q_range(MODE == MODE_QUANT8 ? bits : 4);
      uint16_t sh;
      float m;
      sym_scale(am, c, clip, &sh, &m, rg.qmax);
      sh = (uint16_t)__builtin_amdgcn_readfirstlane(sh);  // the same on every lane
      const float ml = m * sigma;
      const bool clamp = CLAMP || (sh & 0x7fffu) < 0x0400u;  // block-uniform
      if constexpr (MODE == MODE_QUANT8) {
        // four consecutive codes of one byte per (t, ct): one dword each, in place
#pragma unroll
        for (int t = 0; t < 3; ++t)
          if (valid(t))
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
              st_stream((uint32_t*)(q + row * D + elem_of(t, ct)),
                        clamp ? quant_pack4_i8<true>(v[t][ct], ml, rg.lo, rg.hi)
                              : quant_pack4_i8<false>(v[t][ct], ml, rg.lo, rg.hi));
        if (tid == 0) scale[row] = sh;
        __syncthreads();  // s_red is reused by the next row
        continue;
      }
#pragma unroll
      for (int t = 0; t < 3; ++t)
        if (valid(t))
#pragma unroll
          for (int ct = 0; ct < 4; ct += 2) {
            float e8[8];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              e8[r] = v[t][ct][r];
              e8[4 + r] = v[t][ct + 1][r];
            }
            const uint32_t word = clamp ? quant_pack8<true>(e8, ml) : quant_pack8<false>(e8, ml);
            s_stage[elem_of(t, ct) / 4] = (uint16_t)(word & 0xffffu);
            s_stage[elem_of(t, ct + 1) / 4] = (uint16_t)(word >> 16);
          }
      __syncthreads();
      const uint32_t* st32 = (const uint32_t*)s_stage;
      uint32_t* qr32 = (uint32_t*)(q + row * (D / 2));
      for (int i = tid; i < D / 8; i += 256) st_stream(qr32 + i, st32[i]);
      if (tid == 0) scale[row] = sh;
      __syncthreads();  // stage and s_red are reused by the next row
    } else {
      const float cs = c * sigma;
#pragma unroll
      for (int t = 0; t < 3; ++t)
        if (valid(t))
#pragma unroll
          for (int ct = 0; ct < 4; ++ct) {
            const int e0 = elem_of(t, ct);
            if (MODE == MODE_ROT_F32) {
              *(v4f*)((float*)yout + row * D + e0) =
                  v4f{__fmul_rn(v[t][ct][0], cs), __fmul_rn(v[t][ct][1], cs),
                      __fmul_rn(v[t][ct][2], cs), __fmul_rn(v[t][ct][3], cs)};
            } else {
              uint2 o2;
              o2.x = (uint32_t)f2h(__fmul_rn(v[t][ct][0], cs)) |
                     ((uint32_t)f2h(__fmul_rn(v[t][ct][1], cs)) << 16);
              o2.y = (uint32_t)f2h(__fmul_rn(v[t][ct][2], cs)) |
                     ((uint32_t)f2h(__fmul_rn(v[t][ct][3], cs)) << 16);
              *(uint2*)((uint16_t*)yout + row * D + e0) = o2;
            }
          }
    }
  }
}

// ===========================================================================
// Host side
// ===========================================================================
static int grid_for(int64_t work_items, int per_block, int cap) {
  int64_t g = (work_items + per_block - 1) / per_block;
  if (g > cap) g = cap;
  if (g < 1) g = 1;
  return (int)g;
}

template <int MODE, bool CLAMP>
static qr_status launch_pow2(int nb, const uint16_t* x, int64_t T, int64_t ld, const int8_t* s,
                             float c, float clip, uint8_t* q, uint16_t* sc, float* z, void* y,
                             hipStream_t st) {
  // two workgroups per CU, all resident (more workgroups measured no faster)
  const int grid = grid_for(T, 4, 512);
  switch (nb) {
#define QR_CASE(NBV)                                                                   \
  case NBV:                                                                            \
    if (z)                                                                             \
      hipLaunchKernelGGL((k_hq_pow2<NBV, MODE, CLAMP, true>), dim3(grid), dim3(256), 0, st, x, T, \
                         ld, s, c, clip, q, sc, z, y);                                 \
    else                                                                               \
      hipLaunchKernelGGL((k_hq_pow2<NBV, MODE, CLAMP, false>), dim3(grid), dim3(256), 0, st, x, \
                         T, ld, s, c, clip, q, sc, z, y);                              \
    break;
    QR_CASE(1)
    QR_CASE(2)
    QR_CASE(4)
    QR_CASE(8)
    QR_CASE(16)
#undef QR_CASE
    default:
      return QR_ERR_UNSUPPORTED;
  }
  return launch_status();
}

template <int MODE, bool CLAMP>
static qr_status launch_small(int d, int rot, const uint16_t* x, int64_t T, int64_t ld,
                              const int8_t* s, float c, float clip, uint8_t* q, uint16_t* sc,
                              float* z, void* y, hipStream_t st) {
  const int lpr = d / 8;
  const int rows_per_block = 4 * (64 / lpr);
  const int grid = grid_for(T, rows_per_block, 2048);
  switch (lpr) {
#define QR_CASE(L)                                                                     \
  case L:                                                                              \
    hipLaunchKernelGGL((k_hq_small<L, MODE, CLAMP>), dim3(grid), dim3(256), 0, st, x, T, ld, s, \
                       rot, c, clip, q, sc, z, y);                                     \
    break;
    QR_CASE(1)
    QR_CASE(2)
    QR_CASE(4)
    QR_CASE(8)
    QR_CASE(16)
    QR_CASE(32)
#undef QR_CASE
    default:
      return QR_ERR_UNSUPPORTED;
  }
  return launch_status();
}

template <int M, int MODE, bool CLAMP, bool ROT>
static qr_status launch_lds_t(int d, int n, const uint16_t* x, int64_t T, int64_t ld,
                              const int8_t* s, float c, float clip, uint8_t* q, uint16_t* sc,
                              float* z, void* y, hipStream_t st, int bits = 4, int group = 0) {
  const int plen = (d + (d >> 5)) + 1;
  const size_t bytes = ((size_t)((M == 172 && ROT) ? 2 : 1) * plen + 8) * sizeof(float);
  if (bytes > 160 * 1024) return QR_ERR_UNSUPPORTED;
  auto kern = k_hq_lds<M, MODE, CLAMP, ROT>;
  if (bytes > 64 * 1024 &&
      hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)bytes) != hipSuccess)
    return QR_ERR_LAUNCH;
  const int grid = grid_for(T, 1, 2048);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(256), bytes, st, x, T, d, n, ld, s, c, clip, bits,
                     group, q, sc, z, y);
  return launch_status();
}

template <int MODE, bool CLAMP, bool F16>
static qr_status launch_k28(const uint16_t* x, int64_t T, int64_t ld, const int8_t* signs, float c,
                            float clip, uint8_t* qq, uint16_t* ss, float* z, void* y,
                            hipStream_t st, int bits = 4) {
  const int grid = grid_for(T, 1, 512);  // two workgroups per CU, all resident
  hipLaunchKernelGGL((k_hq_k28<MODE, CLAMP, F16>), dim3(grid), dim3(256), 0, st, x, T, ld, signs,
                     c, clip, bits, qq, ss, z, y);
  return launch_status();
}

template <int MODE, bool CLAMP, bool F16>
static qr_status launch_k172(const uint16_t* x, int64_t T, int64_t ld, const int8_t* signs,
                             float c, float clip, uint8_t* qq, uint16_t* ss, float* z, void* y,
                             hipStream_t st, int bits = 4) {
  const int grid = grid_for(T, 1, 512);
  hipLaunchKernelGGL((k_hq_k172<MODE, CLAMP, F16>), dim3(grid), dim3(256), 0, st, x, T, ld,
                     signs, c, clip, bits, qq, ss, z, y);
  return launch_status();
}

template <int MODE, bool CLAMP>
static qr_status dispatch(const void* x_f16, int64_t T, int32_t d, int64_t ld, int rot,
                          const int8_t* signs, float clip, void* q, void* sc, float* z, void* y,
                          hipStream_t st) {
  const uint16_t* x = (const uint16_t*)x_f16;
  uint8_t* qq = (uint8_t*)q;
  uint16_t* ss = (uint16_t*)sc;
  if (!rot)
    return launch_lds_t<1, MODE, CLAMP, false>(d, 0, x, T, ld, signs, 1.0f, clip, qq, ss, z, y, st);
  int n = 0, m = 0;
  if (!factor_width(d, &n, &m)) return QR_ERR_UNSUPPORTED;
  const float c = norm_constant(d);
  if (m == 1) {
    if (d >= 512)
      return launch_pow2<MODE, CLAMP>(d / 512, x, T, ld, signs, c, clip, qq, ss, z, y, st);
    return launch_small<MODE, CLAMP>(d, 1, x, T, ld, signs, c, clip, qq, ss, z, y, st);
  }
  if (m == 28 && n == 10) return launch_k28<MODE, CLAMP, false>(x, T, ld, signs, c, clip, qq, ss, z, y, st);
  if (m == 28)
    return launch_lds_t<28, MODE, CLAMP, true>(d, n, x, T, ld, signs, c, clip, qq, ss, z, y, st);
  if (n == 6) return launch_k172<MODE, CLAMP, false>(x, T, ld, signs, c, clip, qq, ss, z, y, st);
  return launch_lds_t<172, MODE, CLAMP, true>(d, n, x, T, ld, signs, c, clip, qq, ss, z, y, st);
}

// b-bit codes one per byte: d = 1024 * 28 and 64 * 172 through their own
// kernels, every other width through the LDS-staged kernel.
template <bool CLAMP>
static qr_status dispatch_q8(const uint16_t* x, int64_t T, int32_t d, int64_t ld, int rot,
                             const int8_t* signs, float clip, int bits, uint8_t* q, uint16_t* sc,
                             float* z, hipStream_t st) {
  if (!rot)
    return launch_lds_t<1, MODE_QUANT8, CLAMP, false>(d, 0, x, T, ld, signs, 1.0f, clip, q, sc, z,
                                                      nullptr, st, bits);
  int n = 0, m = 0;
  if (!factor_width(d, &n, &m)) return QR_ERR_UNSUPPORTED;
  const float c = norm_constant(d);
  if (m == 1)
    return launch_lds_t<1, MODE_QUANT8, CLAMP, true>(d, n, x, T, ld, signs, c, clip, q, sc, z,
                                                     nullptr, st, bits);
  if (m == 28 && n == 10)
    return launch_k28<MODE_QUANT8, CLAMP, false>(x, T, ld, signs, c, clip, q, sc, z, nullptr, st,
                                                 bits);
  if (m == 28)
    return launch_lds_t<28, MODE_QUANT8, CLAMP, true>(d, n, x, T, ld, signs, c, clip, q, sc, z,
                                                      nullptr, st, bits);
  if (n == 6)
    return launch_k172<MODE_QUANT8, CLAMP, false>(x, T, ld, signs, c, clip, q, sc, z, nullptr, st,
                                                  bits);
  return launch_lds_t<172, MODE_QUANT8, CLAMP, true>(d, n, x, T, ld, signs, c, clip, q, sc, z,
                                                     nullptr, st, bits);
}

// Group-wise scales: every width through the LDS-staged kernel.
template <bool CLAMP>
static qr_status dispatch_groups(const uint16_t* x, int64_t T, int32_t d, int64_t ld, int rot,
                                 const int8_t* signs, float clip, int group, uint8_t* q,
                                 uint16_t* sc, float* z, hipStream_t st) {
  if (!rot)
    return launch_lds_t<1, MODE_QUANT_GROUPS, CLAMP, false>(d, 0, x, T, ld, signs, 1.0f, clip, q,
                                                            sc, z, nullptr, st, 4, group);
  int n = 0, m = 0;
  if (!factor_width(d, &n, &m)) return QR_ERR_UNSUPPORTED;
  const float c = norm_constant(d);
  if (m == 1)
    return launch_lds_t<1, MODE_QUANT_GROUPS, CLAMP, true>(d, n, x, T, ld, signs, c, clip, q, sc,
                                                           z, nullptr, st, 4, group);
  if (m == 28)
    return launch_lds_t<28, MODE_QUANT_GROUPS, CLAMP, true>(d, n, x, T, ld, signs, c, clip, q, sc,
                                                            z, nullptr, st, 4, group);
  return launch_lds_t<172, MODE_QUANT_GROUPS, CLAMP, true>(d, n, x, T, ld, signs, c, clip, q, sc,
                                                           z, nullptr, st, 4, group);
}

}  // namespace qr

using namespace qr;

extern "C" qr_status qr_hadamard_quant_groups(const void* x_f16, int64_t T, int32_t d,
                                              int64_t ld_x, qr_rot rot, const int8_t* signs,
                                              float clip_ratio, int32_t group, void* q_u8,
                                              void* scale_f16, float* z_dbg, hipStream_t stream) {
  if (T < 0 || d <= 0 || ld_x < d) return QR_ERR_SHAPE;
  if (rot != QR_ROT_NONE && rot != QR_ROT_HADAMARD) return QR_ERR_ARG;
  if (!valid_clip(clip_ratio)) return QR_ERR_ARG;
  if (group < 8 || group > 512 || (group & (group - 1)) || d % group) return QR_ERR_UNSUPPORTED;
  int n = 0, m = 0;
  if (rot != QR_ROT_NONE) {
    if (!factor_width(d, &n, &m)) return QR_ERR_UNSUPPORTED;
  } else if (d % 8 != 0 || d > 32768) {
    return QR_ERR_UNSUPPORTED;
  }
  if (T == 0) return QR_OK;
  if (!x_f16 || !q_u8 || !scale_f16) return QR_ERR_NULL;
  if (ld_x % 8 != 0 || !aligned(x_f16, 16) || !aligned(q_u8, 4) || !aligned(scale_f16, 2) ||
      (z_dbg && !aligned(z_dbg, 16)) || (signs && !aligned(signs, 4)))
    return QR_ERR_ALIGN;
  const int r = rot == QR_ROT_HADAMARD ? 1 : 0;
  const uint16_t* x = (const uint16_t*)x_f16;
  if (clip_ratio < 1.0f)
    return dispatch_groups<true>(x, T, d, ld_x, r, signs, clip_ratio, group, (uint8_t*)q_u8,
                                 (uint16_t*)scale_f16, z_dbg, stream);
  return dispatch_groups<false>(x, T, d, ld_x, r, signs, clip_ratio, group, (uint8_t*)q_u8,
                                (uint16_t*)scale_f16, z_dbg, stream);
}

extern "C" qr_status qr_hadamard_quant_i8(const void* x_f16, int64_t T, int32_t d, int64_t ld_x,
                                          qr_rot rot, const int8_t* signs, float clip_ratio,
                                          int32_t bits, void* q_i8, void* scale_f16, float* z_dbg,
                                          hipStream_t stream) {
  if (T < 0 || d <= 0 || ld_x < d) return QR_ERR_SHAPE;
  if (rot != QR_ROT_NONE && rot != QR_ROT_HADAMARD) return QR_ERR_ARG;
  if (!valid_clip(clip_ratio) || bits < 2 || bits > 8) return QR_ERR_ARG;
  int n = 0, m = 0;
  if (rot != QR_ROT_NONE) {
    if (!factor_width(d, &n, &m)) return QR_ERR_UNSUPPORTED;
  } else if (d % 8 != 0 || d > 32768) {
    return QR_ERR_UNSUPPORTED;
  }
  if (T == 0) return QR_OK;
  if (!x_f16 || !q_i8 || !scale_f16) return QR_ERR_NULL;
  if (ld_x % 8 != 0 || !aligned(x_f16, 16) || !aligned(q_i8, 8) || !aligned(scale_f16, 2) ||
      (z_dbg && !aligned(z_dbg, 16)) || (signs && !aligned(signs, 4)))
    return QR_ERR_ALIGN;
  const int r = rot == QR_ROT_HADAMARD ? 1 : 0;
  const uint16_t* x = (const uint16_t*)x_f16;
  if (clip_ratio < 1.0f)
    return dispatch_q8<true>(x, T, d, ld_x, r, signs, clip_ratio, bits, (uint8_t*)q_i8,
                             (uint16_t*)scale_f16, z_dbg, stream);
  return dispatch_q8<false>(x, T, d, ld_x, r, signs, clip_ratio, bits, (uint8_t*)q_i8,
                            (uint16_t*)scale_f16, z_dbg, stream);
}

extern "C" qr_status qr_hadamard_quant(const void* x_f16, int64_t T, int32_t d, int64_t ld_x,
                                       qr_rot rot, const int8_t* signs, float clip_ratio,
                                       void* q_u8, void* scale_f16, float* z_dbg,
                                       hipStream_t stream) {
  if (T < 0 || d <= 0 || ld_x < d) return QR_ERR_SHAPE;
  if (rot != QR_ROT_NONE && rot != QR_ROT_HADAMARD && rot != QR_ROT_HADAMARD_F16) return QR_ERR_ARG;
  if (!valid_clip(clip_ratio)) return QR_ERR_ARG;
  int n = 0, m = 0;
  if (rot != QR_ROT_NONE) {
    if (!factor_width(d, &n, &m)) return QR_ERR_UNSUPPORTED;
    // the fp16 transform exists for the down-projection widths of the configurations
    if (rot == QR_ROT_HADAMARD_F16 && !((m == 28 && n == 10) || (m == 172 && n == 6)))
      return QR_ERR_UNSUPPORTED;
  } else if (d % 8 != 0 || d > 32768) {
    return QR_ERR_UNSUPPORTED;
  }
  if (T == 0) return QR_OK;
  if (!x_f16 || !q_u8 || !scale_f16) return QR_ERR_NULL;
  if (ld_x % 8 != 0 || !aligned(x_f16, 16) || !aligned(q_u8, 4) || !aligned(scale_f16, 2) ||
      (z_dbg && !aligned(z_dbg, 16)) || (signs && !aligned(signs, 4)))
    return QR_ERR_ALIGN;
  if (rot == QR_ROT_HADAMARD_F16) {
    const float c = norm_constant(d);
    const uint16_t* xx = (const uint16_t*)x_f16;
    uint8_t* qq = (uint8_t*)q_u8;
    uint16_t* ss = (uint16_t*)scale_f16;
    if (m == 28)
      return clip_ratio < 1.0f
                 ? launch_k28<MODE_QUANT, true, true>(xx, T, ld_x, signs, c, clip_ratio, qq, ss,
                                                      z_dbg, nullptr, stream)
                 : launch_k28<MODE_QUANT, false, true>(xx, T, ld_x, signs, c, clip_ratio, qq, ss,
                                                       z_dbg, nullptr, stream);
    return clip_ratio < 1.0f
               ? launch_k172<MODE_QUANT, true, true>(xx, T, ld_x, signs, c, clip_ratio, qq, ss,
                                                     z_dbg, nullptr, stream)
               : launch_k172<MODE_QUANT, false, true>(xx, T, ld_x, signs, c, clip_ratio, qq, ss,
                                                      z_dbg, nullptr, stream);
  }
  const int r = rot == QR_ROT_HADAMARD ? 1 : 0;
  if (clip_ratio < 1.0f)
    return dispatch<MODE_QUANT, true>(x_f16, T, d, ld_x, r, signs, clip_ratio, q_u8, scale_f16,
                                      z_dbg, nullptr, stream);
  return dispatch<MODE_QUANT, false>(x_f16, T, d, ld_x, r, signs, clip_ratio, q_u8, scale_f16,
                                     z_dbg, nullptr, stream);
}

extern "C" qr_status qr_hadamard(const void* x_f16, int64_t T, int32_t d, int64_t ld_x,
                                 const int8_t* signs, void* y, int32_t y_is_f32,
                                 hipStream_t stream) {
  if (T < 0 || d <= 0 || ld_x < d) return QR_ERR_SHAPE;
  int n = 0, m = 0;
  if (!factor_width(d, &n, &m)) return QR_ERR_UNSUPPORTED;
  if (T == 0) return QR_OK;
  if (!x_f16 || !y) return QR_ERR_NULL;
  if (ld_x % 8 != 0 || !aligned(x_f16, 16) || !aligned(y, 16) || (signs && !aligned(signs, 4)))
    return QR_ERR_ALIGN;
  if (y_is_f32)
    return dispatch<MODE_ROT_F32, false>(x_f16, T, d, ld_x, 1, signs, 1.0f, nullptr, nullptr,
                                         nullptr, y, stream);
  return dispatch<MODE_ROT_F16, false>(x_f16, T, d, ld_x, 1, signs, 1.0f, nullptr, nullptr,
                                       nullptr, y, stream);
}
