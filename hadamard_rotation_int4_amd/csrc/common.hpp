// Shared definitions for the gfx950 kernels of libquarot_hip.so.
//
// The non-power-of-two Hadamard factors are generated here at compile time
// from their published constructions (QuaRot paper, background on Hadamard
// matrices: H_d = H_{2^n} (x) H_m with m the order of a known Hadamard matrix):
//   * H_28: Paley's second construction over GF(13) -- Jacobsthal matrix
//     Q[i][j] = chi(j - i), symmetric conference matrix C = [[0, 1^T], [1, Q]],
//     H = C (x) [[1, 1], [1, -1]] + I (x) [[1, -1], [-1, -1]];
//   * H_172: Williamson's array [[A, B, C, D], [-B, A, -D, C], [-C, D, A, -B],
//     [-D, -C, B, A]] of four symmetric circulant +-1 matrices of order 43
//     (X[i][j] = x[(j - i) mod 43]) whose squares sum to 172 I.  The four first
//     rows below were found by a meet-in-the-middle search over sequences fixed
//     by the order-6 multiplier subgroup of Z_43^* (row sums 5, 7, 7, 7).
// Any matrix with H H^T = m I is a valid choice; these conventions fix which.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qr.h"

namespace qr {

// ---------------------------------------------------------------------------
// Vector types
// ---------------------------------------------------------------------------
typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
// 16 bytes at 4-byte alignment, for outputs whose contract promises only dword alignment
typedef uint32_t v4u_a4 __attribute__((ext_vector_type(4), aligned(4)));

// fp32 value 1.5 * 2^23: fma(z, m, kMagic) = kMagic + round_half_even(z * m)
// exactly (one rounding of the exact product) whenever |z * m| < 2^22, and the
// integer then sits in the low mantissa bits of the result.
constexpr float kMagic = 12582912.0f;
constexpr uint32_t kMagicBits = 0x4B400000u;

__device__ __forceinline__ float h2f(uint16_t h) {
  return __half2float(__ushort_as_half(h));
}
// fp32 -> fp16, round half to even, of the fp32 value f.  The empty asm makes
// f opaque: without it the compiler fuses a producing fp32 multiply and this
// conversion into one v_fma_mix*_f16, which rounds the exact product once to
// fp16 and differs from the two-step rounding at exact fp16 ties.
__device__ __forceinline__ uint16_t f2h(float f) {
  asm("" : "+v"(f));
  return __half_as_ushort(__float2half_rn(f));
}

// ---------------------------------------------------------------------------
// Compile-time Hadamard factor tables (+1.0f / -1.0f)
// ---------------------------------------------------------------------------
template <int M>
struct HTable {
  float v[M][M];
};

constexpr int legendre13(int a) {
  a %= 13;
  if (a < 0) a += 13;
  if (a == 0) return 0;
  // quadratic residues mod 13: 1, 3, 4, 9, 10, 12
  return (a == 1 || a == 3 || a == 4 || a == 9 || a == 10 || a == 12) ? 1 : -1;
}

constexpr HTable<28> make_h28() {
  HTable<28> t{};
  for (int bi = 0; bi < 14; ++bi)
    for (int bj = 0; bj < 14; ++bj) {
      int c = 0;  // conference matrix entry
      if (bi == 0 && bj == 0) c = 0;
      else if (bi == 0 || bj == 0) c = 1;
      else c = legendre13((bj - 1) - (bi - 1));
      // C (x) [[1, 1], [1, -1]]
      int e00 = c, e01 = c, e10 = c, e11 = -c;
      if (bi == bj) {  // + I (x) [[1, -1], [-1, -1]]
        e00 += 1;
        e01 -= 1;
        e10 -= 1;
        e11 -= 1;
      }
      t.v[2 * bi][2 * bj] = (float)e00;
      t.v[2 * bi][2 * bj + 1] = (float)e01;
      t.v[2 * bi + 1][2 * bj] = (float)e10;
      t.v[2 * bi + 1][2 * bj + 1] = (float)e11;
    }
  return t;
}

// First rows of the Williamson matrices A, B, C, D ('+' = +1, '-' = -1).
constexpr const char* kWill43[4] = {
    "--+-+----++++-++++-++--++-++++-++++----+-+-",
    "++---+++++++-+--++--+--+--++--+-+++++++---+",
    "+--+++--++-+-+-+--++++++++--+-+-+-++--+++--",
    "++++--++-+-++-+---+-++++-+---+-++-+-++--+++",
};

constexpr HTable<172> make_h172() {
  HTable<172> t{};
  // block (I, J) of the Williamson array: sign * circulant(which)
  const int which[4][4] = {{0, 1, 2, 3}, {1, 0, 3, 2}, {2, 3, 0, 1}, {3, 2, 1, 0}};
  const int sign[4][4] = {{1, 1, 1, 1}, {-1, 1, -1, 1}, {-1, 1, 1, -1}, {-1, -1, 1, 1}};
  for (int bi = 0; bi < 4; ++bi)
    for (int bj = 0; bj < 4; ++bj)
      for (int i = 0; i < 43; ++i)
        for (int j = 0; j < 43; ++j) {
          int idx = ((j - i) % 43 + 43) % 43;
          int e = kWill43[which[bi][bj]][idx] == '+' ? 1 : -1;
          t.v[bi * 43 + i][bj * 43 + j] = (float)(sign[bi][bj] * e);
        }
  return t;
}

// ---------------------------------------------------------------------------
// Host helpers
// ---------------------------------------------------------------------------
inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// d = 2^n * m with m in {1, 28, 172}; returns false if unsupported.
inline bool factor_width(int32_t d, int* n, int* m) {
  if (d <= 0) return false;
  const int ms[3] = {1, 28, 172};
  for (int mi = 0; mi < 3; ++mi) {
    int mm = ms[mi];
    if (d % mm) continue;
    int r = d / mm;
    if (r & (r - 1)) continue;
    int nn = 0;
    while ((1 << nn) < r) ++nn;
    if (mm == 1 && (nn < 3 || nn > 13)) return false;
    if (mm == 28 && (nn < 1 || nn > 10)) return false;   // row staged in LDS: d <= 28672
    if (mm == 172 && (nn < 1 || nn > 6)) return false;   // two LDS buffers: d <= 11008
    *n = nn;
    *m = mm;
    return true;
  }
  return false;
}

inline bool valid_clip(float c) { return c >= (1.0f / 1024.0f) && c <= 1.0f; }

inline qr_status launch_status() {
  return hipGetLastError() == hipSuccess ? QR_OK : QR_ERR_LAUNCH;
}

// fp32 rounding of the fp64 value 1/sqrt(d): the normalisation constant c.
float norm_constant(int32_t d);

}  // namespace qr
