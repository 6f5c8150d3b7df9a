// Cross-lane butterfly pieces shared by the rotation kernels of
// libquarot_hip.so: the lane-to-chunk map under which each DPP pattern of a
// 16-lane row flips exactly one chunk-index bit, and one butterfly stage
// (r += dpp(r) * s) over eight registers.
#pragma once

namespace qr {

// Lane-in-row c (0..15) -> chunk index.  Linear over GF(2) with gmap(1) = 1,
// gmap(2) = 2, gmap(7) = 4, gmap(15) = 8, so that the DPP partner patterns
// xor 1 (quad_perm), xor 2 (quad_perm), xor 7 (row_half_mirror) and xor 15
// (row_mirror) each flip exactly one chunk bit.
__device__ __forceinline__ int gmap(int c) {
  const int c0 = c & 1, c1 = (c >> 1) & 1, c2 = (c >> 2) & 1, c3 = (c >> 3) & 1;
  return (c0 ^ c2) | ((c1 ^ c2) << 1) | ((c2 ^ c3) << 2) | (c3 << 3);
}

// One butterfly stage across lanes for eight registers: r += dpp(r) * s.
// The leading s_nop covers the VALU-write -> DPP-read hazard for values
// produced just before; within the block every register is distinct.
#define QR_DPP8(CTRL, r, s)                                                            \
  asm volatile(                                                                        \
      "s_nop 1\n\t"                                                                    \
      "v_fmac_f32_dpp %0, %0, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"              \
      "v_fmac_f32_dpp %1, %1, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"              \
      "v_fmac_f32_dpp %2, %2, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"              \
      "v_fmac_f32_dpp %3, %3, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"              \
      "v_fmac_f32_dpp %4, %4, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"              \
      "v_fmac_f32_dpp %5, %5, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"              \
      "v_fmac_f32_dpp %6, %6, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"              \
      "v_fmac_f32_dpp %7, %7, %8 " CTRL " row_mask:0xf bank_mask:0xf"                  \
      : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]), "+v"(r[4]), "+v"(r[5]), "+v"(r[6]), \
        "+v"(r[7])                                                                     \
      : "v"(s))

}  // namespace qr
