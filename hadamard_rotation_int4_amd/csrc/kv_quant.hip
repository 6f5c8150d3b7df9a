// Head-wise Hadamard rotation of new K (or V) tokens fused with asymmetric
// 4-bit group quantization, written straight into the packed KV cache
// (qr_kv_rotate_quant), for gfx950.
//
// QuaRot paper: keys (and queries) get an online head-wise Hadamard after the
// positional embedding so q.k is unchanged (keys/queries paragraph, post-RoPE
// caching); the cache is quantized asymmetrically in groups of 128 with a
// clipping ratio of 0.95 (implementation paragraph; Table 6); Init fills the
// cache from the prompt and Append quantizes one new token per decode step
// (attention-routines paragraph).  The exact fp32 recipe is in include/qr.h.
//
// Dh = 128 with group 128 (the pages' configuration) runs k_kv_quant128: the
// head-wise H_128 on the matrix cores, 16 rows per wavefront tile.  Other
// shapes run k_kv_quant:
// one (token, head) row of Dh elements is spread over Dh/8 lanes, each
// lane loading 8 contiguous fp16 (16 bytes).  Three butterfly stages run inside
// the lane, log2(Dh/8) across lanes.  Group min/max reduce over the G/8 lanes
// of a group; each lane then writes one dword of codes and the first lane of a
// group writes its (scale, min) pair.  The kernel is HBM-bound: per element it
// reads 2 bytes and writes 0.5 byte plus 4 bytes of metadata per group.
#include "common.hpp"
#include "dpp.hpp"

namespace qr {

// n / d for 0 <= n < 2^31 with a host-computed multiplier:
// q = (umulhi(n, m) + n) >> s with s = ceil(log2 d), m = floor(2^32 (2^s - d) / d) + 1.
struct FastDiv {
  uint32_t d, m, s;
};
static FastDiv make_fastdiv(uint32_t d) {
  FastDiv f;
  f.d = d;
  f.s = 0;
  while ((1ull << f.s) < d) ++f.s;
  f.m = (uint32_t)((((1ull << 32) * ((1ull << f.s) - d)) / d + 1) & 0xffffffffull);
  return f;
}
__device__ __forceinline__ uint32_t fast_div(uint32_t n, const FastDiv& f) {
  return (__umulhi(n, f.m) + n) >> f.s;
}

// Max / min over the 16 lanes of a DPP row (quad_perm [1,0,3,2] and [2,3,0,1],
// row_half_mirror, row_mirror).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL,
                                                            0xF, 0xF, false));
}
#define QR_ROW16(OP, v)                   \
  do {                                    \
    v = OP(v, dpp_f<0xB1>(v));            \
    v = OP(v, dpp_f<0x4E>(v));            \
    v = OP(v, dpp_f<0x141>(v));           \
    v = OP(v, dpp_f<0x140>(v));           \
  } while (0)

template <int LPR, bool ROT>
__global__ __launch_bounds__(256) void k_kv_quant(
    const uint16_t* __restrict__ x, int64_t rows, int S_new, int H, int64_t ld_token,
    const int8_t* __restrict__ signs, int group, float c, float clip, float levels,
    uint8_t* __restrict__ cq, uint16_t* __restrict__ meta, int S_max, int start_pos,
    float* __restrict__ zdbg, FastDiv fdH, FastDiv fdS) {
  constexpr int DH = LPR * 8;
  constexpr int RPW = 64 / LPR;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int sub = lane % LPR;
  const int rw = lane / LPR;
  const int lpg = group / 8;  // lanes per group
  const int ngroups = DH / group;
  // With 16 lanes per row and one group per row the lane holds chunk
  // gmap(sub) and both the butterflies and the min / max run through DPP
  // inside the 16-lane row; the lane then holds sigma * z.  Otherwise chunk
  // sub and lane shuffles.
  const bool dpp = LPR == 16 && group == DH;
  const int gc = dpp ? gmap(sub) : sub;
  const int coff = gc * 8;
  const float sigma = (ROT && dpp && (__builtin_popcount(gc) & 1)) ? -1.0f : 1.0f;
  float sg[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) sg[j] = 1.0f;
  if (ROT && signs) {
    const uint32_t w0 = *(const uint32_t*)(signs + coff), w1 = *(const uint32_t*)(signs + coff + 4);
#pragma unroll
    for (int j = 0; j < 8; ++j) sg[j] = (((j < 4 ? w0 : w1) >> (8 * (j & 3) + 7)) & 1u) ? -1.0f : 1.0f;
  }

  for (int64_t base = ((int64_t)blockIdx.x * 4 + wave) * RPW; base < rows;
       base += (int64_t)gridDim.x * 4 * RPW) {
    const int64_t row = base + rw;  // row = (b * S_new + s) * H + h
    const bool valid = row < rows;
    const uint32_t tok = fast_div((uint32_t)row, fdH);
    const int h = (int)((uint32_t)row - tok * (uint32_t)H);
    float v[8];
    if (valid) {
      const v4u raw = *(const v4u*)(x + (int64_t)tok * ld_token + (int64_t)h * DH + coff);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[2 * j] = h2f((uint16_t)(raw[j] & 0xffffu)) * sg[2 * j];
        v[2 * j + 1] = h2f((uint16_t)(raw[j] >> 16)) * sg[2 * j + 1];
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = 0.0f;
    }
    if (ROT) {
#pragma unroll
      for (int hh = 1; hh < 8; hh <<= 1)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (!(j & hh)) {
            const float a = v[j], b = v[j + hh];
            v[j] = a + b;
            v[j + hh] = a - b;
          }
      if (LPR == 16 && dpp) {
        const float s0 = (gc & 1) ? -1.0f : 1.0f, s1 = (gc & 2) ? -1.0f : 1.0f;
        const float s2 = (gc & 4) ? -1.0f : 1.0f, s3 = (gc & 8) ? -1.0f : 1.0f;
        QR_DPP8("quad_perm:[1,0,3,2]", v, s0);
        QR_DPP8("quad_perm:[2,3,0,1]", v, s1);
        QR_DPP8("row_half_mirror", v, s2);
        QR_DPP8("row_mirror", v, s3);
      } else {
#pragma unroll
        for (int hh = 1; hh < LPR; hh <<= 1) {
          const float s = (sub & hh) ? -1.0f : 1.0f;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float p = __shfl_xor(v[j], hh);
            v[j] = fmaf(v[j], s, p);
          }
        }
      }
    }
    if (valid && zdbg) {
      float* zr = zdbg + row * DH + coff;
      *(v4f*)zr = v4f{v[0] * sigma, v[1] * sigma, v[2] * sigma, v[3] * sigma};
      *(v4f*)(zr + 4) = v4f{v[4] * sigma, v[5] * sigma, v[6] * sigma, v[7] * sigma};
    }
    // y = fp32(z * c) (= sigma * fp32(v * c) exactly)
    const float cs = c * sigma;
    float y[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) y[j] = ROT ? __fmul_rn(v[j], cs) : v[j];
    float mx = y[0], mn = y[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) {
      mx = fmaxf(mx, y[j]);
      mn = fminf(mn, y[j]);
    }
    if (LPR == 16 && dpp) {
      QR_ROW16(fmaxf, mx);
      QR_ROW16(fminf, mn);
    } else {
      for (int hh = 1; hh < lpg; hh <<= 1) {
        mx = fmaxf(mx, __shfl_xor(mx, hh));
        mn = fminf(mn, __shfl_xor(mn, hh));
      }
    }
    const float mxc = __fmul_rn(clip, mx);
    const float mnc = __fmul_rn(clip, mn);
    const uint16_t sh = f2h(__fdiv_rn(__fsub_rn(mxc, mnc), levels));
    const uint16_t mh = f2h(mnc);
    const float shf = h2f(sh);
    const float mhf = h2f(mh);
    const float inv = shf > 0.0f ? __fdiv_rn(1.0f, shf) : 0.0f;
    uint32_t f[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      // kMagic + rne((y - m_h) * inv), clamped to [0, levels].  The clamp is
      // needed even without clipping: m_h is mn rounded to fp16 and s_h is
      // rounded too.
      float t = fmaf(__fsub_rn(y[j], mhf), inv, kMagic);
      t = __builtin_amdgcn_fmed3f(t, kMagic, kMagic + levels);
      f[j] = __float_as_uint(t);
    }
    const uint32_t p0 = (f[1] << 4) | (f[0] & 0xfu);
    const uint32_t p1 = (f[3] << 4) | (f[2] & 0xfu);
    const uint32_t p2 = (f[5] << 4) | (f[4] & 0xfu);
    const uint32_t p3 = (f[7] << 4) | (f[6] & 0xfu);
    const uint32_t word = __builtin_amdgcn_perm(p1, p0, 0x0c0c0400u) |
                          __builtin_amdgcn_perm(p3, p2, 0x04000c0cu);
    if (valid) {
      const int64_t b = fast_div(tok, fdS);
      const int s = (int)(tok - (uint32_t)b * (uint32_t)S_new);
      const int64_t crow = (b * H + h) * (int64_t)S_max + start_pos + s;
      *(uint32_t*)(cq + crow * (DH / 2) + coff / 2) = word;
      if ((gc % lpg) == 0) {
        const int gi = gc / lpg;
        *(uint32_t*)(meta + (crow * ngroups + gi) * 2) = (uint32_t)sh | ((uint32_t)mh << 16);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Dh = 128 with one group per row (the pages' configuration): 16 (token, head)
// rows per wavefront tile, H_128 on the matrix cores.
// ---------------------------------------------------------------------------
// Every row shares the sign vector s, so diag(s) folds into constant A
// fragments: z = H_128 diag(s) x with H_128 = H_4 (x) H_32.  As in k_hq_pow2,
// each of the four 32-element output blocks h is a chain of four
// v_mfma_f32_16x16x32_f16, one per input block kb, on the fp16 input as
// loaded (B column n = row n of the tile, lane (n, g) holding elements
// 32 kb + 8 g .. + 7); the H_32 rows of the A fragments are permuted so that
// lane (n, g) receives outputs 32 h + 8 g .. + 7, and the H_4 sign (-1)^|h & kb|
// picks a negated copy.  Products are +-x and the accumulation fp32, as in the
// butterfly form.  Per element the vector units then only scale, reduce,
// round and pack.  Without rotation the same lane layout holds the input.
// The codes of a row leave as one 64-byte piece: a 4 x 4 transpose across the
// row's four lanes gives each lane 16 contiguous bytes.
// Workgroups of the Dh = 128 kernel: about four 16-row tiles per wavefront at the
// 70B Init shape, so that each wavefront's next tile is in flight (one tile per
// wavefront measured 25% slower).
constexpr int KV128_GRID_CAP = 2048;
template <bool ROT>
__global__ __launch_bounds__(256) void k_kv_quant128(
    const uint16_t* __restrict__ x, int64_t rows, int S_new, int H, int64_t ld_token,
    const int8_t* __restrict__ signs, float c, float clip, float levels, uint8_t* __restrict__ cq,
    uint16_t* __restrict__ meta, int S_max, int start_pos, float* __restrict__ zdbg, FastDiv fdH,
    FastDiv fdS) {
  constexpr int DH = 128;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;

  // A fragments of H_32 diag(s_kb) (row i = n -> output o = 8 (i >> 2) + 4 m + (i & 3),
  // columns k = 8 g + j of block kb) and their negations.
  v8h ap[4][2], an[4][2];
  if constexpr (ROT) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      uint32_t sw0 = 0u, sw1 = 0u;  // int8 signs of elements 32 kb + 8 g .. + 7
      if (signs) {
        sw0 = *(const uint32_t*)(signs + 32 * kb + 8 * g);
        sw1 = *(const uint32_t*)(signs + 32 * kb + 8 * g + 4);
      }
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int o = 8 * (n >> 2) + 4 * m + (n & 3);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int k = 8 * g + j;
          const bool neg_s = (((j < 4 ? sw0 : sw1) >> (8 * (j & 3) + 7)) & 1u) != 0u;
          const bool neg = ((__builtin_popcount(o & k) & 1) != 0) != neg_s;
          ap[kb][m][j] = neg ? (_Float16)-1.0f : (_Float16)1.0f;
        }
        an[kb][m] = -ap[kb][m];
      }
    }
  }

  const int64_t ntiles = (rows + 15) / 16;
  const int64_t tstride = (int64_t)gridDim.x * 4;
  // Rows in input order, r = (b S_new + s) H + h: a tile reads 4 KB of
  // contiguous input (walking the rows in cache order instead, so that a
  // tile's codes land contiguously, measured slower: the input is 4x the bytes).
  struct RowIx {
    uint32_t tok;   // b S_new + s: the input token
    int h, s;
    int64_t bh;     // b H + h
  };
  auto row_ix = [&](int64_t r) {
    RowIx ix;
    ix.tok = fast_div((uint32_t)r, fdH);
    ix.h = (int)((uint32_t)r - ix.tok * (uint32_t)H);
    const uint32_t b = fast_div(ix.tok, fdS);
    ix.s = (int)(ix.tok - b * (uint32_t)S_new);
    ix.bh = (int64_t)b * H + ix.h;
    return ix;
  };
  // B fragments of a tile: row tile * 16 + n, elements 32 kb + 8 g .. + 7
  auto load = [&](int64_t tile, v4u* b) {
    const int64_t row = tile * 16 + n;
    if (tile < ntiles && row < rows) {
      const RowIx ix = row_ix(row);
      const uint16_t* xr = x + (int64_t)ix.tok * ld_token + (int64_t)ix.h * DH + 8 * g;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)  // read once: non-temporal
        b[kb] = __builtin_nontemporal_load((const v4u*)(xr + 32 * kb));
    } else {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) b[kb] = v4u{0u, 0u, 0u, 0u};
    }
  };
  int64_t tile = (int64_t)blockIdx.x * 4 + wave;
  v4u bcur[4], bnext[4];
  load(tile, bcur);
  for (; tile < ntiles; tile += tstride) {
    load(tile + tstride, bnext);
    const int64_t row = tile * 16 + n;
    const bool valid = row < rows;
    // z[h][j]: element 32 h + 8 g + j of row n
    float z[4][8];
    if constexpr (ROT) {
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        v4f r0 = {0.0f, 0.0f, 0.0f, 0.0f}, r1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const v8h bv = __builtin_bit_cast(v8h, bcur[kb]);
          const bool neg = __builtin_popcount(h & kb) & 1;
          r0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(neg ? an[kb][0] : ap[kb][0], bv, r0, 0, 0, 0);
          r1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(neg ? an[kb][1] : ap[kb][1], bv, r1, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          z[h][r] = r0[r];
          z[h][4 + r] = r1[r];
        }
      }
    } else {
#pragma unroll
      for (int h = 0; h < 4; ++h)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          z[h][2 * j] = h2f((uint16_t)(bcur[h][j] & 0xffffu));
          z[h][2 * j + 1] = h2f((uint16_t)(bcur[h][j] >> 16));
        }
    }
    const RowIx ix = row_ix(valid ? row : 0);
    if (valid && zdbg) {  // z_dbg is token-major, like the input
      float* zr = zdbg + ((int64_t)ix.tok * H + ix.h) * DH + 8 * g;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        *(v4f*)(zr + 32 * h) = v4f{z[h][0], z[h][1], z[h][2], z[h][3]};
        *(v4f*)(zr + 32 * h + 4) = v4f{z[h][4], z[h][5], z[h][6], z[h][7]};
      }
    }
    // y = fp32(z * c) (the input itself without rotation); max / min of the row
    float mx = -INFINITY, mn = INFINITY;
#pragma unroll
    for (int h = 0; h < 4; ++h)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (ROT) z[h][j] = __fmul_rn(z[h][j], c);
        mx = fmaxf(mx, z[h][j]);
        mn = fminf(mn, z[h][j]);
      }
    // the row's four lanes are n, n + 16, n + 32, n + 48
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mn = fminf(mn, __shfl_xor(mn, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    mn = fminf(mn, __shfl_xor(mn, 32));
    const float mxc = __fmul_rn(clip, mx);
    const float mnc = __fmul_rn(clip, mn);
    const uint16_t sh = f2h(__fdiv_rn(__fsub_rn(mxc, mnc), levels));
    const uint16_t mh = f2h(mnc);
    const float shf = h2f(sh);
    const float mhf = h2f(mh);
    const float inv = shf > 0.0f ? __fdiv_rn(1.0f, shf) : 0.0f;
    // Code word h of lane (n, g) holds elements 32 h + 8 g .. + 7, bytes 16 h + 4 g of
    // the row's 64.  A 4 x 4 transpose over the row's four lanes (g) and words (h)
    // gives lane g bytes 16 g .. + 15, so each row is one 64-byte piece of a single
    // store instruction (four 4-byte stores per lane cost 11% more time at the 70B
    // Init shape).
    uint32_t wd[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      uint32_t f[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        // kMagic + rne((y - m_h) * inv), clamped to [0, levels] (m_h and s_h
        // are rounded to fp16, so the clamp is needed even without clipping)
        float t = fmaf(__fsub_rn(z[h][j], mhf), inv, kMagic);
        t = __builtin_amdgcn_fmed3f(t, kMagic, kMagic + levels);
        f[j] = __float_as_uint(t);
      }
      const uint32_t p0 = (f[1] << 4) | (f[0] & 0xfu);
      const uint32_t p1 = (f[3] << 4) | (f[2] & 0xfu);
      const uint32_t p2 = (f[5] << 4) | (f[4] & 0xfu);
      const uint32_t p3 = (f[7] << 4) | (f[6] & 0xfu);
      wd[h] = __builtin_amdgcn_perm(p1, p0, 0x0c0c0400u) | __builtin_amdgcn_perm(p3, p2, 0x04000c0cu);
    }
    {
      // v_permlane32_swap(a, b) exchanges a of lanes 32..63 with b of lanes 0..31:
      // lanes g < 2 give words 2, 3 for the upper lanes' words 0, 1.
      // v_permlane16_swap(a, b) exchanges a of the odd 16-lane rows with b of the
      // even ones: even g give word 1 (3) for the odd neighbour's word 0 (2).
      const auto s0 = __builtin_amdgcn_permlane32_swap(wd[0], wd[2], false, false);
      const auto s1 = __builtin_amdgcn_permlane32_swap(wd[1], wd[3], false, false);
      wd[0] = s0[0];
      wd[2] = s0[1];
      wd[1] = s1[0];
      wd[3] = s1[1];
      const auto t0 = __builtin_amdgcn_permlane16_swap(wd[0], wd[1], false, false);
      const auto t1 = __builtin_amdgcn_permlane16_swap(wd[2], wd[3], false, false);
      wd[0] = t0[0];
      wd[1] = t0[1];
      wd[2] = t1[0];
      wd[3] = t1[1];
    }
    if (valid) {
      const int64_t crow = ix.bh * (int64_t)S_max + start_pos + ix.s;
      // cache_q is only required to be 4-byte aligned: a dword-aligned vector type
      __builtin_nontemporal_store(v4u_a4{wd[0], wd[1], wd[2], wd[3]},
                                  (v4u_a4*)(cq + crow * (DH / 2) + 16 * g));
      // (scale, min) pairs as plain stores: 4-byte pieces the L2 merges into lines
      // (non-temporal was slower)
      if (g == 0) *(uint32_t*)(meta + crow * 2) = (uint32_t)sh | ((uint32_t)mh << 16);
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) bcur[kb] = bnext[kb];
  }
}

template <bool ROT>
static qr_status launch_kv(int dh, const uint16_t* x, int64_t rows, int S_new, int H,
                           int64_t ld_token, const int8_t* signs, int group, float c, float clip,
                           float levels, uint8_t* cq, uint16_t* meta, int S_max, int start_pos,
                           float* zdbg, hipStream_t st) {
  if (dh == 128 && group == 128) {
    const int64_t tiles = (rows + 15) / 16;
    int64_t grid = (tiles + 3) / 4;
    if (grid > KV128_GRID_CAP) grid = KV128_GRID_CAP;
    hipLaunchKernelGGL((k_kv_quant128<ROT>), dim3((int)grid), dim3(256), 0, st, x, rows, S_new,
                       H, ld_token, signs, c, clip, levels, cq, meta, S_max, start_pos, zdbg,
                       make_fastdiv((uint32_t)H), make_fastdiv((uint32_t)S_new));
    return launch_status();
  }
  const int lpr = dh / 8;
  const int64_t rows_per_block = 4 * (64 / lpr);
  int64_t grid = (rows + rows_per_block - 1) / rows_per_block;
  if (grid > 8192) grid = 8192;
  switch (lpr) {
#define QR_CASE(L)                                                                              \
  case L:                                                                                       \
    hipLaunchKernelGGL((k_kv_quant<L, ROT>), dim3((int)grid), dim3(256), 0, st, x, rows, \
                       S_new, H, ld_token, signs, group, c, clip, levels, cq, meta, S_max,      \
                       start_pos,                                                               \
                       zdbg, make_fastdiv((uint32_t)H), make_fastdiv((uint32_t)S_new));         \
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

static qr_status kv_entry(const void* kv_f16, int32_t B, int32_t S_new, int32_t H, int32_t Dh,
                          int64_t ld_token, qr_rot rot, const int8_t* signs, int32_t group,
                          float clip_ratio, int32_t bits, void* cache_q, void* cache_meta,
                          int32_t S_max, int32_t start_pos, float* z_dbg, hipStream_t stream) {
  if (B < 1 || H < 1 || S_new < 0 || S_max < 0 || start_pos < 0) return QR_ERR_SHAPE;
  if ((int64_t)start_pos + S_new > S_max) return QR_ERR_SHAPE;
  if (Dh < 8 || Dh > 256 || (Dh & (Dh - 1))) return QR_ERR_UNSUPPORTED;
  if (group < 8 || group > Dh || Dh % group != 0 || (group & (group - 1))) return QR_ERR_UNSUPPORTED;
  if (ld_token < (int64_t)H * Dh) return QR_ERR_SHAPE;
  if (rot != QR_ROT_NONE && rot != QR_ROT_HADAMARD) return QR_ERR_ARG;
  if (!valid_clip(clip_ratio) || bits < 2 || bits > 4) return QR_ERR_ARG;
  if (S_new == 0) return QR_OK;
  if (!kv_f16 || !cache_q || !cache_meta) return QR_ERR_NULL;
  if (ld_token % 8 != 0 || !aligned(kv_f16, 16) || !aligned(cache_q, 4) ||
      !aligned(cache_meta, 4) || (z_dbg && !aligned(z_dbg, 16)) ||
      (rot == QR_ROT_HADAMARD && signs && !aligned(signs, 4)))
    return QR_ERR_ALIGN;
  const int64_t rows = (int64_t)B * S_new * H;
  if (rows > INT32_MAX) return QR_ERR_SHAPE;
  const uint16_t* x = (const uint16_t*)kv_f16;
  uint8_t* cq = (uint8_t*)cache_q;
  uint16_t* meta = (uint16_t*)cache_meta;
  const float levels = (float)((1 << bits) - 1);
  if (rot == QR_ROT_HADAMARD)
    return launch_kv<true>(Dh, x, rows, S_new, H, ld_token, signs, group, norm_constant(Dh),
                           clip_ratio, levels, cq, meta, S_max, start_pos, z_dbg, stream);
  return launch_kv<false>(Dh, x, rows, S_new, H, ld_token, signs, group, 1.0f, clip_ratio, levels,
                          cq, meta, S_max, start_pos, z_dbg, stream);
}

}  // namespace qr

using namespace qr;

extern "C" qr_status qr_kv_rotate_quant(const void* kv_f16, int32_t B, int32_t S_new, int32_t H,
                                        int32_t Dh, int64_t ld_token, qr_rot rot,
                                        const int8_t* signs, int32_t group, float clip_ratio,
                                        void* cache_q, void* cache_meta, int32_t S_max,
                                        int32_t start_pos, float* z_dbg, hipStream_t stream) {
  return kv_entry(kv_f16, B, S_new, H, Dh, ld_token, rot, signs, group, clip_ratio, 4, cache_q,
                  cache_meta, S_max, start_pos, z_dbg, stream);
}

extern "C" qr_status qr_kv_rotate_quant_bits(const void* kv_f16, int32_t B, int32_t S_new,
                                             int32_t H, int32_t Dh, int64_t ld_token, qr_rot rot,
                                             const int8_t* signs, int32_t group, float clip_ratio,
                                             int32_t bits, void* cache_q, void* cache_meta,
                                             int32_t S_max, int32_t start_pos, float* z_dbg,
                                             hipStream_t stream) {
  return kv_entry(kv_f16, B, S_new, H, Dh, ld_token, rot, signs, group, clip_ratio, bits, cache_q,
                  cache_meta, S_max, start_pos, z_dbg, stream);
}
