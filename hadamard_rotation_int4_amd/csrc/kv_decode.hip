// Decode routine: attention of one new query per sequence over the 4-bit
// K/V cache (qr_kv_decode_attention), for gfx950.
//
// What is computed (QuaRot paper, attention paragraph and its attention
// routines Init / Append / Decode): for batch b, query head hq and its KV head
// h = hq / (Hq / Hkv), over cache positions j < L,
//   k_j = code * scale + min, v_j likewise (asymmetric 4-bit, one group per head),
//   s_j = softmax_scale * q . k_j,   o = sum_j softmax(s)_j v_j.
// The query arrives in fp16 and rotated like the keys, so q . k is the score of
// the unrotated model; the pages keep queries in FP16, dequantize each loaded
// segment of the cache and use an online softmax (flash attention).
//
// Design (MI355X first):
//  * Flash-decoding split: workgroup (split, h, b) streams `cpw` chunks of 256
//    cached positions of one KV head for all Hq / Hkv <= 16 query heads that
//    share it.  Its 8 wavefronts form two streams over alternate chunks, each
//    wavefront taking 64 positions of every chunk of its stream (two
//    wavefronts per SIMD); each keeps its own online softmax (no barrier inside
//    the loop) while its next chunk's codes are already in flight.  The
//    wavefronts meet once at the end and write one partial record (max, sum,
//    unnormalised output) per query head; k_kv_decode_combine merges the
//    records of a head.
//  * Both products run on the matrix cores (v_mfma_f32_16x16x32_f16) on exact
//    operands.  A 4-bit code c enters as the fp16 subnormal c 2^-24 (bit
//    pattern c: the masked nibble itself), or 16 c 2^-24 for the high nibble
//    of a byte, whose query operand is then divided by 16; every product is
//    exact in fp32 and no constant has to be cancelled, so the fp32 sums carry
//    only the magnitude of q . c.  The scale / min of the position are applied
//    around the product, in fp32: q . k_j = (2^24 scale_j) (q . c_j 2^-24) +
//    min_j sum(q).
//  * Scores: keys are the M index (16 per tile, lane-major), query heads the N
//    index, head dimensions the contraction; lane (head n, g) ends with the
//    scores of positions 4 g .. 4 g + 3 of each tile.
//  * Values: the product P V contracts over positions, which the cache holds
//    row-wise.  Each 16-position tile is transposed on the matrix cores by a
//    selection matrix with entries 1024 (64 for a high nibble): T = V_tile x
//    Sel = c 2^-14, exact and an fp16 normal number for c >= 1, which leaves
//    position 4 g + r in register r of lane (dim, g): exactly the B-operand
//    layout of P V for the position order the scores already have.  The
//    output rows carry the factor 2^-14 until the wavefronts merge.
//  * The weights P' = p * scale_v enter the product as fp16 (the pages' FP16
//    dot product); sum_j p_j min_j is added in fp32.
//  * When one workgroup per KV head already fills the machine (B * Hkv >= 256
//    compute units) the split is a single chunk run and the workgroup writes
//    the normalised fp16 output itself: no workspace, no merge kernel.
#include <cfloat>
#include <mutex>
#include <type_traits>

#include "common.hpp"

namespace qr {

constexpr int KD_DH = 128;     // head dimension
constexpr int KD_CHUNK = 256;  // positions per workgroup pass: 4 wavefronts x 4 tiles x 16
constexpr int KD_TARGET_WG = 256;  // workgroups the split aims for: one per compute unit

struct KdPlan {
  int chunks, cpw, splits;
};
static KdPlan kd_plan(int64_t B, int64_t Hkv, int64_t L) {
  KdPlan p;
  p.chunks = (int)((L + KD_CHUNK - 1) / KD_CHUNK);
  const int64_t pairs = B * Hkv;
  int64_t want = (KD_TARGET_WG + pairs - 1) / pairs;
  if (want < 1) want = 1;
  const int splits0 = (int)(want < p.chunks ? want : p.chunks);
  p.cpw = (p.chunks + splits0 - 1) / splits0;
  p.splits = (p.chunks + p.cpw - 1) / p.cpw;
  return p;
}

// Packed 4-bit codes (8 per dword: code 2i in the low nibble of byte i) ->
// 8 fp16 subnormals in the element order (c0, c4, c1, c5, c2, c6, c3, c7): even
// codes as c 2^-24, odd codes as 16 c 2^-24 (their nibble left in place), so
// five bit operations per dword with no constant to add.  mlo = 0x000F000F and
// mhi = 0x00F000F0 come in registers.
__device__ __forceinline__ v8h codes8_f16(uint32_t x, uint32_t mlo, uint32_t mhi) {
  const uint32_t x8 = x >> 8;
  v4u r;
  r[0] = x & mlo;   // c0, c4
  r[1] = x & mhi;   // 16 c1, 16 c5
  r[2] = x8 & mlo;  // c2, c6
  r[3] = x8 & mhi;  // 16 c3, 16 c7
  return __builtin_bit_cast(v8h, r);
}
// Code index of fragment element j, and whether it carries the factor 16.
__device__ __forceinline__ constexpr int kd_pi(int j) { return (j >> 2) * 2 + (j & 1) * 4 + ((j >> 1) & 1); }
__device__ __forceinline__ constexpr bool kd_odd(int j) { return (j >> 1) & 1; }

__device__ __forceinline__ float fp16_lo(uint32_t w) { return h2f((uint16_t)(w & 0xffffu)); }
__device__ __forceinline__ float fp16_hi(uint32_t w) { return h2f((uint16_t)(w >> 16)); }

// Head dimension held by lane n' of output tile (kb, hs) after the transpose.
__device__ __forceinline__ int kd_dim(int kb, int hs, int np) {
  return 32 * (2 * hs + (np >> 3)) + 8 * kb + kd_pi(np & 7);
}

// Wavefronts per workgroup: 4 position blocks x KD_SETS chunk streams.
constexpr int KD_SETS = 2;
constexpr int KD_WAVES = 4 * KD_SETS;

__global__ __launch_bounds__(64 * KD_WAVES) void k_kv_decode(
    const uint16_t* __restrict__ q, int Hq, int Hkv, int GQ, const uint8_t* __restrict__ kc,
    const uint32_t* __restrict__ km, const uint8_t* __restrict__ vc,
    const uint32_t* __restrict__ vm, int S_max, int L, float scale_log2e, int chunks, int cpw,
    int splits, float* __restrict__ ws, uint16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) float s_meta[KD_WAVES][4][64];  // k scale, k min, v scale, v min
  __shared__ float s_o[KD_WAVES][16][KD_DH];
  __shared__ float s_l[KD_WAVES][16], s_ms[KD_WAVES][16], s_mw[KD_WAVES][16];

  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // wavefront w takes positions 64 (w % 4) .. + 63 of every KD_SETS-th chunk,
  // starting at chunk c0 + w / 4: two wavefronts per SIMD stream the same KV head.
  const int wq = w & 3, ws0 = w >> 2;
  const int n = lane & 15, g = lane >> 4;

  // This (b, h)'s cache rows; positions >= L are outside the resources and read as zero.
  const int64_t row0 = ((int64_t)b * Hkv + h) * S_max;
  const __amdgpu_buffer_rsrc_t rs_kc =
      __builtin_amdgcn_make_buffer_rsrc((void*)(kc + row0 * 64), 0, L * 64, 0x00020000);
  const __amdgpu_buffer_rsrc_t rs_vc =
      __builtin_amdgcn_make_buffer_rsrc((void*)(vc + row0 * 64), 0, L * 64, 0x00020000);
  const __amdgpu_buffer_rsrc_t rs_km =
      __builtin_amdgcn_make_buffer_rsrc((void*)(km + row0), 0, L * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t rs_vm =
      __builtin_amdgcn_make_buffer_rsrc((void*)(vm + row0), 0, L * 4, 0x00020000);

  // Bit masks of the code unpacking, held in registers.
  uint32_t mlo = 0x000F000Fu, mhi = 0x00F000F0u;
  asm volatile("" : "+v"(mlo), "+v"(mhi));

  // ---- query fragments (B operand of the scores): lane (head n, g), block kb,
  //      element j holds dim 32 g + 8 kb + pi(j), divided by 16 where the code
  //      operand carries 16 c; heads >= GQ are zero.  qsum is the sum of the
  //      query itself ----
  v8h qf[4];
  float qsum = 0.0f;
  {
    const bool real = n < GQ;
    const uint16_t* qh = q + ((int64_t)b * Hq + (int64_t)h * GQ + (real ? n : 0)) * KD_DH + 32 * g;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const v4u raw = real ? *(const v4u*)(qh + 8 * kb) : v4u{0u, 0u, 0u, 0u};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int i = kd_pi(j);
        const float v = (i & 1) ? fp16_hi(raw[i >> 1]) : fp16_lo(raw[i >> 1]);
        const _Float16 o = (_Float16)(kd_odd(j) ? v * 0.0625f : v);
        qf[kb][j] = o;
        qsum += v;
      }
    }
    qsum += __shfl_xor(qsum, 16);
    qsum += __shfl_xor(qsum, 32);
  }

  // Selection matrices of the transpose: Sel_hs[k = 8 g + j][n'] = w_j iff
  // g == 2 hs + (n' >> 3) and j == (n' & 7), with w_j = 1024 (64 on the
  // elements that carry 16 c), so that the product holds c 2^-14.
  v8h sel[2];
#pragma unroll
  for (int hs = 0; hs < 2; ++hs)
#pragma unroll
    for (int j = 0; j < 8; ++j)
      sel[hs][j] = (g == 2 * hs + (n >> 3) && j == (n & 7))
                       ? (_Float16)(kd_odd(j) ? 64.0f : 1024.0f) : (_Float16)0.0f;

  // Running state: max (log2 domain) for head n and for heads 4 g + r (the
  // output rows this lane accumulates), lane-partial sums of p and p * min_v.
  float m_n = -FLT_MAX, m_r[4] = {-FLT_MAX, -FLT_MAX, -FLT_MAX, -FLT_MAX};
  float l_n = 0.0f, ms_n = 0.0f;
  v4f O[4][2];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int hs = 0; hs < 2; ++hs) O[kb][hs] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  // ---- loads of one chunk: codes of tile t (lane m = position 16 t + n, 16
  //      bytes = dims 32 g .. 32 g + 31), one metadata word per lane.  The next
  //      chunk's are issued once the current one's keys are consumed. ----
  v4u kraw[4], vraw[4], vnext[4];
  uint32_t kmeta_reg, vmeta_reg;
  auto load_k = [&](int kw) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
      kraw[t] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(
                                            rs_kc, (kw + 16 * t + n) * 64 + 16 * g, 0, 0));
    kmeta_reg = __builtin_amdgcn_raw_buffer_load_b32(rs_km, (kw + lane) * 4, 0, 0);
    vmeta_reg = __builtin_amdgcn_raw_buffer_load_b32(rs_vm, (kw + lane) * 4, 0, 0);
  };
  auto load_v = [&](int kw, v4u* dst) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
      dst[t] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(
                                           rs_vc, (kw + 16 * t + n) * 64 + 16 * g, 0, 0));
  };

  const int c0 = split * cpw, c1 = min(chunks, c0 + cpw);
  // One chunk: values of this chunk in vcur, the next chunk's fetched into vnxt.
  auto chunk = [&](const int c, v4u (&vcur)[4], v4u (&vnxt)[4]) {
    const int kw = c * KD_CHUNK + 64 * wq;  // first position of this wavefront's 64
    // metadata of the wavefront's 64 positions, converted once per position
    // (the key's scale already carrying the log2-domain softmax scale and the
    // 2^24 of the code operands: exact, a power of two)
    s_meta[w][0][lane] = (scale_log2e * fp16_lo(kmeta_reg)) * 16777216.0f;
    s_meta[w][1][lane] = scale_log2e * fp16_hi(kmeta_reg);
    s_meta[w][2][lane] = fp16_lo(vmeta_reg);
    s_meta[w][3][lane] = fp16_hi(vmeta_reg);
    __builtin_amdgcn_wave_barrier();

    // ---- scores of tile t: lane (head n, g) gets positions 16 t + 4 g + r ----
    float sc[4][4];
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(codes8_f16(kraw[t][kb], mlo, mhi), qf[kb],
                                                     acc, 0, 0, 0);
      const v4f ks = *(const v4f*)&s_meta[w][0][16 * t + 4 * g];
      const v4f kmn = *(const v4f*)&s_meta[w][1][16 * t + 4 * g];
#pragma unroll
      for (int r = 0; r < 4; ++r) sc[t][r] = fmaf(ks[r], acc[r], kmn[r] * qsum);
    }
    if ((c + 1) * KD_CHUNK > L) {  // the last chunk: positions past L take no weight
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (kw + 16 * t + 4 * g + r >= L) sc[t][r] = -INFINITY;
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sc[t][r]);
    const bool more = c + KD_SETS < c1;
    if (more) {
      load_k(kw + KD_SETS * KD_CHUNK);
      load_v(kw + KD_SETS * KD_CHUNK, vnxt);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));

    // ---- online softmax update, per wavefront (no barrier: the wavefronts
    //      meet once, at the end).  The maxima start at -FLT_MAX, not -inf, so
    //      that a wavefront whose positions are all past L keeps weights 0 and
    //      factors 1 instead of NaN. ----
    auto chunk_max = [&](int hd) { return __shfl(mx, hd); };  // lane hd holds head hd's
    const float mnew_n = fmaxf(m_n, mx);
    if (c > c0 + ws0) {
      const float a_n = __builtin_amdgcn_exp2f(m_n - mnew_n);
      l_n *= a_n;
      ms_n *= a_n;
      float a[4];
      bool grew = false;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float mnew = fmaxf(m_r[r], chunk_max(4 * g + r));
        grew |= mnew > m_r[r];
        a[r] = __builtin_amdgcn_exp2f(m_r[r] - mnew);
        m_r[r] = mnew;
      }
      if (__any(grew)) {  // rescale the output rows only when a maximum moved
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int hs = 0; hs < 2; ++hs) O[kb][hs][r] *= a[r];
      }
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) m_r[r] = fmaxf(m_r[r], chunk_max(4 * g + r));
    }
    m_n = mnew_n;

    // ---- weights P' = p * scale_v in fp16, A operands of P V: block kp =
    //      tiles (2 kp, 2 kp + 1), element j -> position 4 g + (j & 3) of tile
    //      2 kp + (j >> 2) ----
    v8h ph[2];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const v4f vs = *(const v4f*)&s_meta[w][2][16 * t + 4 * g];
      const v4f vmn = *(const v4f*)&s_meta[w][3][16 * t + 4 * g];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = __builtin_amdgcn_exp2f(sc[t][r] - m_n);
        l_n += p;
        ms_n = fmaf(p, vmn[r], ms_n);
        ph[t >> 1][4 * (t & 1) + r] = (_Float16)(p * vs[r]);
      }
    }

    // ---- P V: transpose each value tile on the matrix cores, then multiply ----
    const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kp = 0; kp < 2; ++kp) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const v8h va = codes8_f16(vcur[2 * kp][kb], mlo, mhi);
        const v8h vb = codes8_f16(vcur[2 * kp + 1][kb], mlo, mhi);
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
          const v4f ta = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, sel[hs], zero, 0, 0, 0);
          const v4f tb = __builtin_amdgcn_mfma_f32_16x16x32_f16(vb, sel[hs], zero, 0, 0, 0);
          v8h bop;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            bop[r] = (_Float16)ta[r];
            bop[4 + r] = (_Float16)tb[r];
          }
          O[kb][hs] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ph[kp], bop, O[kb][hs], 0, 0, 0);
        }
      }
    }
  };
  const int cs = c0 + ws0;  // this wavefront's first chunk (it may have none)
  if (cs < c1) {
    load_k(cs * KD_CHUNK + 64 * wq);
    load_v(cs * KD_CHUNK + 64 * wq, vraw);
  }
  for (int c = cs; c < c1; c += 2 * KD_SETS) {  // two chunks per trip: the value buffers swap roles
    chunk(c, vraw, vnext);
    if (c + KD_SETS < c1) chunk(c + KD_SETS, vnext, vraw);
  }

  // ---- combine the wavefronts (each with its own running maxima) and write
  //      the partial record of every query head: max, sum, unnormalised output ----
  l_n += __shfl_xor(l_n, 16);
  l_n += __shfl_xor(l_n, 32);
  ms_n += __shfl_xor(ms_n, 16);
  ms_n += __shfl_xor(ms_n, 32);
  if (g == 0) {
    s_l[w][n] = l_n;
    s_ms[w][n] = ms_n;
    s_mw[w][n] = m_n;
  }
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int hs = 0; hs < 2; ++hs)
#pragma unroll
      for (int r = 0; r < 4; ++r)  // the rows carried c 2^-14 (exact power of two)
        s_o[w][4 * g + r][kd_dim(kb, hs, n)] = O[kb][hs][r] * 16384.0f;
  __syncthreads();
  for (int i = tid; i < GQ * KD_DH; i += 64 * KD_WAVES) {
    const int hd = i / KD_DH, d = i % KD_DH;
    float M = s_mw[0][hd];
#pragma unroll
    for (int v = 1; v < KD_WAVES; ++v) M = fmaxf(M, s_mw[v][hd]);
    float o = 0.0f, l = 0.0f;
#pragma unroll
    for (int v = 0; v < KD_WAVES; ++v) {
      const float f = __builtin_amdgcn_exp2f(s_mw[v][hd] - M);
      o = fmaf(f, s_o[v][hd][d] + s_ms[v][hd], o);
      l = fmaf(f, s_l[v][hd], l);
    }
    const int64_t head = (int64_t)b * Hq + (int64_t)h * GQ + hd;
    if (splits == 1) {  // the whole context in one workgroup: the final output
      out[head * KD_DH + d] = f2h(o / l);
    } else {
      float* rec = ws + (head * splits + split) * (KD_DH + 2);
      rec[2 + d] = o;
      if (d == 0) {
        rec[0] = M;
        rec[1] = l;
      }
    }
  }
}

// Merge the split records of one query head in one pass (running max, the
// loads of every record independent of the previous ones):
// o = sum_s o_s 2^(m_s - M) / sum_s l_s 2^(m_s - M).
__global__ __launch_bounds__(KD_DH) void k_kv_decode_combine(const float* __restrict__ ws,
                                                             int splits,
                                                             uint16_t* __restrict__ out) {
  const int64_t head = blockIdx.x;  // b * Hq + hq
  const int d = threadIdx.x;
  const float* rec = ws + head * splits * (KD_DH + 2);
  float M = -FLT_MAX, l = 0.0f, o = 0.0f;
#pragma unroll 4
  for (int s = 0; s < splits; ++s) {
    const float* r = rec + s * (KD_DH + 2);
    const float ms = r[0], ls = r[1], os = r[2 + d];
    const float Mn = fmaxf(M, ms);
    const float a = __builtin_amdgcn_exp2f(M - Mn), bs = __builtin_amdgcn_exp2f(ms - Mn);
    l = fmaf(l, a, ls * bs);
    o = fmaf(o, a, os * bs);
    M = Mn;
  }
  out[head * KD_DH + d] = f2h(o / l);
}

}  // namespace qr

using namespace qr;

extern "C" int64_t qr_kv_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t Dh,
                                                int32_t L) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Dh < 1 || L < 1) return 0;
  const KdPlan p = kd_plan(B, Hkv, L);
  if (p.splits == 1) return 0;  // one workgroup per KV head writes the output directly
  return (int64_t)B * Hq * p.splits * (Dh + 2) * (int64_t)sizeof(float);
}

namespace qr {

// Validation shared by both entry points (everything but the workspace).
static qr_status kd_validate(const void* q_f16, int32_t B, int32_t Hq, int32_t Hkv, int32_t Dh,
                             int32_t S_max, int32_t L, int32_t group, float softmax_scale) {
  if (B < 0 || Hq < 1 || Hkv < 1 || S_max < 1 || L < 1 || L > S_max) return QR_ERR_SHAPE;
  if (Hq % Hkv != 0) return QR_ERR_SHAPE;
  if (Dh != KD_DH || group != KD_DH || Hq / Hkv > 16) return QR_ERR_UNSUPPORTED;
  if (!(softmax_scale > 0.0f) || !(softmax_scale < 1e30f)) return QR_ERR_ARG;
  if ((int64_t)S_max * 64 > INT32_MAX) return QR_ERR_SHAPE;
  if ((int64_t)B * Hq > INT32_MAX || B > 65535 || Hkv > 65535) return QR_ERR_SHAPE;
  (void)q_f16;
  return QR_OK;
}

static qr_status kd_check_pointers(const void* q_f16, const void* k_cache_q,
                                   const void* k_cache_meta, const void* v_cache_q,
                                   const void* v_cache_meta, const void* out_f16) {
  if (!q_f16 || !k_cache_q || !k_cache_meta || !v_cache_q || !v_cache_meta || !out_f16)
    return QR_ERR_NULL;
  if (!aligned(q_f16, 16) || !aligned(k_cache_q, 16) || !aligned(v_cache_q, 16) ||
      !aligned(k_cache_meta, 4) || !aligned(v_cache_meta, 4) || !aligned(out_f16, 2))
    return QR_ERR_ALIGN;
  return QR_OK;
}

// The launches, on validated arguments; ws holds the split records (unused
// when the plan has a single split).
static qr_status kd_run(const void* q_f16, int32_t B, int32_t Hq, int32_t Hkv,
                        const void* k_cache_q, const void* k_cache_meta, const void* v_cache_q,
                        const void* v_cache_meta, int32_t S_max, int32_t L, float softmax_scale,
                        void* out_f16, void* ws, hipStream_t stream) {
  const KdPlan p = kd_plan(B, Hkv, L);
  const float scale_log2e = softmax_scale * 1.4426950408889634f;
  hipLaunchKernelGGL(k_kv_decode, dim3(p.splits, Hkv, B), dim3(64 * KD_WAVES), 0, stream,
                     (const uint16_t*)q_f16, Hq, Hkv, Hq / Hkv, (const uint8_t*)k_cache_q,
                     (const uint32_t*)k_cache_meta, (const uint8_t*)v_cache_q,
                     (const uint32_t*)v_cache_meta, S_max, L, scale_log2e, p.chunks, p.cpw,
                     p.splits, (float*)ws, (uint16_t*)out_f16);
  qr_status st = launch_status();
  if (st != QR_OK || p.splits == 1) return st;
  hipLaunchKernelGGL(k_kv_decode_combine, dim3((unsigned)(B * Hq)), dim3(KD_DH), 0, stream,
                     (const float*)ws, p.splits, (uint16_t*)out_f16);
  return launch_status();
}

// ---------------------------------------------------------------------------
// Allocation-free variant: the split records live in a static device array,
// one copy per GPU (each GPU the library runs on holds it until the process
// ends).  The array's name is only a host-side handle; its device address is
// looked up once per device with that device current and kept per device.
// Every call on a GPU shares that GPU's array: calls that overlap on one GPU
// race.  No record has to start at zero (each split writes all of its
// records before the merge reads them).
// ---------------------------------------------------------------------------
constexpr int64_t KD_SCRATCH_BYTES = QR_KV_DECODE_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[KD_SCRATCH_BYTES];

constexpr int KD_MAX_DEVICES = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[KD_MAX_DEVICES] = {};

static qr_status kd_scratch(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= KD_MAX_DEVICES) {
    (void)hipGetLastError();
    return QR_ERR_LAUNCH;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return QR_ERR_LAUNCH;
    }
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return QR_OK;
}

}  // namespace qr

using namespace qr;

extern "C" qr_status qr_kv_decode_attention(const void* q_f16, int32_t B, int32_t Hq,
                                            int32_t Hkv, int32_t Dh, const void* k_cache_q,
                                            const void* k_cache_meta, const void* v_cache_q,
                                            const void* v_cache_meta, int32_t S_max, int32_t L,
                                            int32_t group, float softmax_scale, void* out_f16,
                                            void* workspace, int64_t workspace_bytes,
                                            hipStream_t stream) {
  qr_status st = kd_validate(q_f16, B, Hq, Hkv, Dh, S_max, L, group, softmax_scale);
  if (st != QR_OK) return st;
  if (B == 0) return QR_OK;
  const int64_t need = qr_kv_decode_workspace_bytes(B, Hq, Hkv, Dh, L);
  st = kd_check_pointers(q_f16, k_cache_q, k_cache_meta, v_cache_q, v_cache_meta, out_f16);
  if (st == QR_OK && need > 0 && !workspace) st = QR_ERR_NULL;
  if (st != QR_OK) return st;
  if (workspace_bytes < need) return QR_ERR_SHAPE;
  if (!aligned(workspace, 4)) return QR_ERR_ALIGN;
  return kd_run(q_f16, B, Hq, Hkv, k_cache_q, k_cache_meta, v_cache_q, v_cache_meta, S_max, L,
                softmax_scale, out_f16, workspace, stream);
}

extern "C" qr_status qr_kv_decode_attention_noalloc(const void* q_f16, int32_t B, int32_t Hq,
                                                    int32_t Hkv, int32_t Dh,
                                                    const void* k_cache_q,
                                                    const void* k_cache_meta,
                                                    const void* v_cache_q,
                                                    const void* v_cache_meta, int32_t S_max,
                                                    int32_t L, int32_t group,
                                                    float softmax_scale, void* out_f16,
                                                    hipStream_t stream) {
  qr_status st = kd_validate(q_f16, B, Hq, Hkv, Dh, S_max, L, group, softmax_scale);
  if (st != QR_OK) return st;
  if (B == 0) return QR_OK;
  const int64_t need = qr_kv_decode_workspace_bytes(B, Hq, Hkv, Dh, L);
  if (need > KD_SCRATCH_BYTES) return QR_ERR_SCRATCH;
  st = kd_check_pointers(q_f16, k_cache_q, k_cache_meta, v_cache_q, v_cache_meta, out_f16);
  if (st != QR_OK) return st;
  void* ws = nullptr;
  if (need > 0) {
    st = kd_scratch(&ws);
    if (st != QR_OK) return st;
  }
  return kd_run(q_f16, B, Hq, Hkv, k_cache_q, k_cache_meta, v_cache_q, v_cache_meta, S_max, L,
                softmax_scale, out_f16, ws, stream);
}
