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
//  * qr_w8a8_gemm (QuaRot paper, 6- and 8-bit RTN results) runs the same
//    kernel on codes stored one per byte: chunks go to the matrix cores as
//    loaded, one per MFMA step, and a K step covers 128 elements.
//  * Tiles: (64 WM) x (64 WN) outputs per workgroup of 4 wavefronts (one per
//    SIMD, 2 x 2), each owning a (32 WM) x (32 WN) block = WM x WN MFMA tiles.
//    256 x 256 (WM = WN = 4, accumulators in the AGPR half of the register
//    file, one workgroup per CU) is the default; 128 x 128 (WM = WN = 2, two
//    workgroups per CU) is used when its estimated time is shorter: small
//    grids that would leave compute units idle.  K advances 256 at a time
//    through two LDS stages.  The buffer unit copies the next step's panels
//    straight into the other stage (buffer_load ... lds: no registers, no LDS
//    write instructions) while the current one is multiplied; each wavefront
//    waits for its own copies before the barrier that ends the step.
//  * Each lane reads whole 16-byte k-chunks (32 codes) and feeds two MFMAs from
//    one chunk: lane (row, half h) takes chunk 2p + h for MFMA steps 2p and
//    2p + 1, identically for A and W, so every k is summed exactly once.  The
//    reads of the next chunk pair and the unpacking of the next half are
//    interleaved with the current MFMAs (pinned with sched_group_barrier).
//  * LDS layout: rows of 128 bytes, chunk c of row r at position c ^ h(r) with
//    h(r) = (r mod 8) ^ (bit 3 of r).  A copy instruction fills 1 KB = 8 whole
//    rows (lane l lands at 16 l, so each lane fetches the chunk the layout puts
//    there and 8 lanes read one row's 128 contiguous bytes), and a fragment
//    read -- 32 consecutive rows, one chunk -- hits distinct banks in both 8-
//    and 16-lane LDS passes.
//  * Tile order: workgroup ids are remapped so that the ids the hardware places
//    on one XCD (id % 8) are consecutive, then grouped 8 tile-rows at a time, so
//    the tiles running together on an XCD share A and W panels in its L2.
//  * Epilogue: the scaled fp16 tile is written row-major into the LDS stages
//    (free once the K loop ends; 256 x 256 x 2 bytes fill them exactly) and
//    leaves as non-temporal 16-byte row pieces, not one 2-byte store per
//    accumulator element.
#include <algorithm>
#include <type_traits>

#include "common.hpp"

namespace qr {

constexpr int KCH = 8;             // 16-byte k-chunks per row and step
constexpr int GEMM_THREADS = 256;
// Codes per 16-byte chunk and per K step for BITS = 4 (packed) or 8 (one per byte).
template <int BITS>
struct CodeFmt {
  static constexpr int EPC = 128 / BITS;     // elements per 16-byte chunk: 32 or 16
  static constexpr int BKE = KCH * EPC;      // elements per K step: 256 or 128
  static constexpr int FR = BITS == 4 ? 1 : 2;  // chunks per lane and MFMA pair
  static constexpr int SHIFT = BITS == 4 ? 8 : 0;  // the int4 accumulator holds 256 * acc
};

__device__ __forceinline__ v4i unpack16(uint2 d) {
  v4i r;
  r[0] = (int)((d.x << 4) & 0xF0F0F0F0u);
  r[1] = (int)(d.x & 0xF0F0F0F0u);
  r[2] = (int)((d.y << 4) & 0xF0F0F0F0u);
  r[3] = (int)(d.y & 0xF0F0F0F0u);
  return r;
}

// LDS byte offset of 16-byte k-chunk `kk` of row r of a panel: rows of
// KCH * 16 = 128 bytes, the chunk position XOR-swizzled by h(r) = (r mod 8) ^
// (bit 3 of r).  h is a permutation on every 8 consecutive rows and on the even
// (and the odd) rows of every 16, so the 8- and 16-lane passes of a fragment
// read (consecutive rows, one chunk) hit distinct banks.
__device__ __forceinline__ int lds_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int lds_off(int kk, int r) {
  return r * (KCH * 16) + ((kk ^ lds_swz(r)) << 4);
}

template <int WM, int WN, int BITS = 4>
struct GemmTile {
  static constexpr int BM = 64 * WM, BN = 64 * WN;
  static constexpr int A_BYTES = BM * KCH * 16, W_BYTES = BN * KCH * 16;
  static constexpr int STAGE = A_BYTES + W_BYTES;
  static constexpr int LDS = 2 * STAGE;
  static constexpr int PA = BM * KCH / GEMM_THREADS, PW = BN * KCH / GEMM_THREADS;
  static constexpr int MF = WM * WN;                      // MFMAs per half step
  // unpack VALU per MFMA (int8 operands go to the matrix cores as loaded)
  static constexpr int VPM = BITS == 4 ? (6 * (WM + WN) + MF - 1) / MF : 1;
  static constexpr int DSR = (WM + WN) * CodeFmt<BITS>::FR;  // fragment reads per pair
};

// BITS = 4: packed INT4 operands (K/2 bytes per row), unpacked in registers.
// BITS = 8: codes stored one per byte (K bytes per row, b <= 8 bits), fed to
// the matrix cores as loaded; the LDS geometry (128 bytes per row and step)
// is the same, so a K step covers 128 instead of 256 elements.
// GROUPED (INT4 only): one scale per group of `kgroup` consecutive k on both
// operands (a_scale [T, K/kgroup], w_scale [N, K/kgroup]).  After each pair of
// MFMA steps that closes a group, every accumulator is scaled by its group's
// token and channel scales, added to an fp32 sum and reset.  PG = kgroup / 64
// pairs per group when a group fits in one K step (PG <= 4): then a group's
// first MFMAs start from a zero accumulator instead of clearing it.
template <int WM, int WN, bool DBG, bool KTAIL, int BITS = 4, bool GROUPED = false, int PG = 0>
__global__ __launch_bounds__(GEMM_THREADS, (WM * WN <= 4 && !GROUPED) ? 2 : 1) void k_w4a4_gemm(
    const uint8_t* __restrict__ A, const uint16_t* __restrict__ a_scale, int T,
    const uint8_t* __restrict__ W, const uint16_t* __restrict__ w_scale, int N, int K,
    uint16_t* __restrict__ Y, int32_t* __restrict__ acc_dbg, int tiles_m, int tiles_n,
    int kgroup = 0) {
  using Tl = GemmTile<WM, WN, BITS>;
  using CF = CodeFmt<BITS>;
  constexpr int BM = Tl::BM, BN = Tl::BN;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

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
  const int wm = (wave >> 1) * (32 * WM), wn = (wave & 1) * (32 * WN);  // wave's block
  const int li = lane & 31, lg = lane >> 5;  // MFMA row/col lane, k-half
  const int64_t rowbytes = (int64_t)K * BITS / 8;

  // ---- global -> LDS, straight through the buffer unit: one wavefront
  //      instruction fills one 1 KB block of 8 whole rows (lane l lands in slot
  //      l: row 8 b + l / 8, position l % 8) and fetches the chunk the layout
  //      puts there, so 8 lanes read one row's 128 contiguous bytes.  Block
  //      b = 4 j + wave, so the lane's chunk ((l % 8) ^ h(row)) is the same for
  //      every j.  Raw buffer loads over the tile's own rows: rows past T (or N)
  //      fall outside the buffer's range (their outputs are never stored). ----
  const int rows_a = min(T - m0, BM), rows_w = min(N - n0, BN);
  const __amdgpu_buffer_rsrc_t rsrc_a = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(A + (int64_t)m0 * rowbytes), 0, (int)(rows_a * rowbytes), 0x00020000);
  const __amdgpu_buffer_rsrc_t rsrc_w = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(W + (int64_t)n0 * rowbytes), 0, (int)(rows_w * rowbytes), 0x00020000);
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int dl_kk = (lane & 7) ^ (lane >> 3) ^ (wave_u & 1);   // chunk of the lane's slot
  const int voff = (8 * wave_u + (lane >> 3)) * (int)rowbytes + dl_kk * 16;
  const int rstep = 32 * (int)rowbytes;                          // 4 blocks of 8 rows
  typedef __attribute__((address_space(3))) void* lds_ptr_t;
  auto dload = [&](int stage, int k0, bool last) {  // k0 in elements
    uint8_t* pa = smem + stage * Tl::STAGE;
    uint8_t* pw = pa + Tl::A_BYTES;
    // the whole global offset goes in the VGPR operand: the range check of a
    // raw buffer covers the VGPR offset, not the SGPR one.  The uniform part
    // is formed per step (readfirstlane keeps the compiler from hoisting one
    // VGPR per j out of the K loop).
#pragma unroll
    for (int j = 0; j < Tl::PA; ++j) {
      const int so = __builtin_amdgcn_readfirstlane(j * rstep + k0 * BITS / 8);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_a, (lds_ptr_t)(pa + (4 * j + wave_u) * 1024), 16,
                                               voff + so, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < Tl::PW; ++j) {
      const int so = __builtin_amdgcn_readfirstlane(j * rstep + k0 * BITS / 8);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_w, (lds_ptr_t)(pw + (4 * j + wave_u) * 1024), 16,
                                               voff + so, 0, 0, 0);
    }
    (void)last;
  };
  // Wait for this wavefront's copies; in the last step of a K with a tail,
  // clear the slots of chunks past K (they hold the next row's codes), each
  // lane its own slot, which its own copy has already written.
  auto dwait = [&](int stage, int k0, bool last) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    if (KTAIL && last && k0 + dl_kk * CF::EPC >= K) {
      uint8_t* pa = smem + stage * Tl::STAGE;
      uint8_t* pw = pa + Tl::A_BYTES;
#pragma unroll
      for (int j = 0; j < Tl::PA; ++j) *(v4u*)(pa + (4 * j + wave_u) * 1024 + lane * 16) = v4u{0u, 0u, 0u, 0u};
#pragma unroll
      for (int j = 0; j < Tl::PW; ++j) *(v4u*)(pw + (4 * j + wave_u) * 1024 + lane * 16) = v4u{0u, 0u, 0u, 0u};
    }
  };
  // fragments of chunk pair p: WM of A (rows wm + 32 i + li) and WN of W.
  // INT4: the lane takes chunk 2p + lg, both halves of which feed the pair's
  // two MFMA steps; int8: chunks 4p + 2e + lg, one per MFMA step e.
  auto lread = [&](int stage, int p, v4u (*fa)[WM], v4u (*fb)[WN]) {
    const uint8_t* pa = smem + stage * Tl::STAGE;
    const uint8_t* pw = pa + Tl::A_BYTES;
#pragma unroll
    for (int f = 0; f < CF::FR; ++f) {
      const int kk = BITS == 4 ? 2 * p + lg : 4 * p + 2 * f + lg;
#pragma unroll
      for (int i = 0; i < WM; ++i)
        fa[f][i] = *(const v4u*)(pa + lds_off(kk, wm + i * 32 + li));
#pragma unroll
      for (int j = 0; j < WN; ++j)
        fb[f][j] = *(const v4u*)(pw + lds_off(kk, wn + j * 32 + li));
    }
  };

  v16i acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

  // group-wise scales: fp32 sums of the scaled per-group accumulators
  constexpr int GW = GROUPED ? WM : 1, GN = GROUPED ? WN : 1;
  float facc[GW][GN][16];
  if constexpr (GROUPED) {
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
      for (int j = 0; j < WN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) facc[i][j][r] = 0.0f;
  }
  const int ngroups = GROUPED ? K / kgroup : 1;
  constexpr int NP = BITS == 4 ? KCH / 2 : KCH / 4;  // MFMA pairs per step
  constexpr bool FRESH = GROUPED && PG >= 1 && PG <= NP;
  // the scales of the next group to close, fetched one group ahead so that
  // their loads are in flight while that group's MFMAs run
  // Raw buffer loads over the tile's own scale rows: rows past T (or N) read
  // as zero (their outputs are never stored); one 32-bit offset per load.
  float asg[GW][16], wsg[GN];
  const __amdgpu_buffer_rsrc_t rsrc_as = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a_scale + (int64_t)m0 * ngroups), 0, rows_a * ngroups * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsrc_ws = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(w_scale + (int64_t)n0 * ngroups), 0, rows_w * ngroups * 2, 0x00020000);
  const int as_off = (wm + 4 * lg) * ngroups * 2, ws_off = (wn + li) * ngroups * 2;
  auto load_scales = [&](int gi) __attribute__((always_inline)) {
    if constexpr (GROUPED) {
#pragma unroll
      for (int j = 0; j < WN; ++j)
        wsg[j] = h2f(__builtin_amdgcn_raw_buffer_load_b16(
            rsrc_ws, ws_off + (j * 32 * ngroups + gi) * 2, 0, 0));
#pragma unroll
      for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          asg[i][r] = h2f(__builtin_amdgcn_raw_buffer_load_b16(
              rsrc_as, as_off + ((i * 32 + 8 * (r >> 2) + (r & 3)) * ngroups + gi) * 2, 0, 0));
    }
  };
  if constexpr (GROUPED) load_scales(0);
  // after pair p of K step ks: if that closes group g,
  // f += fp32(fp32(fp32(acc) * a_s[t, g]) * w_s[n, g]) and acc = 0 (f kept x256)
  auto rescale = [&](int ks, int p) __attribute__((always_inline)) {
    if constexpr (GROUPED) {
      const int done = ks * CF::BKE + 64 * (p + 1);
      // a group longer than a K step (PG > NP) closes only at a step's last pair
      if (FRESH ? (p + 1) % PG != 0 : (PG > NP && p + 1 != NP) || done % kgroup != 0) return;
      if (done > K) return;
      const int gi = done / kgroup - 1;
#pragma unroll
      for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            // the INT4 accumulator holds 256 * acc: converting and scaling it
            // unshifted gives exactly 256 times each fp32 step (no fp32 value
            // here comes near the subnormal range), undone exactly at the end
            const float pr = __fmul_rn(__fmul_rn((float)acc[i][j][r], asg[i][r]), wsg[j]);
            facc[i][j][r] = __fadd_rn(facc[i][j][r], pr);
            if (!FRESH) acc[i][j][r] = 0;
          }
      if (gi + 1 < ngroups) load_scales(gi + 1);
    }
  };
  // Register pipeline per chunk pair p: packed fragments f (read one pair
  // ahead), unpacked halves ua/ub[0] (e = 0) and [1] (e = 1).  While the MFMAs
  // of one half run, the VALU unpacks the other and the LDS reads of the next
  // pair are in flight; sched_group_barrier pins that order.
  v4u fa[2][CF::FR][WM], fb[2][CF::FR][WN];
  v4i ua[2][WM], ub[2][WN];
  auto unpack_half = [&](const v4u (*xa)[WM], const v4u (*xb)[WN], int e, v4i* oa, v4i* ob) {
    if constexpr (BITS == 4) {
#pragma unroll
      for (int i = 0; i < WM; ++i)
        oa[i] = unpack16(make_uint2(xa[0][i][2 * e], xa[0][i][2 * e + 1]));
#pragma unroll
      for (int j = 0; j < WN; ++j)
        ob[j] = unpack16(make_uint2(xb[0][j][2 * e], xb[0][j][2 * e + 1]));
    } else {
#pragma unroll
      for (int i = 0; i < WM; ++i) oa[i] = __builtin_bit_cast(v4i, xa[e][i]);
#pragma unroll
      for (int j = 0; j < WN; ++j) ob[j] = __builtin_bit_cast(v4i, xb[e][j]);
    }
  };
  // fresh: the first MFMAs of a group (FRESH only) start from zero
  auto mfma_half = [&](const v4i* a, const v4i* b, bool fresh = false) {
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
      for (int j = 0; j < WN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(
            a[i], b[j], fresh ? v16i{} : acc[i][j], 0, 0, 0);
  };
  const int ksteps = (K + CF::BKE - 1) / CF::BKE;
  // One K step from LDS stage `stage`.  MORE: a next step exists -- stage its
  // panels (loaded one step earlier) into the other LDS stage during the last
  // half-step, fetch the step after it, and start reading the other stage.
  auto kstep = [&](int stage, int ks, auto more_tag) {
    constexpr bool MORE = decltype(more_tag)::value;
    // the other stage was last read before the barrier that ended step ks - 1
    if (MORE) dload(stage ^ 1, (ks + 1) * CF::BKE, ks + 2 == ksteps);
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int cur = p & 1, nxt = cur ^ 1;
      if (p + 1 < NP) {
        __builtin_amdgcn_sched_barrier(0);
        lread(stage, p + 1, fa[nxt], fb[nxt]);
        mfma_half(ua[0], ub[0], FRESH && p % PG == 0);
        unpack_half(fa[cur], fb[cur], 1, ua[1], ub[1]);
        __builtin_amdgcn_sched_group_barrier(0x100, Tl::DSR, 0);  // DS reads first
#pragma unroll
        for (int m = 0; m < Tl::MF; ++m) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);        // 1 MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, Tl::VPM, 0);  // VALU
        }
        __builtin_amdgcn_sched_barrier(0);
        mfma_half(ua[1], ub[1]);
        unpack_half(fa[nxt], fb[nxt], 0, ua[0], ub[0]);
#pragma unroll
        for (int m = 0; m < Tl::MF; ++m) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
          __builtin_amdgcn_sched_group_barrier(0x002, Tl::VPM, 1);
        }
        __builtin_amdgcn_sched_barrier(0);
        rescale(ks, p);
      } else {
        __builtin_amdgcn_sched_barrier(0);
        mfma_half(ua[0], ub[0], FRESH && p % PG == 0);
        unpack_half(fa[cur], fb[cur], 1, ua[1], ub[1]);
        if (MORE) {
#pragma unroll
          for (int m = 0; m < Tl::MF; ++m) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 2);
            __builtin_amdgcn_sched_group_barrier(0x002, Tl::VPM, 2);
          }
          __builtin_amdgcn_sched_barrier(0);
          dwait(stage ^ 1, (ks + 1) * CF::BKE, ks + 2 == ksteps);
          __syncthreads();
          lread(stage ^ 1, 0, fa[nxt], fb[nxt]);
          mfma_half(ua[1], ub[1]);
          unpack_half(fa[nxt], fb[nxt], 0, ua[0], ub[0]);
          __builtin_amdgcn_sched_group_barrier(0x100, Tl::DSR, 3);
#pragma unroll
          for (int m = 0; m < Tl::MF; ++m) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 3);
            __builtin_amdgcn_sched_group_barrier(0x002, Tl::VPM, 3);
          }
        } else {
          mfma_half(ua[1], ub[1]);
        }
        __builtin_amdgcn_sched_barrier(0);
        rescale(ks, p);
      }
    }
  };

  dload(0, 0, ksteps == 1);
  dwait(0, 0, ksteps == 1);
  __syncthreads();
  lread(0, 0, fa[0], fb[0]);
  unpack_half(fa[0], fb[0], 0, ua[0], ub[0]);
  for (int ks = 0; ks + 1 < ksteps; ++ks) kstep(ks & 1, ks, std::true_type{});
  kstep((ksteps - 1) & 1, ksteps - 1, std::false_type{});

  // ---- epilogue: 32x32 accumulator layout: lane (n = li, k-half lg), register r
  //      holds row 8 (r / 4) + 4 lg + (r % 4).  The scaled fp16 tile is staged
  //      row-major in the LDS stages (free after the K loop) and stored as 16-byte
  //      row pieces: one 2-byte store per element, as the first version made, left
  //      the matrix cores idle for longer (the 256 x 256 tile 5% slower overall). ----
  float wsc[WN];
  if constexpr (!GROUPED) {
#pragma unroll
    for (int j = 0; j < WN; ++j) wsc[j] = h2f(w_scale[min(n0 + wn + j * 32 + li, N - 1)]);
  }
  static_assert(BM * BN * 2 <= Tl::LDS, "the fp16 output tile must fit in the LDS stages");
  __syncthreads();  // every wavefront's last fragment reads are done
  uint16_t* sy = (uint16_t*)smem;  // [BM][BN] fp16; 16-byte pieces XOR-swizzled by row bit 2
#pragma unroll
  for (int i = 0; i < WM; ++i) {
    // [r]: token scale of row 8 (r / 4) + 4 lg + (r % 4) of block i, times 2^-SHIFT:
    // fp32(acc) is exact (|acc| < 2^24 * 2^SHIFT, a multiple of 2^SHIFT) and
    // scaling by a power of two commutes with rounding, so
    // fp32(fp32(acc) * (a_s 2^-SHIFT)) == fp32(fp32(acc >> SHIFT) * a_s)
    float asc[16];
    if constexpr (!GROUPED) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int t0 = m0 + wm + i * 32 + 8 * q4 + 4 * lg;
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2)
          asc[4 * q4 + s2] = h2f(a_scale[min(t0 + s2, T - 1)]) * (1.0f / (1 << CF::SHIFT));
      }
    }
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const int cl = wn + j * 32 + li;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rl = wm + i * 32 + 8 * (r >> 2) + 4 * lg + (r & 3);
        uint16_t yv;
        if constexpr (GROUPED) {
          yv = f2h(__fmul_rn(facc[i][j][r], 1.0f / (1 << CF::SHIFT)));
        } else {
          yv = f2h(__fmul_rn(__fmul_rn((float)acc[i][j][r], asc[r]), wsc[j]));
          if (DBG && m0 + rl < T && n0 + cl < N)
            acc_dbg[(int64_t)(m0 + rl) * N + n0 + cl] = acc[i][j][r] >> CF::SHIFT;  // exact
        }
        sy[rl * BN + (((cl >> 3) ^ (((rl >> 2) & 1) << 2)) << 3) + (cl & 7)] = yv;
      }
    }
  }
  __syncthreads();
  constexpr int CPR = BN / 8;  // 16-byte pieces per tile row
  const bool wide = (N & 1) == 0;  // rows then start 4-byte aligned, as y_f16 is
  for (int c = tid; c < BM * CPR; c += GEMM_THREADS) {
    const int rl = c / CPR, ck = c % CPR;
    const int t = m0 + rl, n = n0 + ck * 8;
    if (t >= T || n >= N) continue;
    const v4u_a4 v = *(const v4u_a4*)(sy + rl * BN + ((ck ^ (((rl >> 2) & 1) << 2)) << 3));
    uint16_t* yp = Y + (int64_t)t * N + n;
    if (wide && n + 8 <= N) {
      __builtin_nontemporal_store(v, (v4u_a4*)yp);  // written once, read by the next op
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (n + e < N) yp[e] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
    }
  }
}


template <int WM, int WN, bool DBG, bool KTAIL, int BITS, bool GROUPED = false, int PG = 0>
static qr_status launch_gemm(const void* a_q, const void* a_scale, int64_t T, const void* w_q,
                             const void* w_scale, int64_t N, int64_t K, void* y, int32_t* acc,
                             hipStream_t stream, int group = 0) {
  using Tl = GemmTile<WM, WN, BITS>;
  auto kern = k_w4a4_gemm<WM, WN, DBG, KTAIL, BITS, GROUPED, PG>;
  // Opting in to more than 64 KB of LDS is a per-kernel attribute; setting it
  // again on every call is cheap and keeps the entry point free of state.
  if (hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                          Tl::LDS) != hipSuccess)
    return QR_ERR_LAUNCH;
  const int tiles_m = (int)((T + Tl::BM - 1) / Tl::BM);
  const int tiles_n = (int)((N + Tl::BN - 1) / Tl::BN);
  const int64_t nblk = (int64_t)tiles_m * tiles_n;
  if (nblk > INT32_MAX) return QR_ERR_SHAPE;
  hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(GEMM_THREADS), Tl::LDS, stream,
                     (const uint8_t*)a_q, (const uint16_t*)a_scale, (int)T, (const uint8_t*)w_q,
                     (const uint16_t*)w_scale, (int)N, (int)K, (uint16_t*)y, acc, tiles_m,
                     tiles_n, group);
  return launch_status();
}

template <int WM, int WN, int BITS = 4>
static qr_status launch_tile(const void* a_q, const void* a_scale, int64_t T, const void* w_q,
                             const void* w_scale, int64_t N, int64_t K, void* y, int32_t* acc,
                             hipStream_t stream) {
  const bool tail = (K % CodeFmt<BITS>::BKE) != 0;
  if (acc)
    return tail ? launch_gemm<WM, WN, true, true, BITS>(a_q, a_scale, T, w_q, w_scale, N, K, y, acc, stream)
                : launch_gemm<WM, WN, true, false, BITS>(a_q, a_scale, T, w_q, w_scale, N, K, y, acc, stream);
  return tail ? launch_gemm<WM, WN, false, true, BITS>(a_q, a_scale, T, w_q, w_scale, N, K, y, nullptr, stream)
              : launch_gemm<WM, WN, false, false, BITS>(a_q, a_scale, T, w_q, w_scale, N, K, y, nullptr, stream);
}

// Fraction of the machine's workgroup slots a tile grid keeps busy, times a
// per-tile efficiency (smaller tiles re-read more operand bytes per MAC).
// Estimated time (arbitrary units) of a grid of bm x bn tiles when `slots`
// workgroups run at once, each at relative throughput `eff`: rounds of
// concurrent tiles times one tile's work.  Edge tiles count whole.
static double tile_time(int64_t T, int64_t N, int bm, int bn, double eff, int slots) {
  const int64_t tiles = ((T + bm - 1) / bm) * ((N + bn - 1) / bn);
  const int64_t rounds = (tiles + slots - 1) / slots;
  return (double)rounds * bm * bn / eff;
}

// 256 x 256 tiles run one workgroup per compute unit (their accumulators fill
// the register file); 128 x 128 tiles run two, which hides each tile's
// prologue and epilogue behind the other's MFMAs but costs 8% of throughput
// per CU.  Launch the one with the shorter estimated time.  (256 x 128 tiles,
// one per CU at 0.9, lose to two 128 x 128 tiles at every shape.)
template <int BITS>
static qr_status launch_best(const void* a_q, const void* a_scale, int64_t T, const void* w_q,
                             const void* w_scale, int64_t N, int64_t K, void* y, int32_t* acc,
                             hipStream_t stream) {
  const double t44 = tile_time(T, N, 256, 256, 1.0, 256);
  const double t22 = tile_time(T, N, 128, 128, 0.46, 512);
  if (t22 <= t44)
    return launch_tile<2, 2, BITS>(a_q, a_scale, T, w_q, w_scale, N, K, y, acc, stream);
  return launch_tile<4, 4, BITS>(a_q, a_scale, T, w_q, w_scale, N, K, y, acc, stream);
}


// ===========================================================================
// Decode (T <= 64): weight-streaming GEMM
// ===========================================================================
// With a handful of tokens the product is bound by reading W once.  A
// workgroup owns S strips of 16 output channels (16 S consecutive rows of W)
// and all T <= 64 tokens (MT MFMA row blocks of 16); its 4 wavefronts split K
// in 128-element blocks and each streams its part of the 16 S weight rows
// exactly once with v_mfma_i32_16x16x64_i8.  Lane (row i, group g) of a block
// holds packed bytes 16 g .. 16 g + 15 (k = 32 g .. 32 g + 31) and feeds two
// MFMAs, one per 8-byte half, identically for A and W.  The activation
// fragments of a block are loaded and unpacked once and used for all S
// strips, so the unpacking of A, which dominates the vector work at T = 64,
// is shared S ways.  Loads run CH blocks ahead in a second register buffer;
// blocks past the wavefront's range or past K read as zero through the
// buffer range check (their offsets point past the resource).  The four
// partial accumulators are summed through LDS; wavefront 0 applies the fp32
// epilogue into an LDS tile [token][channel] that the whole workgroup then
// stores row by row (whole 4-byte words from consecutive lanes, instead of
// one 2-byte store per accumulator element).
constexpr int DEC_BN = 16;

constexpr int DEC_WAVES = 4;
// 16-byte loads in flight per lane and chunk: blocks per chunk CH = DEC_LOADS /
// (S + MT).  The weight stream uses the default cache policy (non-temporal
// measured no faster).
constexpr int DEC_LOADS = 16;
// Strip grouping: strips per workgroup until one workgroup per compute unit
// (DEC_SLOTS) covers N, at most DEC_SMAX.
constexpr int DEC_SLOTS = 256;
constexpr int DEC_SMAX = 4;

template <int MT, int S, int CH, bool DBG>
__global__ __launch_bounds__(64 * DEC_WAVES, 1) void k_w4a4_decode(
    const uint8_t* __restrict__ A, const uint16_t* __restrict__ a_scale, int T,
    const uint8_t* __restrict__ W, const uint16_t* __restrict__ w_scale, int N, int K,
    uint16_t* __restrict__ Y, int32_t* __restrict__ acc_dbg) {
  __shared__ v4i s_part[DEC_WAVES - 1][S][MT][64];
  __shared__ uint32_t s_y[64][DEC_BN * S / 2 + 1];  // fp16 outputs, [token][channel pair]
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * (DEC_BN * S);
  const int rowbytes = K / 2;
  // Rows past T (tokens) or N (channels) are outside the buffers' ranges and read as zero.
  const __amdgpu_buffer_rsrc_t rsrc_a =
      __builtin_amdgcn_make_buffer_rsrc((void*)A, 0, T * rowbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsrc_w = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(W + (int64_t)n0 * rowbytes), 0, min(N - n0, DEC_BN * S) * rowbytes, 0x00020000);
  const int kblocks = (K + 127) / 128;
  const int per = (kblocks + DEC_WAVES - 1) / DEC_WAVES;
  const int kb0 = wave * per, kb1 = min(kblocks, kb0 + per);

  v4u wv[2][CH][S], av[2][CH][MT];
  auto load = [&](auto bt, int kb) {
    constexpr int b = decltype(bt)::value;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int byte = (kb + c) * 64 + 16 * g;
      const bool ok = kb + c < kb1 && byte < rowbytes;
#pragma unroll
      for (int s = 0; s < S; ++s)
        wv[b][c][s] = __builtin_bit_cast(
            v4u, __builtin_amdgcn_raw_buffer_load_b128(
                     rsrc_w, ok ? (16 * s + i) * rowbytes + byte : INT32_MIN, 0, 0));
#pragma unroll
      for (int m = 0; m < MT; ++m)
        av[b][c][m] = __builtin_bit_cast(
            v4u, __builtin_amdgcn_raw_buffer_load_b128(
                     rsrc_a, ok ? (16 * m + i) * rowbytes + byte : INT32_MIN, 0, 0));
    }
  };
  v4i acc[S][MT];
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[s][m] = v4i{0, 0, 0, 0};
  auto compute = [&](auto bt) {
    constexpr int b = decltype(bt)::value;
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        v4i ua[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m)
          ua[m] = unpack16(make_uint2(av[b][c][m][2 * e], av[b][c][m][2 * e + 1]));
#pragma unroll
        for (int s = 0; s < S; ++s) {
          const v4i bw = unpack16(make_uint2(wv[b][c][s][2 * e], wv[b][c][s][2 * e + 1]));
#pragma unroll
          for (int m = 0; m < MT; ++m)
            acc[s][m] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ua[m], bw, acc[s][m], 0, 0, 0);
        }
      }
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  if (kb0 < kb1) load(B0{}, kb0);
  for (int kb = kb0; kb < kb1; kb += 2 * CH) {  // buffer indices stay compile-time
    if (kb + CH < kb1) load(B1{}, kb + CH);
    compute(B0{});
    if (kb + CH >= kb1) break;
    if (kb + 2 * CH < kb1) load(B0{}, kb + 2 * CH);
    compute(B1{});
  }
  if (wave > 0) {
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
      for (int m = 0; m < MT; ++m) s_part[wave - 1][s][m][lane] = acc[s][m];
  }
  __syncthreads();
  // Wavefront 0 sums the partial accumulators and applies the epilogue into
  // LDS ([token][channel], fp16); the 16x16 accumulator layout is lane (col i,
  // group g), register r -> row 4 g + r.
  if (wave == 0) {
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int n = n0 + 16 * s + i;
      const float ws = n < N ? h2f(w_scale[n]) : 0.0f;
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        v4i a4 = acc[s][m];
#pragma unroll
        for (int w2 = 0; w2 < DEC_WAVES - 1; ++w2) a4 += s_part[w2][s][m][lane];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * m + 4 * g + r;
          if (t < T) {
            const int32_t a = a4[r] >> 8;  // exact: the accumulator is 256 * acc
            ((uint16_t*)&s_y[t][0])[16 * s + i] =
                f2h(__fmul_rn(__fmul_rn((float)a, h2f(a_scale[t])), ws));
            if (DBG && n < N) acc_dbg[(int64_t)t * N + n] = a;
          }
        }
      }
    }
  }
  __syncthreads();
  // Every thread stores channel pairs: consecutive lanes write consecutive
  // 4-byte words of a token's row (2-byte stores when N is odd).
  constexpr int P = DEC_BN * S / 2;
  const int nloc = min(N - n0, DEC_BN * S);
  for (int idx = tid; idx < T * P; idx += 64 * DEC_WAVES) {
    const int t = idx / P, nl = 2 * (idx - t * P);
    if (nl >= nloc) continue;
    const uint32_t v = s_y[t][nl / 2];
    uint16_t* yp = Y + (int64_t)t * N + n0 + nl;
    if ((N & 1) == 0 && nl + 1 < nloc) {
      *(uint32_t*)yp = v;  // n0 + nl and t N are even, Y is 4-byte aligned
    } else {
      yp[0] = (uint16_t)(v & 0xffffu);
      if (nl + 1 < nloc) yp[1] = (uint16_t)(v >> 16);
    }
  }
}

template <int MT, int S>
static qr_status launch_decode_s(const void* a_q, const void* a_scale, int64_t T, const void* w_q,
                                 const void* w_scale, int64_t N, int64_t K, void* y, int32_t* acc,
                                 hipStream_t stream) {
  // Blocks per load chunk: two chunks of (S + MT) 16-byte loads per lane in flight.
  constexpr int CH = (DEC_LOADS / (S + MT)) > 0 ? DEC_LOADS / (S + MT) : 1;
  const int64_t blocks = (N + DEC_BN * S - 1) / (DEC_BN * S);
  if (acc)
    hipLaunchKernelGGL((k_w4a4_decode<MT, S, CH, true>), dim3((unsigned)blocks), dim3(64 * DEC_WAVES),
                       0, stream, (const uint8_t*)a_q, (const uint16_t*)a_scale, (int)T,
                       (const uint8_t*)w_q, (const uint16_t*)w_scale, (int)N, (int)K,
                       (uint16_t*)y, acc);
  else
    hipLaunchKernelGGL((k_w4a4_decode<MT, S, CH, false>), dim3((unsigned)blocks), dim3(64 * DEC_WAVES),
                       0, stream, (const uint8_t*)a_q, (const uint16_t*)a_scale, (int)T,
                       (const uint8_t*)w_q, (const uint16_t*)w_scale, (int)N, (int)K,
                       (uint16_t*)y, (int32_t*)nullptr);
  return launch_status();
}

// Strips per workgroup.  With one row block of tokens (T <= 16) the weight
// stream is all that matters and one strip per workgroup gives the most
// workgroups; with more tokens every workgroup re-reads all of A through the
// L2, so strips are grouped until one workgroup per compute unit covers N
// (at most 4), which divides that traffic and the unpacking of A.
template <int MT>
static qr_status launch_decode(const void* a_q, const void* a_scale, int64_t T, const void* w_q,
                               const void* w_scale, int64_t N, int64_t K, void* y, int32_t* acc,
                               hipStream_t stream) {
  const int64_t strips = (N + DEC_BN - 1) / DEC_BN;
  const int64_t s =
      MT == 1 ? 1
              : std::min<int64_t>(DEC_SMAX,
                                  std::max<int64_t>(1, (strips + DEC_SLOTS - 1) / DEC_SLOTS));
  switch (s) {
    case 1: return launch_decode_s<MT, 1>(a_q, a_scale, T, w_q, w_scale, N, K, y, acc, stream);
    case 2: return launch_decode_s<MT, 2>(a_q, a_scale, T, w_q, w_scale, N, K, y, acc, stream);
    case 3: return launch_decode_s<MT, 3>(a_q, a_scale, T, w_q, w_scale, N, K, y, acc, stream);
    default: return launch_decode_s<MT, 4>(a_q, a_scale, T, w_q, w_scale, N, K, y, acc, stream);
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
  if (T <= 64 && (int64_t)T * (K / 2) <= INT32_MAX && N <= INT32_MAX / 2) {
    if (T <= 16)
      return launch_decode<1>(a_q, a_scale_f16, T, w_q, w_scale_f16, N, K, y_f16, acc_dbg, stream);
    if (T <= 32)
      return launch_decode<2>(a_q, a_scale_f16, T, w_q, w_scale_f16, N, K, y_f16, acc_dbg, stream);
    return launch_decode<4>(a_q, a_scale_f16, T, w_q, w_scale_f16, N, K, y_f16, acc_dbg, stream);
  }
  return launch_best<4>(a_q, a_scale_f16, T, w_q, w_scale_f16, N, K, y_f16, acc_dbg, stream);
}

extern "C" qr_status qr_w8a8_gemm(const void* a_q, const void* a_scale_f16, int64_t T,
                                  const void* w_q, const void* w_scale_f16, int64_t N, int64_t K,
                                  void* y_f16, int32_t* acc_dbg, hipStream_t stream) {
  if (T < 0 || N < 0 || K <= 0) return QR_ERR_SHAPE;
  if (K % 16 != 0 || K > 131008) return QR_ERR_UNSUPPORTED;
  if (T > INT32_MAX / 2 || N > INT32_MAX / 2) return QR_ERR_SHAPE;
  if (T == 0 || N == 0) return QR_OK;
  if (!a_q || !a_scale_f16 || !w_q || !w_scale_f16 || !y_f16) return QR_ERR_NULL;
  if (!aligned(a_q, 16) || !aligned(w_q, 16) || !aligned(y_f16, 4) || !aligned(a_scale_f16, 2) ||
      !aligned(w_scale_f16, 2) || (acc_dbg && !aligned(acc_dbg, 4)))
    return QR_ERR_ALIGN;
  // no weight-streaming kernel for this format: every T goes through the tiles
  return launch_best<8>(a_q, a_scale_f16, T, w_q, w_scale_f16, N, K, y_f16, acc_dbg, stream);
}

// one instantiation per group size: 64, 128 and 256 fit in one K step of 256
// k, 512 spans two
template <bool KTAIL>
static qr_status launch_groups(const void* a_q, const void* a_s, int64_t T, const void* w_q,
                               const void* w_s, int64_t N, int64_t K, int group, void* y,
                               hipStream_t stream) {
  switch (group) {
    case 64:
      return launch_gemm<2, 2, false, KTAIL, 4, true, 1>(a_q, a_s, T, w_q, w_s, N, K, y, nullptr,
                                                         stream, group);
    case 128:
      return launch_gemm<2, 2, false, KTAIL, 4, true, 2>(a_q, a_s, T, w_q, w_s, N, K, y, nullptr,
                                                         stream, group);
    case 256:
      return launch_gemm<2, 2, false, KTAIL, 4, true, 4>(a_q, a_s, T, w_q, w_s, N, K, y, nullptr,
                                                         stream, group);
    default:  // 512 (the only other size the entry point accepts)
      return launch_gemm<2, 2, false, KTAIL, 4, true, 8>(a_q, a_s, T, w_q, w_s, N, K, y, nullptr,
                                                         stream, group);
  }
}

extern "C" qr_status qr_w4a4_gemm_groups(const void* a_q, const void* a_scale_f16, int64_t T,
                                         const void* w_q, const void* w_scale_f16, int64_t N,
                                         int64_t K, int32_t group, void* y_f16,
                                         hipStream_t stream) {
  if (T < 0 || N < 0 || K <= 0) return QR_ERR_SHAPE;
  if (K % 64 != 0 || K > 131008) return QR_ERR_UNSUPPORTED;
  if (group < 64 || group > 512 || (group & (group - 1)) || K % group) return QR_ERR_UNSUPPORTED;
  if (T > INT32_MAX / 2 || N > INT32_MAX / 2) return QR_ERR_SHAPE;
  if (T == 0 || N == 0) return QR_OK;
  if (!a_q || !a_scale_f16 || !w_q || !w_scale_f16 || !y_f16) return QR_ERR_NULL;
  if (!aligned(a_q, 16) || !aligned(w_q, 16) || !aligned(y_f16, 4) || !aligned(a_scale_f16, 2) ||
      !aligned(w_scale_f16, 2))
    return QR_ERR_ALIGN;
  // 128 x 128 tiles: the fp32 sums sit beside the int32 accumulators
  const bool tail = (K % CodeFmt<4>::BKE) != 0;
  return tail ? launch_groups<true>(a_q, a_scale_f16, T, w_q, w_scale_f16, N, K, group, y_f16, stream)
              : launch_groups<false>(a_q, a_scale_f16, T, w_q, w_scale_f16, N, K, group, y_f16,
                                     stream);
}
