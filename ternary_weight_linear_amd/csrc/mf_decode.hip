// Fused quantise + int8-matrix-core product from T2-MF64 weights (decode, M <= 16 tokens).
//
// [b158] "BitNet b1.58 介绍": per-token absmax quantisation of the activations into
// [-127, 127] (gamma = max |x| over the row); "实验及结果", Fig. 3: the product with the
// ternary weights is an int8 accumulation. One launch does the whole linear: gamma, the
// int8 activations, their product with the weights on v_mfma_i32_16x16x64_i8 and the
// scaling epilogue.
//
// Why matrix cores for a matrix-vector product: with T2-MF64 a 64 x 64 weight tile costs a
// lane 16 ALU ops (one AND per operand dword) and four MFMAs, against 34 select + popcount
// ops in the add-only kernel, and quantising an input costs ~10 ops instead of eight ballots
// per tile. The 16 rows of an A operand hold the M <= 16 tokens (rows past M repeat the last
// one; their outputs are never stored), so every M up to 16 reads the weights once.
//
// Mapping: a workgroup of kMW waves owns kMW consecutive 64-row bands (one per wave) and a
// range of 64-input tiles, processed in chunks of up to kChunk tiles:
//  1. the loads that only x feeds are issued first: this thread's share of every row for
//     gamma (through one buffer resource per row, zero past the row's end) and the x it
//     quantises in the first chunk; then the wave's first weight batch;
//  2. gamma per row: integer max over the fp16 bit patterns with the sign cleared (the
//     magnitude order of finite fp16; >= 0x7C00 flags NaN/inf), folded two halves at a time,
//     reduced across the wave with DPP and across waves in LDS;
//  3. the waves quantise the chunk into LDS, q[tile][row][64 inputs] (eight inputs per lane
//     per step, 16-byte loads, one 8-byte LDS store), and add their q to the rows' sums;
//  4. each wave runs its band over the chunk: per tile one 16-byte LDS read (A: row u,
//     inputs 16g .. 16g + 15 for lane 16g + u), four ANDs per weight word (B) and four
//     MFMAs, weights streaming through a ring of register batches refilled as soon as a
//     batch is consumed (buffer loads: zero past the range, so issue is unconditional).
// Epilogue: fragment f's sums are exact multiples of 4^f: shift right by 2f, take away the
// range's sum of q for f < 3, hand the exact int32 partials to the other K splits through
// the split words (one returning atomic each) and scale the total by gamma / 127 and beta.
// The integers equal those of bl_quant_act_int8 followed by the T2-MF64 or T2-PN-64 product.
#include "bl_internal.h"

#include <type_traits>

namespace bl {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr int kMW = 4;                  // waves (bands) per workgroup
constexpr int kMBatch = 4;              // tiles per register batch
constexpr int kMRing = 4;               // register batches per wave
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer resource, 32-bit elements

// q of a workgroup's whole K range sits in LDS: at most kMaxTiles(MR) tiles (48 KiB).
template <int MR>
constexpr int mfd_max_tiles() { return 48 * 1024 / (MR * 64); }
// quantisation steps whose x is loaded with the first weights (more where a range holds
// many rows: each later step waits for loads of its own)
constexpr int mfd_xr(int MR) { return MR >= 8 ? 8 : 2; }
// Weight batches issued before gamma is folded: one up to four rows; none from eight rows on,
// where every workgroup folds eight or more rows of x and weight requests queued ahead of those
// reads delay the fold (measured on MI355X, 70B-shaped decode passes, ms: M = 8 6.08-6.13 ->
// 6.04-6.07, M = 16 7.47 -> 7.36-7.41; at M = 1 none before gamma was slower, 3.93 against 3.79)
constexpr int mfd_pre(int MR) { return MR >= 8 ? 0 : 1; }

// Split-K hand-off of a lane's MR outputs (rows m < M, bit m of `live`, one column): one
// split word per output, or per pair of rows where the split count allows (half the
// atomics). Returns the rows whose totals this lane completed (then in v).
template <int MR>
__device__ __forceinline__ uint32_t hand_over(int32_t (&v)[MR], uint32_t live, int M, int64_t N,
                                              int64_t col, uint64_t* ws_acc, int nsplit) {
  if (nsplit == 1) return live;
  if constexpr (MR >= 2) {
    if (nsplit <= kMaxPairSplits) {
      constexpr int kP = MR / 2;
      const int pairs = (M + 1) / 2;
      auto pword = [&](int e) __attribute__((always_inline)) {
        return ws_acc + static_cast<int64_t>(min(e, pairs - 1)) * N + col;
      };
      const uint32_t pd = split_arrive_pairs<kP>(pword, v, (1u << pairs) - 1, nsplit);
      uint32_t done = 0;
#pragma unroll
      for (int e = 0; e < kP; ++e)
        if ((pd >> e) & 1u) done |= 3u << (2 * e);
      return done & live;
    }
  }
  auto word = [&](int m) __attribute__((always_inline)) {
    return ws_acc + static_cast<int64_t>(min(m, M - 1)) * N + col;
  };
  return split_arrive_batch<MR>(word, v, live, nsplit);
}

template <int MR, int GL>
__global__ __launch_bounds__(64 * kMW) void mf_decode_kernel(
    const uint16_t* __restrict__ x, int M, int64_t K, const u32x4* __restrict__ W,
    const float* __restrict__ beta, int64_t beta_len, int64_t N, float* __restrict__ y,
    uint64_t* __restrict__ ws_acc, int tiles_per_split) {
  constexpr int kMaxTiles = mfd_max_tiles<MR>();
  constexpr int kXR = mfd_xr(MR);
  constexpr int kPre = mfd_pre(MR);
  __shared__ __attribute__((aligned(16))) int8_t qb[kMaxTiles * MR * 64];
  __shared__ uint32_t red_max[kMW][MR];
  __shared__ int rsum[MR];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, u = lane & 15;
  const int64_t nbands = N / 64;
  const int64_t band = static_cast<int64_t>(blockIdx.x) * kMW + wave;
  const bool active = band < nbands;
  const int split = blockIdx.y, nsplit = gridDim.y;
  const int KT = static_cast<int>(K / 64);
  const int t0 = split * tiles_per_split;
  const int t1 = min(KT, t0 + tiles_per_split);   // t1 - t0 <= kMaxTiles (host plan)
  if (tid < MR) rsum[tid] = 0;   // first touched after the gamma barrier

  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<u32x4*>(W + ((active ? band : 0) * KT + t0) * 64), 0,
      active && t1 > t0 ? (t1 - t0) * 1024 : 0, kRsrcWord3);
  u32x4 w[kMRing][kMBatch];
  auto load_batch = [&](u32x4 (&dst)[kMBatch], int rel) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < kMBatch; ++t)
      dst[t] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(   // nt: read once
                                             wr, (rel + t) * 1024 + lane * 16, 0, 2));
    __builtin_amdgcn_sched_barrier(0);   // keep each batch where it is issued
  };

  // Quantisation units: unit v = 8 r + lane / 8 of step r is the wave's tile v / MR (tile
  // t0 + wave + kMW (v / MR) of the range) and row v % MR; the lane takes inputs
  // 8 (lane % 8) .. + 7 of it. Units of rows past M or tiles past the range load clamped
  // data and store nothing.
  const int64_t K8 = K / 8;
  const int wtiles = (t1 - t0 - wave + kMW - 1) / kMW;   // tiles this wave quantises
  const int nsteps = (wtiles * MR + 7) / 8;               // wave-uniform
  auto unit_row = [&](int r) __attribute__((always_inline)) { return (8 * r + (lane >> 3)) % MR; };
  auto unit_tt = [&](int r) __attribute__((always_inline)) {
    return t0 + wave + kMW * ((8 * r + (lane >> 3)) / MR);
  };
  auto load_unit = [&](int r) __attribute__((always_inline)) {
    const int row = min(unit_row(r), M - 1);
    const int tt = min(unit_tt(r), t1 - 1);
    return reinterpret_cast<const u32x4*>(x)[row * K8 + tt * 8 + (lane & 7)];
  };
  u32x4 xv[kXR];

  // 1. gamma loads: row m through a resource of its own (loads past the row read zero),
  // RG rows at a time (register budget); 2. per row, the wave's maximum goes to LDS
  constexpr int RG = GL >= 16 ? 1 : (MR < 4 ? MR : 4);
  {
    u32x4 gx[RG][GL];
    auto issue_rows = [&](int m0) __attribute__((always_inline)) {
#pragma unroll
      for (int mm = 0; mm < RG; ++mm) {
        const int row = min(m0 + mm, M - 1);
        const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(x + static_cast<int64_t>(row) * K), 0,
            static_cast<int>(K * 2), kRsrcWord3);
#pragma unroll
        for (int i = 0; i < GL; ++i)   // the whole offset in the range-checked part
          gx[mm][i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                    xr, (tid + i * 64 * kMW) * 16, 0, 0));
      }
    };
    auto fold_rows = [&](int m0) __attribute__((always_inline)) {
#pragma unroll
      for (int mm = 0; mm < RG; ++mm) {
        u16x2 m2 = {0, 0};
#pragma unroll
        for (int i = 0; i < GL; ++i) {
          const uint32_t w4[4] = {gx[mm][i].x, gx[mm][i].y, gx[mm][i].z, gx[mm][i].w};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2, w4[e] & 0x7FFF7FFFu));
        }
        const uint32_t v =
            wave_max_u32(max(static_cast<uint32_t>(m2.x), static_cast<uint32_t>(m2.y)));
        if (lane == 0) red_max[wave][m0 + mm] = v;
      }
    };
    // kPre weight batches are issued behind the x loads (vector loads complete in issue
    // order, so the folds wait only for x); the rest of the ring goes out between the
    // quantisation steps: the texture path takes ~16 cycles per KiB per CU, and a longer
    // queue in front would hold the gamma loads of the other waves back
    if constexpr (MR == RG) {   // every row in one go, issued before the weights
      issue_rows(0);
#pragma unroll
      for (int r = 0; r < kXR; ++r) xv[r] = load_unit(r);
#pragma unroll
      for (int r = 0; r < kPre; ++r) load_batch(w[r], r * kMBatch);
      fold_rows(0);
    } else {
#pragma unroll
      for (int r = 0; r < kXR; ++r) xv[r] = load_unit(r);
#pragma unroll
      for (int r = 0; r < kPre; ++r) load_batch(w[r], r * kMBatch);
#pragma unroll 1
      for (int m0 = 0; m0 < MR; m0 += RG) {
        issue_rows(m0);
        fold_rows(m0);
      }
    }
  }
  __syncthreads();
  auto row_gamma = [&](int m, float& gam, float& rg, bool& zero) __attribute__((always_inline)) {
    uint32_t v = red_max[0][m];
#pragma unroll
    for (int w2 = 1; w2 < kMW; ++w2) v = max(v, red_max[w2][m]);
    const bool bad = v >= 0x7C00u;
    gam = bad ? __uint_as_float(0x7FC00000u) : half_bits_to_float(static_cast<uint16_t>(v));
    zero = bad || v == 0u;
    rg = __builtin_amdgcn_rcpf(zero ? 1.0f : gam);
  };
  // the rows this lane quantises: one per step parity (MR = 16), else one
  constexpr int kQR = MR == 16 ? 2 : 1;
  float qg[kQR], qrg[kQR];
  bool qz[kQR];
#pragma unroll
  for (int p = 0; p < kQR; ++p) row_gamma(unit_row(p), qg[p], qrg[p], qz[p]);
  int qs[kQR];
#pragma unroll
  for (int p = 0; p < kQR; ++p) qs[p] = 0;

  // 3. quantise the range into LDS, q[tile - t0][row][64 inputs]
  auto quantise = [&](const u32x4& xr, int r, int p) __attribute__((always_inline)) {
    // p = r % kQR, a constant at every call
    const int row = unit_row(r), tt = unit_tt(r);
    const uint32_t h[4] = {xr.x, xr.y, xr.z, xr.w};
    float a[8], ge[8], rge[8];
    bool ze[8];
    int q[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = half_bits_to_float(static_cast<uint16_t>(h[e / 2] >> (16 * (e % 2)))) * 127.0f;
      ge[e] = qg[p], rge[e] = qrg[p], ze[e] = qz[p];
    }
    quant_q_n(a, ge, rge, ze, q);
    // bytes in input order: perm picks the low byte of each 16-bit half
    const uint32_t d0 = __builtin_amdgcn_perm(
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pk_i16(q[2], q[3])),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pk_i16(q[0], q[1])), 0x06040200u);
    const uint32_t d1 = __builtin_amdgcn_perm(
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pk_i16(q[6], q[7])),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pk_i16(q[4], q[5])), 0x06040200u);
    if (row < M && tt < t1) {
      qs[p] = __builtin_amdgcn_sdot4(static_cast<int>(d0), 0x01010101, qs[p], false);
      qs[p] = __builtin_amdgcn_sdot4(static_cast<int>(d1), 0x01010101, qs[p], false);
      *reinterpret_cast<uint2*>(&qb[((tt - t0) * MR + row) * 64 + 8 * (lane & 7)]) =
          make_uint2(d0, d1);
    }
  };
  // the first kXR steps from registers; further steps (long ranges, many rows) load as
  // they go
  static_assert(kXR % kQR == 0, "steps keep their row parity");
#pragma unroll
  for (int r = 0; r < kXR; ++r) {
    if (kPre + r < kMRing) load_batch(w[kPre + r], (kPre + r) * kMBatch);
    if (r < nsteps) quantise(xv[r], r, r % kQR);
  }
#pragma unroll
  for (int r = kPre + kXR; r < kMRing; ++r) load_batch(w[r], r * kMBatch);
  for (int r = kXR; r < nsteps; r += kQR) {
#pragma unroll
    for (int p = 0; p < kQR; ++p)
      if (r + p < nsteps) quantise(load_unit(r + p), r + p, p);
  }
  // the rows' sums: lanes 8k .. 8k + 7 share a unit row, (8p + k) % MR for parity p; sum
  // each group of eight with DPP, gather the groups in scalars, one LDS add per row
  // (a same-address LDS atomic from every lane is compiled into a 64-step scalar loop)
  {
    int rs[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) rs[m] = 0;
#pragma unroll
    for (int p = 0; p < kQR; ++p) {
      const int v = group8_sum_i32(qs[p]);
#pragma unroll
      for (int k = 0; k < 8; ++k) rs[(8 * p + k) % MR] += __builtin_amdgcn_readlane(v, 8 * k);
    }
    if (lane == 0) {
#pragma unroll
      for (int m = 0; m < MR; ++m)
        if (m < M) __hip_atomic_fetch_add(&rsum[m], rs[m], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
  }
  __syncthreads();

  // 4. the band over the range: batch i sits in ring slot i % kMRing; once consumed, the
  // slot is refilled with batch i + kMRing (past the range it reads zero for free)
  i32x4 acc[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) acc[f] = i32x4{0, 0, 0, 0};
  const int rowu = min(u, M - 1);   // A operand row of this lane (M <= MR)
  if (active) {
    for (int tb = t0; tb < t1; tb += kMRing * kMBatch) {
#pragma unroll
      for (int r = 0; r < kMRing; ++r) {
        const int tr = tb + r * kMBatch;
        if (tr < t1) {   // tiles past the range hold zero weights; their q index is clamped
#pragma unroll
          for (int t = 0; t < kMBatch; ++t) {
            const int pt = min(tr + t - t0, kMaxTiles - 1);
            const i32x4 av = *reinterpret_cast<const i32x4*>(&qb[(pt * MR + rowu) * 64 + 16 * g]);
            const uint32_t w4[4] = {w[r][t].x, w[r][t].y, w[r][t].z, w[r][t].w};
#pragma unroll
            for (int f = 0; f < 4; ++f) {
              i32x4 b;
#pragma unroll
              for (int j = 0; j < 4; ++j) b[j] = static_cast<int>(w4[j] & (0x03030303u << (2 * f)));
              acc[f] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, b, acc[f], 0, 0, 0);
            }
          }
        }
        load_batch(w[r], tr - t0 + kMRing * kMBatch);
      }
    }
  }
  if (!active) return;
  // Outputs to lane = column within the wave (ds_bpermute, no LDS traffic between waves):
  // row m, column 16f + u sits in lane 16 (m / 4) + u, element m % 4 of fragment f. Each
  // lane then hands over at most MR outputs, all of them live for rows < M (from the MFMA
  // layout directly a lane would hold 16 outputs, most of them for rows past M).
  const int64_t col = band * 64 + lane;
  int32_t v[MR];
  uint32_t live = 0;
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    const int src = (16 * (m >> 2) + (lane & 15)) * 4;
    int got = 0;
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const int t = __builtin_amdgcn_ds_bpermute(src, (acc[f][m & 3] >> (2 * f)) - (f < 3 ? rsum[min(m, MR - 1)] : 0));
      got = (lane >> 4) == f ? t : got;
    }
    v[m] = got;
    if (m < M) live |= 1u << m;
  }
  const uint32_t done = hand_over<MR>(v, live, M, N, col, ws_acc, nsplit);
  const float b = beta[beta_len == 1 ? 0 : col];
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    if (!((done >> m) & 1u)) continue;
    float gam, rg;
    bool zero;
    row_gamma(m, gam, rg, zero);
    y[m * N + col] = static_cast<float>(v[m]) * (gam / 127.0f) * b;
  }
}

// The same product with q given (int8 [M, K], gamma [M], rowsum [M] from the quantiser):
// the workgroup copies q of its K range into LDS (QL 16-byte loads per thread, issued
// before the weights, addresses past the copy clamped), streams its four bands through the
// register ring as above, and hands the raw fragment sums to the split words; the workgroup
// completing an output takes the row's whole-K sum of q away once (fragments f < 3), so no
// per-range sums are needed.
template <int MR, int QL>
__global__ __launch_bounds__(64 * kMW) void mf_qgemv_kernel(
    const int8_t* __restrict__ q, const float* __restrict__ gamma,
    const int32_t* __restrict__ rowsum, int M, int64_t K, const u32x4* __restrict__ W,
    const float* __restrict__ beta, int64_t beta_len, int64_t N, float* __restrict__ y,
    int32_t* __restrict__ acc_out, uint64_t* __restrict__ ws_acc, int tiles_per_split) {
  constexpr int kMaxTiles = mfd_max_tiles<MR>();
  __shared__ __attribute__((aligned(16))) int8_t qb[kMaxTiles * MR * 64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, u = lane & 15;
  const int64_t nbands = N / 64;
  const int64_t band = static_cast<int64_t>(blockIdx.x) * kMW + wave;
  const bool active = band < nbands;
  const int split = blockIdx.y, nsplit = gridDim.y;
  const int KT = static_cast<int>(K / 64);
  const int t0 = split * tiles_per_split;
  const int t1 = min(KT, t0 + tiles_per_split);   // t1 - t0 <= kMaxTiles (host plan)

  // the epilogue's row sums and scales, lane l holding row min(l, M - 1) (read back with
  // readlane), loaded first so that no load waits at the end
  const int rs_l = rowsum[min(lane, M - 1)];
  const float gs_l = y != nullptr ? gamma[min(lane, M - 1)] / 127.0f : 0.0f;
  // q of the range: unit i = (tile i / (4 M), row (i / 4) % M, 16-byte piece i % 4); the
  // host picks QL with QL * 256 >= the range's units
  const int units = (t1 - t0) * M * 4;
  u32x4 qv[QL];
#pragma unroll
  for (int l = 0; l < QL; ++l) {
    const int i = min(tid + 64 * kMW * l, units - 1);
    const int tile = i / (4 * M), row = (i >> 2) % M;
    qv[l] = *reinterpret_cast<const u32x4*>(q + static_cast<int64_t>(row) * K +
                                             static_cast<int64_t>(t0 + tile) * 64 + 16 * (i & 3));
  }
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<u32x4*>(W + ((active ? band : 0) * KT + t0) * 64), 0,
      active && t1 > t0 ? (t1 - t0) * 1024 : 0, kRsrcWord3);
  u32x4 w[kMRing][kMBatch];
  auto load_batch = [&](u32x4 (&dst)[kMBatch], int rel) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < kMBatch; ++t)
      dst[t] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(   // nt: read once
                                             wr, (rel + t) * 1024 + lane * 16, 0, 2));
    __builtin_amdgcn_sched_barrier(0);   // keep each batch where it is issued
  };
#pragma unroll
  for (int r = 0; r < kMRing; ++r) load_batch(w[r], r * kMBatch);
#pragma unroll
  for (int l = 0; l < QL; ++l) {
    const int i = tid + 64 * kMW * l;
    if (i < units) {
      const int tile = i / (4 * M), row = (i >> 2) % M;
      *reinterpret_cast<u32x4*>(&qb[(tile * MR + row) * 64 + 16 * (i & 3)]) = qv[l];
    }
  }
  __syncthreads();

  i32x4 acc[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) acc[f] = i32x4{0, 0, 0, 0};
  const int rowu = min(u, M - 1);   // A operand row of this lane (M <= MR)
  if (!active) return;
  for (int tb = t0; tb < t1; tb += kMRing * kMBatch) {
#pragma unroll
    for (int r = 0; r < kMRing; ++r) {
      const int tr = tb + r * kMBatch;
      if (tr < t1) {   // tiles past the range hold zero weights; their q index is clamped
#pragma unroll
        for (int t = 0; t < kMBatch; ++t) {
          const int pt = min(tr + t - t0, kMaxTiles - 1);
          const i32x4 av = *reinterpret_cast<const i32x4*>(&qb[(pt * MR + rowu) * 64 + 16 * g]);
          const uint32_t w4[4] = {w[r][t].x, w[r][t].y, w[r][t].z, w[r][t].w};
#pragma unroll
          for (int f = 0; f < 4; ++f) {
            i32x4 b;
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = static_cast<int>(w4[j] & (0x03030303u << (2 * f)));
            acc[f] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, b, acc[f], 0, 0, 0);
          }
        }
      }
      load_batch(w[r], tr - t0 + kMRing * kMBatch);
    }
  }
  // outputs to lane = column (as above); raw fragment sums, at most MR per lane
  const int64_t col = band * 64 + lane;
  int32_t v[MR];
  uint32_t live = 0;
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    const int src = (16 * (m >> 2) + (lane & 15)) * 4;
    int got = 0;
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const int t = __builtin_amdgcn_ds_bpermute(src, acc[f][m & 3] >> (2 * f));
      got = (lane >> 4) == f ? t : got;
    }
    v[m] = got;
    if (m < M) live |= 1u << m;
  }
  const uint32_t done = hand_over<MR>(v, live, M, N, col, ws_acc, nsplit);
  const float b = y != nullptr ? beta[beta_len == 1 ? 0 : col] : 0.0f;
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    if (!((done >> m) & 1u)) continue;
    const int r = v[m] - (lane < 48 ? __builtin_amdgcn_readlane(rs_l, m) : 0);   // f < 3: q (w + 1)
    if (acc_out) acc_out[m * N + col] = r;
    if (y)
      y[m * N + col] = static_cast<float>(r) *
                       __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gs_l), m)) * b;
  }
}

struct MfdPlan { int64_t groups, nsplit, tps; };

int mfd_rows(int M) { return M == 1 ? 1 : M == 2 ? 2 : M <= 4 ? 4 : M <= 8 ? 8 : 16; }

int mfd_tiles_cap(int MR) {
  switch (MR) {
    case 1: return mfd_max_tiles<1>();
    case 2: return mfd_max_tiles<2>();
    case 4: return mfd_max_tiles<4>();
    case 8: return mfd_max_tiles<8>();
    default: return mfd_max_tiles<16>();
  }
}

MfdPlan plan_mf_decode(int M, int64_t N, int64_t K) {
  const int64_t max_tiles = mfd_tiles_cap(mfd_rows(M));
  const int64_t bands = N / 64;
  const int64_t groups = (bands + kMW - 1) / kMW;
  const int64_t KT = K / 64;
  // as the add-only kernel: one workgroup per CU for narrow outputs, two for wide ones,
  // never more than the target (a partial extra wave of workgroups would run last)
  const int64_t target = bands < 512 ? 256 : 512;
  int64_t nsplit = std::max<int64_t>(1, target / groups);
  nsplit = std::min<int64_t>(nsplit, std::max<int64_t>(1, KT / kMBatch));
  // q of a whole range sits in LDS: at least KT / max_tiles splits
  nsplit = std::max<int64_t>(nsplit, (KT + max_tiles - 1) / max_tiles);
  nsplit = std::min<int64_t>(nsplit, kMaxIntSplits);
  if (static_cast<int64_t>(M) * N > kAccCap || K > kMaxIntSplitK) nsplit = 1;
  const int64_t tps = (KT + nsplit - 1) / nsplit;
  if (tps > max_tiles) return {0, 0, 0};   // a range would not fit: not this kernel
  return {groups, (KT + tps - 1) / tps, tps};
}

}  // namespace

bool mf_decode_fits(int64_t M, int64_t N, int64_t K) {
  return M >= 1 && M <= 16 && K <= 32768 && plan_mf_decode(static_cast<int>(M), N, K).groups > 0;
}

bool mf_qgemv_fits(int64_t M, int64_t N, int64_t K) { return mf_decode_fits(M, N, K); }

hipError_t launch_mf_qgemv(const int8_t* q, const float* gamma, const int32_t* rowsum, int M,
                           int64_t K, const void* wmf, const float* beta, int64_t beta_len,
                           int64_t N, float* y, int32_t* acc_out, uint64_t* ws_acc,
                           hipStream_t s) {
  if (!mf_qgemv_fits(M, N, K)) return hipErrorInvalidValue;
  const MfdPlan p = plan_mf_decode(M, N, K);
  const dim3 grid(static_cast<unsigned>(p.groups), static_cast<unsigned>(p.nsplit));
  const u32x4* W = static_cast<const u32x4*>(wmf);
  // 16-byte pieces of q per workgroup: <= 4 per thread (copy of up to 1024), else <= 12
  // (the LDS bound: kMaxTiles(MR) * MR * 4 = 3072 pieces)
  const bool few = p.tps * M * 4 <= 64 * kMW * 4;
#define BL_MFQ2(MR_, QL_)                                                                   \
  hipLaunchKernelGGL((mf_qgemv_kernel<MR_, QL_>), grid, dim3(64 * kMW), 0, s, q, gamma,   \
                     rowsum, M, K, W, beta, beta_len, N, y, acc_out, ws_acc,               \
                     static_cast<int>(p.tps))
#define BL_MFQ(MR_)               \
  do {                            \
    if (few) BL_MFQ2(MR_, 4);     \
    else BL_MFQ2(MR_, 12);        \
  } while (0)
  if (M == 1) BL_MFQ(1);
  else if (M == 2) BL_MFQ(2);
  else if (M <= 4) BL_MFQ(4);
  else if (M <= 8) BL_MFQ(8);
  else BL_MFQ(16);
#undef BL_MFQ
#undef BL_MFQ2
  return hipGetLastError();
}

hipError_t launch_mf_decode(const uint16_t* x, int M, int64_t K, const void* wmf,
                            const float* beta, int64_t beta_len, int64_t N, float* y,
                            uint64_t* ws_acc, hipStream_t s) {
  if (!mf_decode_fits(M, N, K)) return hipErrorInvalidValue;
  const MfdPlan p = plan_mf_decode(M, N, K);
  const dim3 grid(static_cast<unsigned>(p.groups), static_cast<unsigned>(p.nsplit));
  const u32x4* W = static_cast<const u32x4*>(wmf);
  // gamma loads per thread and row: K <= 8 * 64 kMW GL
  const bool longrow = K > 8 * 64 * kMW * 4;
#define BL_MFD(MR_)                                                                        \
  do {                                                                                     \
    if (longrow)                                                                           \
      hipLaunchKernelGGL((mf_decode_kernel<MR_, 16>), grid, dim3(64 * kMW), 0, s, x, M, K, \
                         W, beta, beta_len, N, y, ws_acc, static_cast<int>(p.tps));        \
    else                                                                                   \
      hipLaunchKernelGGL((mf_decode_kernel<MR_, 4>), grid, dim3(64 * kMW), 0, s, x, M, K,  \
                         W, beta, beta_len, N, y, ws_acc, static_cast<int>(p.tps));        \
  } while (0)
  if (M == 1) BL_MFD(1);
  else if (M == 2) BL_MFD(2);
  else if (M <= 4) BL_MFD(4);
  else if (M <= 8) BL_MFD(8);
  else BL_MFD(16);
#undef BL_MFD
  return hipGetLastError();
}

}  // namespace bl
