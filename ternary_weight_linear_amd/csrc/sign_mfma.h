// Matrix-core kernel shared by the two fp16-activation layers whose weights are sign planes
// (S1-128): the OneBit layer and the residual-binarisation format.
//
// OneBit:   y[m, n] = h[n] * sum_k x[m, k] * (+-g[k])            (one plane, B = +-g)
// residual: y[m, n] = sum_t a0[n, t] (x_t . B0[n, t]) + a1[n, t] (x_t . B1[n, t])
//                                                                 (two planes, B = +-1)
// The B operand of v_mfma_f32_16x16x32_f16 is built from the packed bits. Lane 16g + u of a
// wave loads the 16-byte S1-128 record 16g + u of a tile: word f holds the signs of row
// 16f + u at the inputs 32s + 8g + 2q + e this lane feeds to the matrix core for slice s,
// at bits 16e + 4s + q. Shifting the word left by 15 - 4s - q puts the pair (e = 0, 1) at
// bits 15 and 31, the sign bits of two fp16 values, so each B register costs one shift and
// one mask-and-combine with g (OneBit) or with 1.0 (residual). Every product x * (+-g) or
// x * (+-1) is exact in the fp32 accumulator.
//
// Mapping: a workgroup of four waves owns one band of 64 output columns (four 16-column
// fragments), one 16-row tile of x and a range of 128-input tiles. The waves take the range's
// tiles in turn (wave w: tiles w, w + 4, ...). Each wave keeps sign_depth() - 1 tiles of loads
// in flight (weights, x and g of a tile are issued together, so the in-order completion of
// vector loads never makes a wave wait on a later tile) and their fp32 results meet in LDS,
// added in wave order. Ranges of one band in different workgroups (a K split, used only when
// the grid would otherwise not fill the chip) meet through fp32 partials in the workspace:
// the last workgroup to arrive adds them in split order, with all of its loads issued
// together. Every sum runs in an order fixed by the shape, so results repeat bit for bit.
#pragma once

#include <algorithm>

#include "bl_internal.h"

namespace bl {

typedef uint32_t sm_u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 sm_f16x8 __attribute__((ext_vector_type(8)));
typedef float sm_f32x4 __attribute__((ext_vector_type(4)));

constexpr int kSignMaxSplits = 16;

struct SignMfmaArgs {
  const uint16_t* x;                           // fp16 [M, K]
  const uint16_t* g;                           // OneBit: fp16 [K]
  const uint16_t* h;                           // OneBit: fp16 [N]
  const sm_u32x4* p0;                          // plane 0, S1-128
  const sm_u32x4* p1;                          // residual: plane 1, S1-128
  const float* a0;                             // residual: fp32 [N, K/128] scales of plane 0
  const float* a1;                             // residual: fp32 [N, K/128] scales of plane 1
  int64_t M, N, K;
  float* y;                                    // fp32 [M, N]
  float* part;                                 // fp32 [nsplit, M, N] (nsplit > 1)
  uint32_t* cnt;                               // one counter per (x tile, band) (nsplit > 1)
  int tiles_per_split;
  uint32_t one;                                // fp16 pair (1.0, 1.0) = 0x3C003C00, passed as
                                               // data so it stays in a register: the sign
                                               // bits then join it in one instruction
};

// Loads of one 128-input tile for one lane.
template <bool RES>
struct SignTile {
  sm_u32x4 s0;                                 // plane 0 record: word f for fragment f
  sm_u32x4 s1;                                 // residual: plane 1 record
  sm_u32x4 xv[4];                              // x[xr, 128t + 32s + 8g ..+7], s = 0..3
  sm_u32x4 gv[RES ? 1 : 4];                    // OneBit: g[128t + 32s + 8g ..+7]
  float c0[RES ? 4 : 1], c1[RES ? 4 : 1];      // residual: scales of column 16f + u
};

// Per-lane byte offsets, fixed for the whole K loop. Each load of a tile is a wave-uniform
// base (scalar registers) plus one of these 32-bit offsets plus an immediate.
struct SignLaneOffsets {
  uint32_t s;    // record of lane l: 16 * l
  uint32_t x;    // x[xr, 8g]: 2 * (xr * K + 8g), xr = u, or row 0 for lanes past M:
                 // those rows only reach output rows >= M, which are never stored
  uint32_t g;    // g[8g]: 16 * g
  uint32_t a;    // scale of column u: 4 * u * KT
};

template <typename T>
__device__ __forceinline__ T sm_load(const void* base, uint32_t off) {
  return *reinterpret_cast<const T*>(static_cast<const char*>(base) + off);
}

template <bool RES>
__device__ __forceinline__ void sign_load_tile(SignTile<RES>& T, const SignMfmaArgs& a,
                                               const SignLaneOffsets& L, int64_t band, int64_t m0,
                                               int t, int KT) {
  const int64_t tile = band * KT + t;
  T.s0 = sm_load<sm_u32x4>(reinterpret_cast<const char*>(a.p0) + (tile << 10), L.s);
  if constexpr (RES) {
    T.s1 = sm_load<sm_u32x4>(reinterpret_cast<const char*>(a.p1) + (tile << 10), L.s);
    const float* c0 = a.a0 + band * 64 * KT + t;
    const float* c1 = a.a1 + band * 64 * KT + t;
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      T.c0[f] = sm_load<float>(c0 + static_cast<int64_t>(16 * f) * KT, L.a);
      T.c1[f] = sm_load<float>(c1 + static_cast<int64_t>(16 * f) * KT, L.a);
    }
  }
  const uint16_t* xb = a.x + m0 * a.K + static_cast<int64_t>(t) * 128;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    T.xv[s] = sm_load<sm_u32x4>(xb + 32 * s, L.x);
    if constexpr (!RES) T.gv[s] = sm_load<sm_u32x4>(a.g + static_cast<int64_t>(t) * 128 + 32 * s, L.g);
  }
}

// Signs of pair q of slice s at bits 15 and 31.
template <int S, int Q>
__device__ __forceinline__ uint32_t sign_pair_bits(uint32_t word) {
  return (word << (15 - 4 * S - Q)) & 0x80008000u;
}

// The same shift for two words held in adjacent registers (hi:lo), as one v_lshlrev_b64 (the
// compiler turns a 64-bit shift by a constant into two 32-bit operations). The shift is at
// most 15, so bits 15 and 31 of the high word still come from the high word alone.
template <int S, int Q>
__device__ __forceinline__ uint64_t sign_pair_shift64(uint64_t words) {
  uint64_t r;
  asm("v_lshlrev_b64 %0, %1, %2" : "=v"(r) : "I"(15 - 4 * S - Q), "v"(words));
  return r;
}

template <bool RES, int S>
__device__ __forceinline__ void sign_slice(const SignTile<RES>& T, sm_f32x4 (&acc)[4],
                                           sm_f32x4 (&p)[4], sm_f32x4 (&r)[4], uint32_t one) {
  const sm_f16x8 av = __builtin_bit_cast(sm_f16x8, T.xv[S]);
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    if constexpr (!RES) {
      const uint32_t w = T.s0[f];
      sm_u32x4 b;
      b[0] = T.gv[S][0] ^ sign_pair_bits<S, 0>(w);
      b[1] = T.gv[S][1] ^ sign_pair_bits<S, 1>(w);
      b[2] = T.gv[S][2] ^ sign_pair_bits<S, 2>(w);
      b[3] = T.gv[S][3] ^ sign_pair_bits<S, 3>(w);
      acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, __builtin_bit_cast(sm_f16x8, b), acc[f], 0, 0, 0);
    } else {
      const uint32_t w0 = T.s0[f], w1 = T.s1[f];
      sm_u32x4 b0, b1;
      b0[0] = one ^ sign_pair_bits<S, 0>(w0);
      b0[1] = one ^ sign_pair_bits<S, 1>(w0);
      b0[2] = one ^ sign_pair_bits<S, 2>(w0);
      b0[3] = one ^ sign_pair_bits<S, 3>(w0);
      b1[0] = one ^ sign_pair_bits<S, 0>(w1);
      b1[1] = one ^ sign_pair_bits<S, 1>(w1);
      b1[2] = one ^ sign_pair_bits<S, 2>(w1);
      b1[3] = one ^ sign_pair_bits<S, 3>(w1);
      p[f] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, __builtin_bit_cast(sm_f16x8, b0), p[f], 0, 0, 0);
      r[f] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, __builtin_bit_cast(sm_f16x8, b1), r[f], 0, 0, 0);
    }
  }
}

template <bool RES>
__device__ __forceinline__ void sign_compute_tile(const SignTile<RES>& T, sm_f32x4 (&acc)[4],
                                                  uint32_t one) {
  sm_f32x4 p[4], r[4];
  if constexpr (RES) {
#pragma unroll
    for (int f = 0; f < 4; ++f) p[f] = r[f] = sm_f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  sign_slice<RES, 0>(T, acc, p, r, one);
  sign_slice<RES, 1>(T, acc, p, r, one);
  sign_slice<RES, 2>(T, acc, p, r, one);
  sign_slice<RES, 3>(T, acc, p, r, one);
  if constexpr (RES) {
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[f][i] += T.c0[f] * p[f][i] + T.c1[f] * r[f][i];
  }
}

// Tile sets per wave: sign_depth() - 1 tiles in flight while one is multiplied.
template <bool RES>
constexpr int sign_depth() { return 3; }

template <bool RES>
__global__ __launch_bounds__(256) void sign_mfma_kernel(const SignMfmaArgs a) {
  constexpr int kPad = 68;                              // LDS row stride (bank spread)
  constexpr int P = sign_depth<RES>();
  __shared__ float red[4][16 * kPad];
  __shared__ uint32_t s_arrived;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = lane >> 4, r16 = lane & 15;
  const int64_t band = blockIdx.x;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * 16;
  const int split = blockIdx.z, nsplit = gridDim.z;
  const int KT = static_cast<int>(a.K / 128);
  const int t0 = split * a.tiles_per_split;
  const int t1 = min(KT, t0 + a.tiles_per_split);
  const bool mrow = m0 + r16 < a.M;
  SignLaneOffsets L;
  L.s = 16u * lane;
  L.x = 2u * ((mrow ? static_cast<uint32_t>(r16) : 0u) * static_cast<uint32_t>(a.K) + 8u * grp);
  L.g = 16u * grp;
  L.a = 4u * static_cast<uint32_t>(r16) * static_cast<uint32_t>(KT);

  sm_f32x4 acc[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) acc[f] = sm_f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  // This wave's tiles: j = 0..n-1 at t0 + wave + 4j.
  const int first = t0 + wave;
  const int n = first < t1 ? (t1 - first + 3) / 4 : 0;
  SignTile<RES> T[P];
#pragma unroll
  for (int d = 0; d < P - 1; ++d)
    if (d < n) sign_load_tile<RES>(T[d], a, L, band, m0, first + 4 * d, KT);
  for (int j0 = 0; j0 < n; j0 += P) {
#pragma unroll
    for (int d = 0; d < P; ++d) {
      const int j = j0 + d;
      if (j < n) {
        if (j + P - 1 < n)
          sign_load_tile<RES>(T[(d + P - 1) % P], a, L, band, m0, first + 4 * (j + P - 1), KT);
        // keep the loads where they are: the scheduler would otherwise sink them towards
        // their use and the tiles in flight would collapse to one
        __builtin_amdgcn_sched_barrier(0);
        sign_compute_tile<RES>(T[d], acc, a.one);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // D layout: lane l holds rows 4*(l/16) + i of the x tile, column l % 16 of fragment f.
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][(4 * f + i) * kPad + lane] = acc[f][i];
  __syncthreads();
  // Thread tid, j: output row ml = 4j + tid/64 of the x tile, column nl = tid % 64 of the band.
  float sum[4];
  int64_t mo[4];
  const int nl = tid & 63;
  const int64_t ncol = band * 64 + nl;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int ml = 4 * j + (tid >> 6);
    const int idx = (4 * (nl >> 4) + (ml & 3)) * kPad + 16 * (ml >> 2) + (nl & 15);
    sum[j] = ((red[0][idx] + red[1][idx]) + red[2][idx]) + red[3][idx];
    mo[j] = m0 + ml;
  }
  const float hn = RES ? 1.0f : half_bits_to_float(a.h[ncol]);
  if (nsplit == 1) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (mo[j] < a.M) a.y[mo[j] * a.N + ncol] = RES ? sum[j] : sum[j] * hn;
    return;
  }
  // nsplit > 1 only when M * N < 2^30 (see plan_sign_mfma): element offsets fit 32 bits.
  const int64_t MN = a.M * a.N;
  uint32_t po[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) po[j] = static_cast<uint32_t>(mo[j] * a.N + ncol);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (mo[j] < a.M) atomic_store_agent(a.part + split * MN + po[j], sum[j]);
  wait_own_memory_ops();
  __syncthreads();
  const int64_t cidx = static_cast<int64_t>(blockIdx.y) * gridDim.x + band;
  if (tid == 0) s_arrived = arrive_agent(&a.cnt[cidx]);
  __syncthreads();
  if (s_arrived != static_cast<uint32_t>(nsplit - 1)) return;   // uniform over the workgroup
  float v[4][kSignMaxSplits];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int s = 0; s < kSignMaxSplits; ++s)
      v[j][s] = (s < nsplit && mo[j] < a.M) ? atomic_load_agent(a.part + s * MN + po[j]) : 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float s = 0.0f;
#pragma unroll
    for (int q = 0; q < kSignMaxSplits; ++q)
      if (q < nsplit) s += v[j][q];                     // split order
    if (mo[j] < a.M) a.y[mo[j] * a.N + ncol] = RES ? s : s * hn;
  }
  if (tid == 0) reset_agent(&a.cnt[cidx]);
}

// ---- staged kernel: decode-sized batches (M <= 4) --------------------------------------
// A workgroup of kStWaves waves owns NF 16-column fragments of a band (NF = 4: the whole
// band; NF = 1: fragment f0, so that a layer of few bands still fills the chip without
// splitting K) and a range of 128-input tiles. It stages x (M rows) and g of its range in
// LDS with all threads at once and issues the sign words its waves need in one burst (the
// lane's S1-128 record, or only word f0 of it; with one fragment per workgroup, part of the burst
// after the staging barrier), so a wave waits for memory about once
// instead of once per tile or two; then it multiplies: A = x from LDS (lanes of rows past M
// read row M - 1; those output rows are never stored), B = g from LDS with the sign bits
// assigned, one v_mfma_f32_16x16x32_f16 per fragment and 32-input slice. The waves' sums
// meet in LDS (over the staging buffer) in wave order.
constexpr int kStWaves = 8;
constexpr int kStLdsBytes = 48 * 1024;                 // x rows and g of one range
constexpr int kStStage = kStLdsBytes / 16 / (64 * kStWaves);   // 16-byte pieces per thread
// 128-input tiles one range may hold: M rows of x and (OneBit) g, 256 bytes each per tile.
__host__ __device__ constexpr int st_max_tiles(int64_t M) {
  return static_cast<int>(kStLdsBytes / ((M + 1) * 256));
}
constexpr int kStMaxPerWave = (st_max_tiles(1) + kStWaves - 1) / kStWaves;
// PW: tiles per wave the kernel is built for (4, 8 or kStMaxPerWave): every one of them is
// loaded (clamped into the range), so short ranges take a smaller build (measured on MI355X,
// 28672 x 8192 at M = 1, 64 tiles per range: 17.0 us built for 12 tiles per wave, 16.3 for
// 8). XG (5..16 rows of x): x is not staged but loaded per tile into registers with the sign
// words (lanes of rows past M load row M - 1), only g goes through LDS; built for PW = 4.
template <bool RES, int NF, int PW, bool XG>
__global__ __launch_bounds__(64 * kStWaves) void sign_staged_kernel(const SignMfmaArgs a) {
  constexpr int kPad = 68;
  static_assert(kStWaves * 4 * NF * kPad * 4 <= kStLdsBytes, "reduction fits the staging buffer");
  __shared__ __attribute__((aligned(16))) uint16_t st[kStLdsBytes / 2];
  __shared__ uint32_t s_arrived;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = lane >> 4, r16 = lane & 15;
  // NF = 1: dispatch ids are dealt round-robin over the 8 XCDs (id i runs on XCD i % 8);
  // ids i, i + 8, i + 16, i + 24 take the four fragments of one band, so they share an XCD
  // and the band's sign records come from HBM once and from that XCD's L2 three times (with
  // consecutive ids per band, every fragment missed in its own XCD's L2: 4x the HBM bytes).
  // The grid is rounded up to 32; ids past the last band have nothing to do.
  const int64_t band = NF == 4 ? blockIdx.x : (blockIdx.x >> 5) * 8 + (blockIdx.x & 7);
  const int f0 = NF == 4 ? 0 : static_cast<int>((blockIdx.x >> 3) & 3);
  if (band >= a.N / 64) return;
  const int split = blockIdx.z, nsplit = gridDim.z;
  const int M = static_cast<int>(a.M);
  const int KT = static_cast<int>(a.K / 128);
  const int t0 = split * a.tiles_per_split;
  const int t1 = min(KT, t0 + a.tiles_per_split);
  const int nt = max(t1 - t0, 0);

  // 1. issue the staging loads (x rows, then g), then the sign words of this wave's tiles (with
  // one fragment per workgroup, part of them after the staging barrier).
  // Every load is unconditional (indices past the range are clamped into it): loads under
  // branches made the compiler wait for each one before issuing the next.
  static_assert(!XG || PW == 4, "registers: x of four tiles per wave");
  constexpr bool kStage = !(XG && RES);                 // anything to stage in LDS
  const int Ms = XG ? 0 : M;                            // rows of x staged
  const int xpieces = Ms * nt * 16, npieces = xpieces + (RES ? 0 : nt * 16);
  sm_u32x4 sv[kStStage];
  if constexpr (kStage) {
#pragma unroll
    for (int i = 0; i < kStStage; ++i) {
      const int pc = min(tid + 64 * kStWaves * i, npieces - 1);
      const int m = pc / (nt * 16), q = pc - m * nt * 16;   // m == Ms: g
      const uint16_t* src = m < Ms ? a.x + static_cast<int64_t>(m) * a.K : a.g;
      sv[i] = *reinterpret_cast<const sm_u32x4*>(src + static_cast<int64_t>(t0) * 128 + 8 * q);
    }
  }
  const int first = t0 + wave;
  const int n = first < t1 ? (t1 - first + kStWaves - 1) / kStWaves : 0;
  uint32_t w0[PW][NF], w1[RES ? PW : 1][NF];
  float c0[RES ? PW : 1][NF], c1[RES ? PW : 1][NF];
  sm_u32x4 xv[XG ? PW : 1][4];
  const uint16_t* xg_row = a.x + static_cast<int64_t>(min(r16, M - 1)) * a.K + 8 * grp;
  const uint32_t soff = 16u * lane + 4u * static_cast<uint32_t>(f0);
  // the sign words (and, at 5..16 rows, x) of the wave's tile j
  auto issue = [&](int j) __attribute__((always_inline)) {
    const int t = min(first + kStWaves * j, t1 - 1);
    const char* rec0 = reinterpret_cast<const char*>(a.p0) + ((band * KT + t) << 10);
    const char* rec1 = reinterpret_cast<const char*>(a.p1) + ((band * KT + t) << 10);
    if constexpr (NF == 4) {
      const sm_u32x4 r0 = sm_load<sm_u32x4>(rec0, soff);
#pragma unroll
      for (int f = 0; f < 4; ++f) w0[j][f] = r0[f];
      if constexpr (RES) {
        const sm_u32x4 r1 = sm_load<sm_u32x4>(rec1, soff);
#pragma unroll
        for (int f = 0; f < 4; ++f) w1[j][f] = r1[f];
      }
    } else {
      // non-temporal (measured on MI355X, 4096^2 at M = 1 / 16: 4.21 -> 3.89 / 7.74 -> 7.49 us;
      // for the whole-band mapping it was slower)
      w0[j][0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(rec0 + soff));
      if constexpr (RES) w1[j][0] = sm_load<uint32_t>(rec1, soff);
    }
    if constexpr (XG) {
#pragma unroll
      for (int sl = 0; sl < 4; ++sl)
        xv[j][sl] = *reinterpret_cast<const sm_u32x4*>(xg_row + static_cast<int64_t>(t) * 128 + 32 * sl);
    }
    if constexpr (RES) {
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const int64_t ci = (band * 64 + 16 * (NF == 4 ? f : f0) + r16) * KT + t;
        c0[j][f] = a.a0[ci];
        c1[j][f] = a.a1[ci];
      }
    }
  };
  // One fragment per workgroup: part of the burst goes out behind the staging loads and the
  // rest after the staging barrier, so that the staging reads of every workgroup are not
  // queued behind all of the sign words (measured on MI355X, 256-layer graph pools, us per
  // layer, whole burst first -> half / three quarters / a quarter before the barrier:
  // OneBit 4096^2 M = 1 3.92 -> 3.74 / 3.81 / 4.00, M = 16 7.48 -> 7.24 / 7.11 / 7.19,
  // residual 4096^2 M = 1 6.58 -> 5.96 / 6.00 / 6.05); the whole-band mapping (NF = 4) keeps
  // the whole burst first (28672 x 8192 at M = 1: 14.7 against 15.3 us with half).
  constexpr int kEarly = NF == 4 ? PW : (XG ? 3 * PW / 4 : PW / 2);
#pragma unroll
  for (int j = 0; j < kEarly; ++j) issue(j);
  // 2. staged pieces to LDS: x row m at m * nt * 128 halves, g after the M rows
  if constexpr (kStage) {
#pragma unroll
    for (int i = 0; i < kStStage; ++i) {
      const int pc = tid + 64 * kStWaves * i;
      if (pc < npieces) *reinterpret_cast<sm_u32x4*>(st + 8 * pc) = sv[i];
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = kEarly; j < PW; ++j) issue(j);

  // 3. products: lane (grp, r16) feeds row min(r16, M - 1) of x and column 16 f + r16
  const uint16_t* xrow = st + static_cast<int64_t>(min(r16, M - 1)) * nt * 128 + 8 * grp;
  const uint16_t* grow = st + static_cast<int64_t>(Ms) * nt * 128 + 8 * grp;
  sm_f32x4 acc[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) acc[f] = sm_f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  // The LDS operands of the next slice (x unless it comes from registers, g for OneBit) are
  // read while the current slice's products run; read just before use, every slice waited
  // for its LDS reads in front of its MFMAs. Past the wave's last tile the reads stay inside
  // the staged range (their values are not used).
  sm_f16x8 an{};
  sm_u32x4 gn{};
  auto read_next = [&](int tile, int sl) __attribute__((always_inline)) {
    const int t = min(tile, nt - 1);
    if constexpr (!XG) an = *reinterpret_cast<const sm_f16x8*>(xrow + t * 128 + 32 * sl);
    if constexpr (!RES) gn = *reinterpret_cast<const sm_u32x4*>(grow + t * 128 + 32 * sl);
  };
  read_next(wave, 0);
#pragma unroll
  for (int j = 0; j < PW; ++j) {
    if (j < n) {
      const int tl = wave + kStWaves * j;   // tile within the range
      sm_f32x4 pp[NF], rr[NF];
      if constexpr (RES) {
#pragma unroll
        for (int f = 0; f < NF; ++f) pp[f] = rr[f] = sm_f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      }
      auto slice = [&](auto sc) __attribute__((always_inline)) {
        constexpr int S = decltype(sc)::value;
        sm_f16x8 av;
        if constexpr (XG) av = __builtin_bit_cast(sm_f16x8, xv[j][S]);
        else av = an;
        const sm_u32x4 gv = gn;
        if constexpr (S < 3) read_next(tl, S + 1);
        else read_next(tl + kStWaves, 0);
        if constexpr (!RES && NF == 4) {
          // one 64-bit shift aligns the words of fragments 2p and 2p + 1 (one sign record,
          // adjacent registers): 12 VALU operations per two MFMAs instead of 16, which are the
          // bound at M = 1 (measured on MI355X, 28672 x 8192 at M = 1: 16.3 -> 15.55 us)
#pragma unroll
          for (int fp = 0; fp < 2; ++fp) {
            const uint64_t pw = (static_cast<uint64_t>(w0[j][2 * fp + 1]) << 32) | w0[j][2 * fp];
            const uint64_t sh[4] = {sign_pair_shift64<S, 0>(pw), sign_pair_shift64<S, 1>(pw),
                                    sign_pair_shift64<S, 2>(pw), sign_pair_shift64<S, 3>(pw)};
            sm_u32x4 b0, b1;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              b0[q] = gv[q] ^ (static_cast<uint32_t>(sh[q]) & 0x80008000u);
              b1[q] = gv[q] ^ (static_cast<uint32_t>(sh[q] >> 32) & 0x80008000u);
            }
            acc[2 * fp] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, __builtin_bit_cast(sm_f16x8, b0), acc[2 * fp], 0, 0, 0);
            acc[2 * fp + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, __builtin_bit_cast(sm_f16x8, b1), acc[2 * fp + 1], 0, 0, 0);
          }
        } else if constexpr (!RES) {
#pragma unroll
          for (int f = 0; f < NF; ++f) {
            sm_u32x4 b;
            b[0] = gv[0] ^ sign_pair_bits<S, 0>(w0[j][f]);
            b[1] = gv[1] ^ sign_pair_bits<S, 1>(w0[j][f]);
            b[2] = gv[2] ^ sign_pair_bits<S, 2>(w0[j][f]);
            b[3] = gv[3] ^ sign_pair_bits<S, 3>(w0[j][f]);
            acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, __builtin_bit_cast(sm_f16x8, b), acc[f], 0, 0, 0);
          }
        } else {
#pragma unroll
          for (int f = 0; f < NF; ++f) {
            sm_u32x4 b0, b1;
            b0[0] = a.one ^ sign_pair_bits<S, 0>(w0[j][f]);
            b0[1] = a.one ^ sign_pair_bits<S, 1>(w0[j][f]);
            b0[2] = a.one ^ sign_pair_bits<S, 2>(w0[j][f]);
            b0[3] = a.one ^ sign_pair_bits<S, 3>(w0[j][f]);
            b1[0] = a.one ^ sign_pair_bits<S, 0>(w1[j][f]);
            b1[1] = a.one ^ sign_pair_bits<S, 1>(w1[j][f]);
            b1[2] = a.one ^ sign_pair_bits<S, 2>(w1[j][f]);
            b1[3] = a.one ^ sign_pair_bits<S, 3>(w1[j][f]);
            pp[f] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, __builtin_bit_cast(sm_f16x8, b0), pp[f], 0, 0, 0);
            rr[f] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, __builtin_bit_cast(sm_f16x8, b1), rr[f], 0, 0, 0);
          }
        }
      };
      slice(std::integral_constant<int, 0>{});
      slice(std::integral_constant<int, 1>{});
      slice(std::integral_constant<int, 2>{});
      slice(std::integral_constant<int, 3>{});
      if constexpr (RES) {
#pragma unroll
        for (int f = 0; f < NF; ++f)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[f][i] += c0[j][f] * pp[f][i] + c1[j][f] * rr[f][i];
      }
    }
  }

  // D layout: lane l holds rows 4*(l/16) + i of x, column l % 16 of fragment f. The sums
  // meet in the staging buffer once every wave is done reading it.
  __syncthreads();
  float* red = reinterpret_cast<float*>(st);
#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[(wave * 4 * NF + 4 * f + i) * kPad + lane] = acc[f][i];
  __syncthreads();
  // output o = tid + 512 j: row ml = o / (16 NF) of x, column nl = o % (16 NF) of the
  // workgroup's columns (threads past the 256 NF outputs only take part in the barriers)
  constexpr int kOutPer = NF == 4 ? 2 : 1;
  float sum[kOutPer];
  int64_t ncol[kOutPer];
  int ml[kOutPer];
  bool live[kOutPer];
#pragma unroll
  for (int q = 0; q < kOutPer; ++q) {
    const int o = tid + 64 * kStWaves * q;
    ml[q] = (o / (16 * NF)) & 15;
    const int nl = o % (16 * NF);
    const int idx = (4 * (nl >> 4) + (ml[q] & 3)) * kPad + 16 * (ml[q] >> 2) + (nl & 15);
    float acc_s = red[idx];
#pragma unroll
    for (int w = 1; w < kStWaves; ++w) acc_s += red[w * 4 * NF * kPad + idx];
    sum[q] = acc_s;
    ncol[q] = band * 64 + 16 * f0 + nl;
    live[q] = o < 256 * NF && ml[q] < M;
  }
  float hn[kOutPer];
#pragma unroll
  for (int q = 0; q < kOutPer; ++q) hn[q] = RES ? 1.0f : half_bits_to_float(a.h[ncol[q]]);
  if (nsplit == 1) {
#pragma unroll
    for (int q = 0; q < kOutPer; ++q)
      if (live[q]) a.y[static_cast<int64_t>(ml[q]) * a.N + ncol[q]] = RES ? sum[q] : sum[q] * hn[q];
    return;
  }
  // nsplit > 1 only when M * N < 2^30 (see plan_sign_mfma): element offsets fit 32 bits.
  const int64_t MN = a.M * a.N;
  uint32_t po[kOutPer];
#pragma unroll
  for (int q = 0; q < kOutPer; ++q) {
    po[q] = static_cast<uint32_t>(ml[q] * a.N + ncol[q]);
    if (live[q]) atomic_store_agent(a.part + split * MN + po[q], sum[q]);
  }
  wait_own_memory_ops();
  __syncthreads();
  if (tid == 0) s_arrived = arrive_agent(&a.cnt[blockIdx.x]);
  __syncthreads();
  if (s_arrived != static_cast<uint32_t>(nsplit - 1)) return;   // uniform over the workgroup
#pragma unroll
  for (int q = 0; q < kOutPer; ++q) {
    float v[kSignMaxSplits];
#pragma unroll
    for (int sp = 0; sp < kSignMaxSplits; ++sp)
      v[sp] = (sp < nsplit && live[q]) ? atomic_load_agent(a.part + sp * MN + po[q]) : 0.0f;
    float t = 0.0f;
#pragma unroll
    for (int sp = 0; sp < kSignMaxSplits; ++sp)
      if (sp < nsplit) t += v[sp];                      // split order
    if (live[q]) a.y[static_cast<int64_t>(ml[q]) * a.N + ncol[q]] = RES ? t : t * hn[q];
  }
  if (tid == 0) reset_agent(&a.cnt[blockIdx.x]);
}

// kernel: 0 = band kernel (sign_mfma_kernel), 1 = staged kernel with one fragment per
// workgroup, 4 = staged kernel with one band per workgroup; xg: x loaded per tile (5..16 rows).
struct SignPlan { int64_t cols, mtiles, nsplit, tps; int kernel; bool xg; };

// Workgroups to aim for (one per CU); the workspace is sized with the same plan.
constexpr int64_t kSignWgTarget = 256;

// Decode-sized batches (M <= 16) take the staged kernel: one fragment per workgroup where
// the bands leave the chip short of `target` workgroups; at M <= 4 (x staged in LDS) one band
// per workgroup otherwise (OneBit only: the residual's two planes and scales would not fit the
// registers of a deep burst); else the band kernel. K is split across workgroups while the
// workgroups still fall short of `target`, and for the staged kernel also where a range would
// not fit (its LDS at M <= 4, four tiles per wave above); at most kSignMaxSplits splits, beyond
// that the band kernel. Each split keeps at least one tile per wave.
inline SignPlan plan_sign_mfma(int64_t M, int64_t N, int64_t K, int64_t target, bool res) {
  const int64_t KT = K / 128, bands = N / 64, mtiles = (M + 15) / 16;
  const bool xg = M > 4;
  int64_t need = 0;   // splits the staged kernel's range bound needs
  int kernel = 0;
  if (M <= 16) {
    const int64_t cap = xg ? 4 * kStWaves : st_max_tiles(M);
    need = (KT + cap - 1) / cap;
    if (need <= kSignMaxSplits) kernel = bands < target ? 1 : (res || xg ? 0 : 4);
  }
  // a K split needs one counter per workgroup column and 32-bit element offsets
  auto can_split = [&](int k) {
    return mtiles * (k == 1 ? 4 * bands + 31 : bands) <= kMaxCounters && M * N < (int64_t(1) << 30);
  };
  if (kernel != 0 && need > 1 && !can_split(kernel)) kernel = 0;
  const int64_t cols = kernel == 1 ? (4 * bands + 31) / 32 * 32 : bands;
  const int64_t per_wave = kernel ? kStWaves : 4;
  int64_t nsplit = (target + cols * mtiles - 1) / (cols * mtiles);
  nsplit = std::min<int64_t>(nsplit, std::max<int64_t>(1, KT / per_wave));
  if (kernel) nsplit = std::max<int64_t>(nsplit, need);
  nsplit = std::min<int64_t>(std::max<int64_t>(nsplit, 1), kSignMaxSplits);
  if (!can_split(kernel)) nsplit = 1;
  const int64_t tps = (KT + nsplit - 1) / nsplit;
  return {cols, mtiles, (KT + tps - 1) / tps, tps, kernel, kernel != 0 && xg};
}

template <bool RES>
inline hipError_t launch_sign_mfma(const SignMfmaArgs& args, hipStream_t s) {
  const SignPlan p = plan_sign_mfma(args.M, args.N, args.K, kSignWgTarget, RES);
  SignMfmaArgs a = args;
  a.tiles_per_split = static_cast<int>(p.tps);
  a.one = 0x3C003C00u;
  const dim3 grid(static_cast<unsigned>(p.cols), static_cast<unsigned>(p.mtiles),
                  static_cast<unsigned>(p.nsplit));
  const dim3 block(64 * kStWaves);
  const bool small = p.tps <= 4 * kStWaves;   // at most four tiles per wave
  const bool mid = p.tps <= 8 * kStWaves;     // at most eight
  if (p.kernel == 1) {
    if (p.xg) hipLaunchKernelGGL((sign_staged_kernel<RES, 1, 4, true>), grid, block, 0, s, a);
    else if (small) hipLaunchKernelGGL((sign_staged_kernel<RES, 1, 4, false>), grid, block, 0, s, a);
    else if (mid) hipLaunchKernelGGL((sign_staged_kernel<RES, 1, 8, false>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((sign_staged_kernel<RES, 1, kStMaxPerWave, false>), grid, block, 0, s, a);
  } else if constexpr (!RES) {
    if (p.kernel == 4) {
      if (small) hipLaunchKernelGGL((sign_staged_kernel<RES, 4, 4, false>), grid, block, 0, s, a);
      else if (mid) hipLaunchKernelGGL((sign_staged_kernel<RES, 4, 8, false>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((sign_staged_kernel<RES, 4, kStMaxPerWave, false>), grid, block, 0, s, a);
    } else {
      hipLaunchKernelGGL(sign_mfma_kernel<RES>, grid, dim3(256), 0, s, a);
    }
  } else {
    hipLaunchKernelGGL(sign_mfma_kernel<RES>, grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

// fp32 partials the kernel needs for a shape under the default plan.
inline size_t sign_mfma_part_floats(int64_t M, int64_t N, int64_t K, bool res) {
  const SignPlan p = plan_sign_mfma(M, N, K, kSignWgTarget, res);
  return p.nsplit > 1 ? static_cast<size_t>(p.nsplit) * M * N : 0;
}

}  // namespace bl
