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

struct SignPlan { int64_t bands, mtiles, nsplit, tps; };

// Workgroups to aim for. Tuning harnesses that compile the sources directly may set it
// (0 = the default); the workspace is sized for the default.
constexpr int64_t kSignWgTarget = 256;
inline int64_t sign_wg_target() { return kSignWgTarget; }

// Splits K across workgroups only while bands x x-tiles leaves the chip short of `target`
// workgroups; each split keeps at least one tile per wave.
inline SignPlan plan_sign_mfma(int64_t M, int64_t N, int64_t K, int64_t target) {
  const int64_t KT = K / 128, bands = N / 64, mtiles = (M + 15) / 16;
  int64_t nsplit = (target + bands * mtiles - 1) / (bands * mtiles);
  nsplit = std::min<int64_t>(nsplit, std::max<int64_t>(1, KT / 4));
  nsplit = std::min<int64_t>(std::max<int64_t>(nsplit, 1), kSignMaxSplits);
  if (mtiles * bands > kMaxCounters || M * N >= (int64_t(1) << 30)) nsplit = 1;
  const int64_t tps = (KT + nsplit - 1) / nsplit;
  return {bands, mtiles, (KT + tps - 1) / tps, tps};
}

template <bool RES>
inline hipError_t launch_sign_mfma(const SignMfmaArgs& args, hipStream_t s) {
  const SignPlan p = plan_sign_mfma(args.M, args.N, args.K, sign_wg_target());
  SignMfmaArgs a = args;
  a.tiles_per_split = static_cast<int>(p.tps);
  a.one = 0x3C003C00u;
  hipLaunchKernelGGL(sign_mfma_kernel<RES>,
                     dim3(static_cast<unsigned>(p.bands), static_cast<unsigned>(p.mtiles),
                          static_cast<unsigned>(p.nsplit)),
                     dim3(256), 0, s, a);
  return hipGetLastError();
}

// fp32 partials the kernel needs for a shape under the default plan.
inline size_t sign_mfma_part_floats(int64_t M, int64_t N, int64_t K) {
  const SignPlan p = plan_sign_mfma(M, N, K, kSignWgTarget);
  return p.nsplit > 1 ? static_cast<size_t>(p.nsplit) * M * N : 0;
}

}  // namespace bl
