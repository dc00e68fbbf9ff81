// OneBit linear layer: y = ((x ⊙ g) · S^T) ⊙ h with S in {-1, +1} packed as S1-128.
//
// [onebit] "OneBit 框架 / 1. 新的1bit结构" (Fig. 3): the weight is a +-1 matrix and only the
// value vectors g (per input) and h (per output) stay FP16. "讨论与分析 / 1. 效率": with
// binary weights the element products become bit assignments and additions.
//
// t_k = x_k * g_k is exact in fp32 (11-bit x 11-bit significands). A term s * t_k is t_k
// with its sign bit assigned from the packed bit, so the layer is a sum of +-t terms. This
// kernel groups the four inputs of each packed nibble: the 16 possible signed sums of a
// group are built once per workgroup in LDS, and each weight nibble then costs one LDS
// lookup and one fp32 add (about 0.75 VALU ops per weight instead of 2 for XOR-and-add).
//
// Mapping: a 256-thread workgroup = 4 waves = 4 bands of 64 output rows sharing one table;
// lane = output row, streaming its 16-byte S1-128 tile rows (one coalesced 1 KiB load per
// wave per 128 inputs). K is split across workgroups; partial sums are written to the
// workspace and the last workgroup of a band adds them in split order (deterministic) and
// applies h.
#include "bl_internal.h"

namespace bl {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxTableTiles = 16;   // MR * tiles per workgroup <= this (32 KiB of tables)

template <int MR>
__global__ __launch_bounds__(256) void onebit_lut_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ g, const u32x4* __restrict__ S,
    const uint16_t* __restrict__ hvec, int m0, int64_t M, int64_t N, int64_t K,
    float* __restrict__ y, float* __restrict__ ws_part, uint32_t* __restrict__ ws_cnt,
    int tiles_per_split) {
  __shared__ float table[kMaxTableTiles * 32 * 16];      // [m][tile][group][entry]
  __shared__ float tval[kMaxTableTiles * 128];           // [m][tile*128 + c]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int KT = static_cast<int>(K / 128);
  const int split = blockIdx.y, nsplit = gridDim.y;
  const int t0 = split * tiles_per_split;
  const int t1 = min(KT, t0 + tiles_per_split);
  constexpr int CH = kMaxTableTiles / MR;                 // tiles per table build
  const int64_t band = static_cast<int64_t>(blockIdx.x) * 4 + wave;
  const bool active = band * 64 < N;
  const int64_t n = band * 64 + lane;
  const u32x4* sp = S + band * KT * 64 + lane;
  float acc[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) acc[m] = 0.0f;

  for (int c0 = t0; c0 < t1; c0 += CH) {
    const int nt = min(CH, t1 - c0);
    __syncthreads();                                      // previous chunk's table consumed
    // t = x * g for this chunk's inputs (exact)
    for (int i = tid; i < MR * nt * 128; i += 256) {
      const int m = i / (nt * 128), kk = i % (nt * 128);
      const int64_t k = static_cast<int64_t>(c0) * 128 + kk;
      tval[m * nt * 128 + kk] = half_bits_to_float(x[(m0 + m) * K + k]) * half_bits_to_float(g[k]);
    }
    __syncthreads();
    // 16 signed sums per nibble group. Group (tile, word hw, nibble u) holds the inputs at
    // S1-128 bit positions p = 4u + i, i.e. c = 2p (p < 16) or 2(p - 16) + 1.
    for (int i = tid; i < MR * nt * 32 * 16; i += 256) {
      const int e = i & 15, grp = (i >> 4) % (nt * 32), m = (i >> 4) / (nt * 32);
      const int tl = grp >> 5, hw = (grp >> 3) & 3, u = grp & 7;
      const float* tv = tval + m * nt * 128 + tl * 128 + hw * 32;
      float sum = 0.0f;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int p = 4 * u + b;
        const int c = p < 16 ? 2 * p : 2 * (p - 16) + 1;
        const float v = tv[c];
        sum += ((e >> b) & 1) ? -v : v;
      }
      table[(m * nt * 32 + grp) * 16 + e] = sum;
    }
    __syncthreads();
    if (active) {
      for (int tl = 0; tl < nt; ++tl) {
        const u32x4 w = sp[static_cast<int64_t>(c0 + tl) * 64];
        const uint32_t words[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int hw = 0; hw < 4; ++hw) {
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const uint32_t idx = (words[hw] >> (4 * u)) & 15u;
#pragma unroll
            for (int m = 0; m < MR; ++m) acc[m] += table[((m * nt + tl) * 32 + hw * 8 + u) * 16 + idx];
          }
        }
      }
    }
  }
  if (!active) return;
  if (nsplit == 1) {
    const float hn = half_bits_to_float(hvec[n]);
#pragma unroll
    for (int m = 0; m < MR; ++m) y[(m0 + m) * N + n] = acc[m] * hn;
    return;
  }
#pragma unroll
  for (int m = 0; m < MR; ++m) atomic_store_agent(&ws_part[(static_cast<int64_t>(split) * MR + m) * N + n], acc[m]);
  wait_own_memory_ops();
  uint32_t old = 0;
  if (lane == 0) old = arrive_agent(&ws_cnt[band]);
  old = __shfl(old, 0);
  if (old != static_cast<uint32_t>(nsplit - 1)) return;
  const float hn = half_bits_to_float(hvec[n]);
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    float s = 0.0f;
    for (int s0 = 0; s0 < nsplit; s0 += 8) {          // eight loads in flight, summed in order
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        v[j] = s0 + j < nsplit ? atomic_load_agent(&ws_part[(static_cast<int64_t>(s0 + j) * MR + m) * N + n]) : 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) s += v[j];
    }
    y[(m0 + m) * N + n] = s * hn;
  }
  if (lane == 0) reset_agent(&ws_cnt[band]);
}

// OneBit on fp16 matrix cores. y = ((x ⊙ g) S^T) ⊙ h = x · (diag(g) S^T) · diag(h): the
// B operand of v_mfma_f32_16x16x32_f16 is g itself with each element's sign bit set from
// the packed weight bit (the "bit assignment"), so every product x * (+-g) is exact in the
// fp32 accumulator and h is applied once at the end. For a lane holding fp16 pairs
// (inputs c = 8*grp + 2q, 2q + 1 of a 32-input word), the S1-128 bits sit at positions
// 4*grp + q and 16 + 4*grp + q, so one shift and mask put both signs at bits 15 and 31.
// A workgroup = 4 waves = 4 bands of 64 output rows (four 16-row fragments each) for one
// 16-row tile of x and one K range; K splits meet through fp32 partials summed in split
// order by the last workgroup (deterministic), with the loads issued together.
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void onebit_mfma_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ g, const u32x4* __restrict__ S,
    const uint16_t* __restrict__ hvec, int64_t M, int64_t N, int64_t K, float* __restrict__ y,
    float* __restrict__ ws_part, uint32_t* __restrict__ ws_cnt, int tiles_per_split) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = lane >> 4, r16 = lane & 15;
  const int64_t nbands = N / 64;
  const int64_t band = static_cast<int64_t>(blockIdx.x) * 4 + wave;
  const bool active = band < nbands;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * 16;
  const int split = blockIdx.z, nsplit = gridDim.z;
  const int KT = static_cast<int>(K / 128);
  const int t0 = split * tiles_per_split;
  const int t1 = min(KT, t0 + tiles_per_split);
  const bool mrow = m0 + r16 < M;
  const u32x4* xrow = reinterpret_cast<const u32x4*>(x + (mrow ? m0 + r16 : 0) * K);
  const u32x4* g4 = reinterpret_cast<const u32x4*>(g);
  const u32x4* sp = S + (active ? band : 0) * KT * 64 + r16;

  f32x4 acc[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) acc[f] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  if (active) {
    for (int t = t0; t < t1; ++t) {
      u32x4 srow[4];
#pragma unroll
      for (int f = 0; f < 4; ++f) srow[f] = sp[static_cast<int64_t>(t) * 64 + 16 * f];
      u32x4 av[4], gv[4];
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int64_t kb8 = (static_cast<int64_t>(t) * 128 + 32 * st + 8 * grp) / 8;
        av[st] = mrow ? xrow[kb8] : u32x4{0, 0, 0, 0};
        gv[st] = g4[kb8];
      }
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const f16x8 a = __builtin_bit_cast(f16x8, av[st]);
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          const uint32_t word = srow[f][st];
          u32x4 bw;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            bw[q] = gv[st][q] ^ (((word >> (4 * grp + q)) & 0x00010001u) << 15);
          acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, __builtin_bit_cast(f16x8, bw), acc[f], 0, 0, 0);
        }
      }
    }
  }
  if (!active) return;
  // D layout: lane l holds rows 4*(l/16) + i of the x tile, column l % 16 of the fragment.
  if (nsplit == 1) {
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const int64_t n = band * 64 + 16 * f + r16;
      const float hn = half_bits_to_float(hvec[n]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t m = m0 + 4 * grp + i;
        if (m < M) y[m * N + n] = acc[f][i] * hn;
      }
    }
    return;
  }
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t m = m0 + 4 * grp + i, n = band * 64 + 16 * f + r16;
      if (m < M) atomic_store_agent(&ws_part[(static_cast<int64_t>(split) * M + m) * N + n], acc[f][i]);
    }
  wait_own_memory_ops();
  const int64_t cidx = static_cast<int64_t>(blockIdx.y) * nbands + band;
  uint32_t old = 0;
  if (lane == 0) old = arrive_agent(&ws_cnt[cidx]);
  old = __shfl(old, 0);
  if (old != static_cast<uint32_t>(nsplit - 1)) return;
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const int64_t n = band * 64 + 16 * f + r16;
    const float hn = half_bits_to_float(hvec[n]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t m = m0 + 4 * grp + i;
      if (m >= M) continue;
      float s = 0.0f;
      for (int s0 = 0; s0 < nsplit; s0 += 8) {        // eight loads in flight, summed in order
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
          v[j] = s0 + j < nsplit ? atomic_load_agent(&ws_part[(static_cast<int64_t>(s0 + j) * M + m) * N + n]) : 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) s += v[j];
      }
      y[m * N + n] = s * hn;
    }
  }
  if (lane == 0) reset_agent(&ws_cnt[cidx]);
}

struct OnebitPlan { int mr, tps, nsplit; };


OnebitPlan plan_onebit(int64_t M, int64_t N, int64_t K) {
  const int mr = M >= 4 ? 4 : static_cast<int>(M);
  const int64_t KT = K / 128;
  const int64_t bx = (N / 64 + 3) / 4;
  int64_t tps = std::max<int64_t>(4, (KT * bx) / 512);        // aim for ~512 workgroups
  if (N / 64 > kMaxCounters) tps = KT;                         // no split: no counters
  tps = std::min<int64_t>(tps, KT);
  const int64_t nsplit = (KT + tps - 1) / tps;
  return {mr, static_cast<int>(tps), static_cast<int>(nsplit)};
}

// Tuning knob (harnesses that compile this file directly): -1 by M, 0 tables, 1 matrix cores.
int g_onebit_force = -1;

// Measured on MI355X: the nibble tables win for one to three rows, matrix cores from four.
bool onebit_use_mfma(int64_t M) { return g_onebit_force >= 0 ? g_onebit_force == 1 : M > 3; }

struct OnebitMfmaPlan { int64_t groups, mtiles, nsplit, tps; };

OnebitMfmaPlan plan_onebit_mfma(int64_t M, int64_t N, int64_t K) {
  const int64_t KT = K / 128;
  const int64_t groups = (N / 64 + 3) / 4, mtiles = (M + 15) / 16;
  int64_t nsplit = std::max<int64_t>(1, 512 / (groups * mtiles));
  nsplit = std::min<int64_t>(nsplit, std::max<int64_t>(1, KT / 2));
  if (mtiles * (N / 64) > kMaxCounters) nsplit = 1;
  const int64_t tps = (KT + nsplit - 1) / nsplit;
  return {groups, mtiles, (KT + tps - 1) / tps, tps};
}

}  // namespace

int onebit_splits(int64_t M, int64_t N, int64_t K) {
  const OnebitPlan p = plan_onebit(M, N, K);
  return p.nsplit;
}

size_t onebit_part_floats(int64_t M, int64_t N, int64_t K) {
  if (N % 64 || K % 128) return 0;
  const OnebitPlan p = plan_onebit(M, N, K);
  const OnebitMfmaPlan q = plan_onebit_mfma(M, N, K);
  return std::max<size_t>(static_cast<size_t>(p.nsplit) * p.mr * N,
                          static_cast<size_t>(q.nsplit) * M * N);
}

hipError_t launch_onebit(const uint16_t* x, const uint16_t* g, const void* spacked,
                         const uint16_t* h, int64_t M, int64_t N, int64_t K, float* y,
                         float* ws_part, uint32_t* ws_cnt, hipStream_t s) {
  const u32x4* S = static_cast<const u32x4*>(spacked);
  if (onebit_use_mfma(M)) {
    const OnebitMfmaPlan q = plan_onebit_mfma(M, N, K);
    hipLaunchKernelGGL(onebit_mfma_kernel,
                       dim3(static_cast<unsigned>(q.groups), static_cast<unsigned>(q.mtiles),
                            static_cast<unsigned>(q.nsplit)),
                       dim3(256), 0, s, x, g, S, h, M, N, K, y, ws_part, ws_cnt,
                       static_cast<int>(q.tps));
    return hipGetLastError();
  }
  const OnebitPlan p = plan_onebit(M, N, K);
  const dim3 grid(static_cast<unsigned>((N / 64 + 3) / 4), static_cast<unsigned>(p.nsplit));
  for (int64_t m0 = 0; m0 < M; m0 += p.mr) {
    const int mr = static_cast<int>(std::min<int64_t>(p.mr, M - m0));
    const int m0i = static_cast<int>(m0);
#define BL_ONEBIT_LAUNCH(MR_)                                                                \
  hipLaunchKernelGGL(onebit_lut_kernel<MR_>, grid, dim3(256), 0, s, x, g, S, h, m0i, M, N, K, \
                     y, ws_part, ws_cnt, p.tps)
    switch (mr) {
      case 1: BL_ONEBIT_LAUNCH(1); break;
      case 2: BL_ONEBIT_LAUNCH(2); break;
      case 3: BL_ONEBIT_LAUNCH(3); break;
      default: BL_ONEBIT_LAUNCH(4); break;
    }
#undef BL_ONEBIT_LAUNCH
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace bl
