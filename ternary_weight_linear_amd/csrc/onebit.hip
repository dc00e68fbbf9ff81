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
    for (int sp2 = 0; sp2 < nsplit; ++sp2)
      s += atomic_load_agent(&ws_part[(static_cast<int64_t>(sp2) * MR + m) * N + n]);
    y[(m0 + m) * N + n] = s * hn;
  }
  if (lane == 0) reset_agent(&ws_cnt[band]);
}

struct OnebitPlan { int mr, tps, nsplit; };

OnebitPlan plan_onebit(int64_t M, int64_t N, int64_t K) {
  const int mr = M >= 4 ? 4 : static_cast<int>(M);
  const int64_t KT = K / 128;
  const int64_t bx = (N / 64 + 3) / 4;
  int64_t tps = std::max<int64_t>(1, (KT * bx) / 512);        // aim for ~512 workgroups
  if (N / 64 > kMaxCounters) tps = KT;                         // no split: no counters
  tps = std::min<int64_t>(tps, KT);
  const int64_t nsplit = (KT + tps - 1) / tps;
  return {mr, static_cast<int>(tps), static_cast<int>(nsplit)};
}

}  // namespace

int onebit_splits(int64_t M, int64_t N, int64_t K) {
  const OnebitPlan p = plan_onebit(M, N, K);
  return p.nsplit;
}

hipError_t launch_onebit(const uint16_t* x, const uint16_t* g, const void* spacked,
                         const uint16_t* h, int64_t M, int64_t N, int64_t K, float* y,
                         float* ws_part, uint32_t* ws_cnt, hipStream_t s) {
  const OnebitPlan p = plan_onebit(M, N, K);
  const u32x4* S = static_cast<const u32x4*>(spacked);
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
