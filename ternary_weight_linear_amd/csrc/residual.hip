// Residual binarisation as an inference format: W ~ alpha_o ⊙ B_o + alpha_r ⊙ B_r.
//
// [billm] "方法细节", step 2 (binary residual approximation): the weight is binarised once
// and the residual of that approximation is binarised again; the sum of the two scaled sign
// matrices replaces W. Here every group is one output row by 128 consecutive inputs (one
// S1-128 tile row), each group carrying two fp32 scales, and the two sign planes use the
// S1-128 layout of the OneBit path.
//
// Packing (offline): alpha is the group's mean magnitude, formed in fp32 as a balanced
// pairwise sum in input order times 1/128. A wave holds one group with inputs 2l, 2l+1 in
// lane l: the lane adds its pair, then a butterfly over lanes 1, 2, 4, ..., 32 apart adds
// pairs of pairs, which is exactly that tree (fp32 addition is commutative, so every lane
// ends with the same bits). The residual R = W -+ alpha_o is one fp32 rounding, and the
// lanes' sign bits are gathered into S1-128 words with two ballots.
//
// Forward: y[m, n] = sum_b alpha_o[n, b] (x_b . B_o[n, b]) + alpha_r[n, b] (x_b . B_r[n, b]).
// Both group dot products run on fp16 matrix cores with B = +-1.0 built from the packed
// bits (the products x * +-1 are exact); each 128-input tile's two fp32 results are scaled
// by the lane's own column scales and added to the running sum. Mapping, K splitting and
// the deterministic in-order sum of the split partials follow the OneBit matrix-core kernel.
#include <algorithm>

#include "bl_internal.h"

namespace bl {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float wave_pair_tree_sum(float v) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) v += __shfl_xor(v, off);
  return v;
}

// Two ballots (even inputs, odd inputs) -> the four S1-128 words of one tile row.
__device__ __forceinline__ u32x4 s1_words(uint64_t even, uint64_t odd) {
  u32x4 w;
#pragma unroll
  for (int h = 0; h < 4; ++h)
    w[h] = static_cast<uint32_t>((even >> (16 * h)) & 0xFFFFu) |
           (static_cast<uint32_t>((odd >> (16 * h)) & 0xFFFFu) << 16);
  return w;
}

__global__ __launch_bounds__(256) void residual_pack_kernel(
    const float* __restrict__ W, int64_t N, int64_t K, u32x4* __restrict__ Po,
    float* __restrict__ alpha_o, u32x4* __restrict__ Pr, float* __restrict__ alpha_r) {
  const int lane = threadIdx.x & 63;
  const int64_t KB = K / 128;
  const int64_t item = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (item >= N * KB) return;                           // whole waves leave together
  const int64_t n = item / KB, b = item % KB;
  const float2 w = reinterpret_cast<const float2*>(W + n * K + b * 128)[lane];
  const float ao = wave_pair_tree_sum(fabsf(w.x) + fabsf(w.y)) * (1.0f / 128.0f);
  const bool n0 = w.x < 0.0f, n1 = w.y < 0.0f;
  const float r0 = w.x - (n0 ? -ao : ao);
  const float r1 = w.y - (n1 ? -ao : ao);
  const float ar = wave_pair_tree_sum(fabsf(r0) + fabsf(r1)) * (1.0f / 128.0f);
  const uint64_t bo_e = __builtin_amdgcn_ballot_w64(n0), bo_o = __builtin_amdgcn_ballot_w64(n1);
  const uint64_t br_e = __builtin_amdgcn_ballot_w64(r0 < 0.0f);
  const uint64_t br_o = __builtin_amdgcn_ballot_w64(r1 < 0.0f);
  if (lane == 0) {
    const int64_t row = ((n >> 6) * KB + b) * 64 + (n & 63);
    Po[row] = s1_words(bo_e, bo_o);
    Pr[row] = s1_words(br_e, br_o);
    alpha_o[n * KB + b] = ao;
    alpha_r[n * KB + b] = ar;
  }
}

// fp16 +-1.0 pairs for the MFMA B operand: the lane's inputs 8*grp + 2q, 2q + 1 of a
// 32-input word sit at S1-128 bits 4*grp + q and 16 + 4*grp + q.
__device__ __forceinline__ f16x8 pm_one(uint32_t word, int grp) {
  u32x4 r;
#pragma unroll
  for (int q = 0; q < 4; ++q) r[q] = 0x3C003C00u | (((word >> (4 * grp + q)) & 0x00010001u) << 15);
  return __builtin_bit_cast(f16x8, r);
}

__global__ __launch_bounds__(256) void residual_mfma_kernel(
    const uint16_t* __restrict__ x, const u32x4* __restrict__ Po, const float* __restrict__ alpha_o,
    const u32x4* __restrict__ Pr, const float* __restrict__ alpha_r, int64_t M, int64_t N,
    int64_t K, float* __restrict__ y, float* __restrict__ ws_part, uint32_t* __restrict__ ws_cnt,
    int tiles_per_split) {
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
  const int64_t bandc = active ? band : 0;
  const u32x4* po = Po + bandc * KT * 64 + r16;
  const u32x4* pr = Pr + bandc * KT * 64 + r16;
  const float* ao = alpha_o + (bandc * 64 + r16) * KT;   // column 16f + r16: + 16 f KT
  const float* ar = alpha_r + (bandc * 64 + r16) * KT;

  f32x4 acc[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) acc[f] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  if (active) {
    for (int t = t0; t < t1; ++t) {
      u32x4 so[4], sr[4];
      float sco[4], scr[4];
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        so[f] = po[static_cast<int64_t>(t) * 64 + 16 * f];
        sr[f] = pr[static_cast<int64_t>(t) * 64 + 16 * f];
        sco[f] = ao[static_cast<int64_t>(16 * f) * KT + t];
        scr[f] = ar[static_cast<int64_t>(16 * f) * KT + t];
      }
      u32x4 av[4];
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int64_t kb8 = (static_cast<int64_t>(t) * 128 + 32 * st + 8 * grp) / 8;
        av[st] = mrow ? xrow[kb8] : u32x4{0, 0, 0, 0};
      }
      f32x4 p[4], q[4];
#pragma unroll
      for (int f = 0; f < 4; ++f) p[f] = q[f] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const f16x8 a = __builtin_bit_cast(f16x8, av[st]);
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          p[f] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pm_one(so[f][st], grp), p[f], 0, 0, 0);
          q[f] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pm_one(sr[f][st], grp), q[f], 0, 0, 0);
        }
      }
#pragma unroll
      for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[f][i] += sco[f] * p[f][i] + scr[f] * q[f][i];
    }
  }
  if (!active) return;
  // D layout: lane l holds rows 4*(l/16) + i of the x tile, column l % 16 of the fragment.
  if (nsplit == 1) {
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const int64_t n = band * 64 + 16 * f + r16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t m = m0 + 4 * grp + i;
        if (m < M) y[m * N + n] = acc[f][i];
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
      y[m * N + n] = s;
    }
  }
  if (lane == 0) reset_agent(&ws_cnt[cidx]);
}

struct ResidualPlan { int64_t groups, mtiles, nsplit, tps; };

// Tuning knob (harnesses that compile this file directly): workgroups to aim for (0 = 512).
int g_residual_wg_target = 0;

ResidualPlan plan_residual(int64_t M, int64_t N, int64_t K) {
  const int64_t KT = K / 128;
  const int64_t groups = (N / 64 + 3) / 4, mtiles = (M + 15) / 16;
  const int64_t target = g_residual_wg_target > 0 ? g_residual_wg_target : 512;
  int64_t nsplit = std::max<int64_t>(1, target / (groups * mtiles));
  nsplit = std::min<int64_t>(nsplit, std::max<int64_t>(1, KT / 2));
  if (mtiles * (N / 64) > kMaxCounters) nsplit = 1;
  const int64_t tps = (KT + nsplit - 1) / nsplit;
  return {groups, mtiles, (KT + tps - 1) / tps, tps};
}

}  // namespace

size_t residual_part_floats(int64_t M, int64_t N, int64_t K) {
  if (N % 64 || K % 128) return 0;
  const ResidualPlan p = plan_residual(M, N, K);
  return p.nsplit > 1 ? static_cast<size_t>(p.nsplit) * M * N : 0;
}

hipError_t launch_residual_binarize(const float* W, int64_t N, int64_t K, void* planes_o,
                                    float* alpha_o, void* planes_r, float* alpha_r,
                                    hipStream_t s) {
  const int64_t items = N * (K / 128);
  hipLaunchKernelGGL(residual_pack_kernel, dim3(static_cast<unsigned>((items + 3) / 4)), dim3(256),
                     0, s, W, N, K, static_cast<u32x4*>(planes_o), alpha_o,
                     static_cast<u32x4*>(planes_r), alpha_r);
  return hipGetLastError();
}

hipError_t launch_residual_linear(const uint16_t* x, const void* planes_o, const float* alpha_o,
                                  const void* planes_r, const float* alpha_r, int64_t M, int64_t N,
                                  int64_t K, float* y, float* ws_part, uint32_t* ws_cnt,
                                  hipStream_t s) {
  const ResidualPlan p = plan_residual(M, N, K);
  hipLaunchKernelGGL(residual_mfma_kernel,
                     dim3(static_cast<unsigned>(p.groups), static_cast<unsigned>(p.mtiles),
                          static_cast<unsigned>(p.nsplit)),
                     dim3(256), 0, s, x, static_cast<const u32x4*>(planes_o), alpha_o,
                     static_cast<const u32x4*>(planes_r), alpha_r, M, N, K, y, ws_part, ws_cnt,
                     static_cast<int>(p.tps));
  return hipGetLastError();
}

}  // namespace bl
