// Add-only decode GEMV for ternary weights (M <= 4 tokens).
//
// [b158] "实验及结果" (energy paragraph, Fig. 3): with weights in {-1, 0, +1} the matrix
// product needs only int8 additions. [onebit] "讨论与分析 / 1. 效率": element products turn
// into bit operations plus additions. This kernel takes that literally: no multiplies.
//
// For a 32-input word of the T2-PN-64 layout, with P (w = +1) and N (w = -1) bit masks and
// the activation bit planes X_b (bit b of the two's-complement int8 q, same bit order):
//     popcount((P & X_b) | (N & ~X_b)) = #{k : w = +1, bit b set} + #{k : w = -1, bit b clear}
// and, with plane weights c_b = 2^b (b < 7), c_7 = -128 (sum of c_b = -1),
//     sum_b c_b * popcount(...) + popcount(N) = sum_k w_k q_k        exactly.
// Each (P, N, X_b) step is one v_bfi_b32 and one v_bcnt_u32_b32 (popcount with add), so the
// inner loop costs 16 VALU ops per 32 weights per token.
//
// Mapping: a wave owns one 64-row band; lane = output row, so each lane streams its 16-byte
// tile row and a wave's load is one fully coalesced 1 KiB tile. The planes of the current
// tile are wave-uniform and come through scalar loads. Four waves of a workgroup take
// interleaved tiles of the workgroup's K range and reduce in LDS. When K is split across
// workgroups, partial sums go to int32 atomics in the workspace (exact, order-free) and the
// last workgroup of a band, found with a completion counter, applies the epilogue and
// restores the workspace to zero.
#include "bl_internal.h"

namespace bl {
namespace {

constexpr int kWaves = 4;
constexpr int kUnroll = 8;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int MR>
__global__ __launch_bounds__(256) void gemv_kernel(
    const uint32_t* __restrict__ planes, const float* __restrict__ gamma, int64_t K,
    const u32x4* __restrict__ W, const float* __restrict__ beta, int64_t beta_len, int64_t N,
    float* __restrict__ y, int32_t* __restrict__ acc_out, uint64_t* __restrict__ ws_acc,
    uint32_t* __restrict__ ws_cnt, int tiles_per_split) {
  __shared__ int red[kWaves - 1][MR][64];
  const int band = blockIdx.x;
  const int split = blockIdx.y;
  const int nsplit = gridDim.y;
  const int KT = static_cast<int>(K / 64);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t0 = split * tiles_per_split;
  const int t1 = min(KT, t0 + tiles_per_split);
  const u32x4* wp = W + static_cast<int64_t>(band) * KT * 64 + lane;

  int A[MR][8];
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int b = 0; b < 8; ++b) A[m][b] = 0;
  int cn = 0;

  for (int t = t0 + wave; t < t1; t += kWaves * kUnroll) {
    u32x4 w[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int tt = t + kWaves * u;
      w[u] = tt < t1 ? wp[static_cast<int64_t>(tt) * 64] : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int tt = t + kWaves * u;
      if (tt < t1) {
#pragma unroll
        for (int m = 0; m < MR; ++m) {
          const uint32_t* X = planes + (static_cast<int64_t>(m) * KT + tt) * 16;
#pragma unroll
          for (int b = 0; b < 8; ++b) {
            const uint32_t x0 = X[2 * b], x1 = X[2 * b + 1];
            A[m][b] += __builtin_popcount((x0 & w[u].x) | (~x0 & w[u].z));
            A[m][b] += __builtin_popcount((x1 & w[u].y) | (~x1 & w[u].w));
          }
        }
        cn += __builtin_popcount(w[u].z) + __builtin_popcount(w[u].w);
      }
    }
  }

  int acc[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    int s = A[m][0] + 2 * A[m][1] + 4 * A[m][2] + 8 * A[m][3] + 16 * A[m][4] + 32 * A[m][5] +
            64 * A[m][6] - 128 * A[m][7];
    acc[m] = s + cn;
  }
  if (wave > 0) {
#pragma unroll
    for (int m = 0; m < MR; ++m) red[wave - 1][m][lane] = acc[m];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int w = 0; w < kWaves - 1; ++w) acc[m] += red[w][m][lane];

  const int64_t n = static_cast<int64_t>(band) * 64 + lane;
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    int total = acc[m];
    if (nsplit > 1 && !split_arrive(&ws_acc[m * N + n], acc[m], nsplit, &total)) continue;
    if (acc_out) acc_out[m * N + n] = total;
    if (y) {
      const float scale = gamma[m] / 127.0f;
      const float b = beta[beta_len == 1 ? 0 : n];
      y[m * N + n] = static_cast<float>(total) * scale * b;
    }
  }
}

// Fused quantise + GEMV: the same add-only product, with the activation bit planes built
// inside the kernel instead of read from X8-64 memory. A workgroup owns four consecutive
// 64-row bands (one per wave) and one K range, processed in chunks of up to kChunk tiles:
//  1. the first weight batch of the wave's band is issued at once, so HBM streaming starts
//     before anything else;
//  2. gamma: every workgroup reduces |x| over the whole row. For finite fp16 the magnitude
//     order equals the integer order of the bits with the sign cleared, so this is an
//     integer max over masked bit patterns (no conversions); a maximum >= 0x7C00 flags
//     NaN/inf;
//  3. each wave quantises every fourth tile of the chunk (lane l takes the input whose plane
//     bit is l; eight wave ballots give the tile's planes) into LDS, then one barrier;
//  4. each wave runs the select + popcount loop over the chunk for its own band, weight
//     loads one batch ahead, planes read from LDS as wave-uniform broadcasts.
// The integer results are identical to bl_quant_act_int8 followed by the GEMV.
constexpr int kBatch = 8;
constexpr int kChunk = 64;                   // tiles whose planes sit in LDS at once

template <int MR>
__global__ __launch_bounds__(256) void gemv_fused_kernel(
    const uint16_t* __restrict__ x, int64_t K, const u32x4* __restrict__ W,
    const float* __restrict__ beta, int64_t beta_len, int64_t N, float* __restrict__ y,
    uint64_t* __restrict__ ws_acc, uint32_t* __restrict__ ws_cnt, int tiles_per_split) {
  __shared__ __attribute__((aligned(16))) uint32_t pl[kChunk][MR][16];
  __shared__ uint32_t red_max[kWaves][MR];
  const int64_t nbands = N / 64;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t band = static_cast<int64_t>(blockIdx.x) * kWaves + wave;
  const bool active = band < nbands;
  const int split = blockIdx.y;
  const int nsplit = gridDim.y;
  const int KT = static_cast<int>(K / 64);
  const int t0 = split * tiles_per_split;
  const int t1 = min(KT, t0 + tiles_per_split);
  const u32x4* wp = W + (active ? band : 0) * KT * 64 + lane;
  // lane l <-> plane bit l of a tile: half h = l / 32, bit p = l % 32 = 8i + j <-> c = 4j + i
  const int koff = 32 * (lane >> 5) + 4 * (lane & 7) + ((lane & 31) >> 3);

  u32x4 w[kBatch];
  auto load_batch = [&](int tb, int tend) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int tt = tb + u;
      w[u] = (active && tt < tend) ? wp[static_cast<int64_t>(tt) * 64] : u32x4{0, 0, 0, 0};
    }
  };
  load_batch(t0, min(t1, t0 + kChunk));

  // gamma_m = max |x_m| over the whole row (NaN if the row holds NaN/inf)
  float g[MR];
  bool zero[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    const u32x4* row4 = reinterpret_cast<const u32x4*>(x + m * K);
    uint32_t mb = 0;
#pragma unroll 4
    for (int64_t i = threadIdx.x; i < K / 8; i += 256) {
      const u32x4 v = row4[i];
      const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) mb = max(mb, max(w4[j] & 0x7FFFu, (w4[j] >> 16) & 0x7FFFu));
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mb = max(mb, static_cast<uint32_t>(__shfl_xor(mb, off)));
    if (lane == 0) red_max[wave][m] = mb;
  }
  __syncthreads();
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    uint32_t mb = red_max[0][m];
#pragma unroll
    for (int w2 = 1; w2 < kWaves; ++w2) mb = max(mb, red_max[w2][m]);
    const bool bad = mb >= 0x7C00u;
    g[m] = bad ? __uint_as_float(0x7FC00000u) : half_bits_to_float(static_cast<uint16_t>(mb));
    zero[m] = bad || mb == 0u;
  }

  int A[MR][8];
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int b = 0; b < 8; ++b) A[m][b] = 0;
  int cn = 0;

  for (int c0 = t0; c0 < t1; c0 += kChunk) {
    const int c1 = min(t1, c0 + kChunk);
    if (c0 != t0) {
      __syncthreads();                    // the previous chunk's planes are consumed
      load_batch(c0, c1);
    }
    // quantise tiles c0 + wave + 4j of this chunk into LDS (x loads issued together)
    constexpr int kPerWave = kChunk / kWaves;
    uint16_t xq[kPerWave][MR];
#pragma unroll
    for (int j = 0; j < kPerWave; ++j) {
      const int tt = c0 + wave + kWaves * j;
#pragma unroll
      for (int m = 0; m < MR; ++m) xq[j][m] = tt < c1 ? x[m * K + 64 * tt + koff] : uint16_t(0);
    }
#pragma unroll
    for (int j = 0; j < kPerWave; ++j) {
      const int tt = c0 + wave + kWaves * j;
      if (tt < c1) {
#pragma unroll
        for (int m = 0; m < MR; ++m) {
          int qv = 0;
          if (!zero[m]) {
            const float r = rintf(half_bits_to_float(xq[j][m]) * 127.0f / g[m]);
            qv = static_cast<int>(fminf(fmaxf(r, -127.0f), 127.0f));
          }
          uint32_t mine = 0;
#pragma unroll
          for (int b = 0; b < 8; ++b) {
            const unsigned long long mask = __ballot((qv >> b) & 1);
            if ((lane >> 1) == b) mine = (lane & 1) ? static_cast<uint32_t>(mask >> 32) : static_cast<uint32_t>(mask);
          }
          if (lane < 16) pl[tt - c0][m][lane] = mine;
        }
      }
    }
    __syncthreads();
    if (active) {
      for (int tb = c0; tb < c1; tb += kBatch) {
        u32x4 wc[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) wc[u] = w[u];
        if (tb + kBatch < c1) load_batch(tb + kBatch, c1);
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          if (tb + u < c1) {
#pragma unroll
            for (int m = 0; m < MR; ++m) {
              const u32x4* X4 = reinterpret_cast<const u32x4*>(&pl[tb + u - c0][m][0]);
              const u32x4 p0 = X4[0], p1 = X4[1], p2 = X4[2], p3 = X4[3];
              const uint32_t X[16] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w,
                                      p2.x, p2.y, p2.z, p2.w, p3.x, p3.y, p3.z, p3.w};
#pragma unroll
              for (int b = 0; b < 8; ++b) {
                const uint32_t x0 = X[2 * b], x1 = X[2 * b + 1];
                A[m][b] += __builtin_popcount((x0 & wc[u].x) | (~x0 & wc[u].z));
                A[m][b] += __builtin_popcount((x1 & wc[u].y) | (~x1 & wc[u].w));
              }
            }
            cn += __builtin_popcount(wc[u].z) + __builtin_popcount(wc[u].w);
          }
        }
      }
    }
  }
  if (!active) return;

  int acc[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m)
    acc[m] = A[m][0] + 2 * A[m][1] + 4 * A[m][2] + 8 * A[m][3] + 16 * A[m][4] + 32 * A[m][5] +
             64 * A[m][6] - 128 * A[m][7] + cn;
  const int64_t n = band * 64 + lane;
  const float b = beta[beta_len == 1 ? 0 : n];
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    int total = acc[m];
    if (nsplit > 1 && !split_arrive(&ws_acc[m * N + n], acc[m], nsplit, &total)) continue;
    y[m * N + n] = static_cast<float>(total) * (g[m] / 127.0f) * b;
  }
}

// Split plan of the fused kernel: workgroups own four bands each.
int64_t g_gemvf_wg_target = 0;   // 0: by shape; changed only by tuning harnesses

struct GemvFusedPlan { int64_t groups, nsplit, tps; };

GemvFusedPlan plan_gemv_fused(int M, int64_t N, int64_t K) {
  const int64_t bands = N / 64;
  const int64_t groups = (bands + kWaves - 1) / kWaves;
  const int64_t KT = K / 64;
  const int64_t target = g_gemvf_wg_target ? g_gemvf_wg_target : 768;   // measured on MI355X
  int64_t nsplit = (target + groups / 2) / groups;
  nsplit = std::min<int64_t>(nsplit, std::max<int64_t>(1, KT / kBatch));
  nsplit = std::max<int64_t>(nsplit, 1);
  if (static_cast<int64_t>(M) * N > kAccCap || K > kMaxIntSplitK) nsplit = 1;
  nsplit = std::min<int64_t>(nsplit, kMaxIntSplits);
  const int64_t tps = (KT + nsplit - 1) / nsplit;
  return {groups, (KT + tps - 1) / tps, tps};
}

struct GemvPlan { int64_t nsplit, tps; };

// Workgroups the split-K plan aims for (0: by shape). Only tuning harnesses that compile
// this file directly change it.
int64_t g_gemv_wg_target = 0;

GemvPlan plan_gemv(int M, int64_t N, int64_t K) {
  const int64_t bands = N / 64;
  const int64_t KT = K / 64;
  // Split K so the launch has about `target` workgroups (measured on MI355X: ~512 suit
  // narrow outputs, ~1024 wide ones), keeping at least 8 tiles (2 per wave) per workgroup.
  const int64_t target = g_gemv_wg_target ? g_gemv_wg_target : (bands < 256 ? 512 : 1024);
  int64_t nsplit = (target + bands / 2) / bands;
  nsplit = std::min<int64_t>(nsplit, std::max<int64_t>(1, KT / 8));
  nsplit = std::max<int64_t>(nsplit, 1);
  if (static_cast<int64_t>(M) * N > kAccCap || K > kMaxIntSplitK) nsplit = 1;
  nsplit = std::min<int64_t>(nsplit, kMaxIntSplits);
  const int64_t tps = (KT + nsplit - 1) / nsplit;
  return {(KT + tps - 1) / tps, tps};
}

}  // namespace

hipError_t launch_gemv(const uint32_t* planes, const float* gamma, int M, int64_t K,
                       const void* wpacked, const float* beta, int64_t beta_len, int64_t N,
                       float* y, int32_t* acc_out, uint64_t* ws_acc, uint32_t* ws_cnt,
                       hipStream_t s) {
  const int64_t bands = N / 64;
  const GemvPlan p = plan_gemv(M, N, K);
  const dim3 grid(static_cast<unsigned>(bands), static_cast<unsigned>(p.nsplit));
  const u32x4* W = static_cast<const u32x4*>(wpacked);
#define BL_GEMV_LAUNCH(MR_)                                                                  \
  hipLaunchKernelGGL(gemv_kernel<MR_>, grid, dim3(256), 0, s, planes, gamma, K, W, beta,     \
                     beta_len, N, y, acc_out, ws_acc, ws_cnt, static_cast<int>(p.tps))
  switch (M) {
    case 1: BL_GEMV_LAUNCH(1); break;
    case 2: BL_GEMV_LAUNCH(2); break;
    case 3: BL_GEMV_LAUNCH(3); break;
    case 4: BL_GEMV_LAUNCH(4); break;
    default: return hipErrorInvalidValue;
  }
#undef BL_GEMV_LAUNCH
  return hipGetLastError();
}

hipError_t launch_gemv_fused(const uint16_t* x, int M, int64_t K, const void* wpacked,
                             const float* beta, int64_t beta_len, int64_t N, float* y,
                             uint64_t* ws_acc, uint32_t* ws_cnt, hipStream_t s) {
  const GemvFusedPlan p = plan_gemv_fused(M, N, K);
  const dim3 grid(static_cast<unsigned>(p.groups), static_cast<unsigned>(p.nsplit));
  const u32x4* W = static_cast<const u32x4*>(wpacked);
#define BL_GEMVF_LAUNCH(MR_)                                                                 \
  hipLaunchKernelGGL(gemv_fused_kernel<MR_>, grid, dim3(256), 0, s, x, K, W, beta, beta_len, \
                     N, y, ws_acc, ws_cnt, static_cast<int>(p.tps))
  switch (M) {
    case 1: BL_GEMVF_LAUNCH(1); break;
    case 2: BL_GEMVF_LAUNCH(2); break;
    case 3: BL_GEMVF_LAUNCH(3); break;
    case 4: BL_GEMVF_LAUNCH(4); break;
    default: return hipErrorInvalidValue;
  }
#undef BL_GEMVF_LAUNCH
  return hipGetLastError();
}

}  // namespace bl
