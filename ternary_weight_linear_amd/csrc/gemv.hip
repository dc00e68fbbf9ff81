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
    float* __restrict__ y, int32_t* __restrict__ acc_out, int32_t* __restrict__ ws_acc,
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
  if (nsplit > 1) {
#pragma unroll
    for (int m = 0; m < MR; ++m) atomic_add_agent(&ws_acc[m * N + n], acc[m]);
    wait_own_memory_ops();
    uint32_t old = 0;
    if (lane == 0) old = arrive_agent(&ws_cnt[band]);
    old = __shfl(old, 0);
    if (old != static_cast<uint32_t>(nsplit - 1)) return;
#pragma unroll
    for (int m = 0; m < MR; ++m) acc[m] = atomic_take_agent(&ws_acc[m * N + n]);
    if (lane == 0) reset_agent(&ws_cnt[band]);
  }
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    if (acc_out) acc_out[m * N + n] = acc[m];
    if (y) {
      const float scale = gamma[m] / 127.0f;
      const float b = beta[beta_len == 1 ? 0 : n];
      y[m * N + n] = static_cast<float>(acc[m]) * scale * b;
    }
  }
}

// Fused quantise + GEMV: the same add-only product, but each wave builds the activation
// bit planes of its current tile itself instead of reading X8-64 planes from memory.
// Every workgroup first reduces |x| over the whole row to gamma (the row is small and
// stays in L2), then for each tile lane l quantises the input whose plane bit is l and
// eight wave ballots give the tile's planes directly in scalar registers, where the
// select + popcount loop wants them. This removes the separate quantiser launch from the
// decode path; the integer results are identical to bl_quant_act_int8 + GEMV.
template <int MR>
__global__ __launch_bounds__(256) void gemv_fused_kernel(
    const uint16_t* __restrict__ x, int64_t K, const u32x4* __restrict__ W,
    const float* __restrict__ beta, int64_t beta_len, int64_t N, float* __restrict__ y,
    int32_t* __restrict__ ws_acc, uint32_t* __restrict__ ws_cnt, int tiles_per_split) {
  __shared__ int red[kWaves - 1][MR][64];
  __shared__ float red_max[kWaves][MR];
  __shared__ int red_bad[kWaves][MR];
  const int band = blockIdx.x;
  const int split = blockIdx.y;
  const int nsplit = gridDim.y;
  const int KT = static_cast<int>(K / 64);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t0 = split * tiles_per_split;
  const int t1 = min(KT, t0 + tiles_per_split);
  const u32x4* wp = W + static_cast<int64_t>(band) * KT * 64 + lane;
  // lane l <-> plane bit l of a tile: half h = l / 32, bit p = l % 32 = 8i + j <-> c = 4j + i
  const int koff = 32 * (lane >> 5) + 4 * (lane & 7) + ((lane & 31) >> 3);

  // Software pipeline: weight tiles and the x elements they pair with are loaded one batch
  // ahead of the batch being reduced. The first batch is issued before gamma is computed,
  // so the HBM stream starts at once and the row reduction hides under its latency.
  u32x4 w[kUnroll];
  uint16_t xv[kUnroll][MR];
  auto load_batch = [&](int t) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int tt = t + kWaves * u;
      w[u] = tt < t1 ? wp[static_cast<int64_t>(tt) * 64] : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int m = 0; m < MR; ++m) xv[u][m] = tt < t1 ? x[m * K + 64 * tt + koff] : uint16_t(0);
    }
  };
  load_batch(t0 + wave);

  // gamma_m = max |x_m| over the whole row (NaN if the row holds NaN/inf)
  float g[MR];
  bool zero[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    const u32x4* row4 = reinterpret_cast<const u32x4*>(x + m * K);
    float mx = 0.0f;
    int bad = 0;
    for (int64_t i = threadIdx.x; i < K / 8; i += 256) {
      const u32x4 v = row4[i];
      const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint16_t lo = static_cast<uint16_t>(w4[j] & 0xFFFFu), hi = static_cast<uint16_t>(w4[j] >> 16);
        bad |= ((lo & 0x7C00u) == 0x7C00u) | ((hi & 0x7C00u) == 0x7C00u);
        mx = fmaxf(mx, fabsf(half_bits_to_float(lo)));
        mx = fmaxf(mx, fabsf(half_bits_to_float(hi)));
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      mx = fmaxf(mx, __shfl_xor(mx, off));
      bad |= __shfl_xor(bad, off);
    }
    if (lane == 0) { red_max[wave][m] = mx; red_bad[wave][m] = bad; }
  }
  __syncthreads();
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    float mx = red_max[0][m];
    int bad = red_bad[0][m];
#pragma unroll
    for (int w2 = 1; w2 < kWaves; ++w2) { mx = fmaxf(mx, red_max[w2][m]); bad |= red_bad[w2][m]; }
    g[m] = bad ? __uint_as_float(0x7FC00000u) : mx;
    zero[m] = bad || mx == 0.0f;
  }

  int A[MR][8];
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int b = 0; b < 8; ++b) A[m][b] = 0;
  int cn = 0;

  for (int t = t0 + wave; t < t1; t += kWaves * kUnroll) {
    u32x4 wc[kUnroll];
    uint16_t xc[kUnroll][MR];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      wc[u] = w[u];
#pragma unroll
      for (int m = 0; m < MR; ++m) xc[u][m] = xv[u][m];
    }
    if (t + kWaves * kUnroll < t1) load_batch(t + kWaves * kUnroll);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int tt = t + kWaves * u;
      if (tt < t1) {
#pragma unroll
        for (int m = 0; m < MR; ++m) {
          int qv = 0;
          if (!zero[m]) {
            const float r = rintf(half_bits_to_float(xc[u][m]) * 127.0f / g[m]);
            qv = static_cast<int>(fminf(fmaxf(r, -127.0f), 127.0f));
          }
#pragma unroll
          for (int b = 0; b < 8; ++b) {
            const unsigned long long mask = __ballot((qv >> b) & 1);
            const uint32_t x0 = static_cast<uint32_t>(mask), x1 = static_cast<uint32_t>(mask >> 32);
            A[m][b] += __builtin_popcount((x0 & wc[u].x) | (~x0 & wc[u].z));
            A[m][b] += __builtin_popcount((x1 & wc[u].y) | (~x1 & wc[u].w));
          }
        }
        cn += __builtin_popcount(wc[u].z) + __builtin_popcount(wc[u].w);
      }
    }
  }

  int acc[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m)
    acc[m] = A[m][0] + 2 * A[m][1] + 4 * A[m][2] + 8 * A[m][3] + 16 * A[m][4] + 32 * A[m][5] +
             64 * A[m][6] - 128 * A[m][7] + cn;
  if (wave > 0) {
#pragma unroll
    for (int m = 0; m < MR; ++m) red[wave - 1][m][lane] = acc[m];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int w2 = 0; w2 < kWaves - 1; ++w2) acc[m] += red[w2][m][lane];

  const int64_t n = static_cast<int64_t>(band) * 64 + lane;
  if (nsplit > 1) {
#pragma unroll
    for (int m = 0; m < MR; ++m) atomic_add_agent(&ws_acc[m * N + n], acc[m]);
    wait_own_memory_ops();
    uint32_t old = 0;
    if (lane == 0) old = arrive_agent(&ws_cnt[band]);
    old = __shfl(old, 0);
    if (old != static_cast<uint32_t>(nsplit - 1)) return;
#pragma unroll
    for (int m = 0; m < MR; ++m) acc[m] = atomic_take_agent(&ws_acc[m * N + n]);
    if (lane == 0) reset_agent(&ws_cnt[band]);
  }
  const float b = beta[beta_len == 1 ? 0 : n];
#pragma unroll
  for (int m = 0; m < MR; ++m) y[m * N + n] = static_cast<float>(acc[m]) * (g[m] / 127.0f) * b;
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
  if (static_cast<int64_t>(M) * N > kAccCap || bands > kMaxCounters) nsplit = 1;
  const int64_t tps = (KT + nsplit - 1) / nsplit;
  return {(KT + tps - 1) / tps, tps};
}

}  // namespace

hipError_t launch_gemv(const uint32_t* planes, const float* gamma, int M, int64_t K,
                       const void* wpacked, const float* beta, int64_t beta_len, int64_t N,
                       float* y, int32_t* acc_out, int32_t* ws_acc, uint32_t* ws_cnt,
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
                             int32_t* ws_acc, uint32_t* ws_cnt, hipStream_t s) {
  const GemvPlan p = plan_gemv(M, N, K);
  const dim3 grid(static_cast<unsigned>(N / 64), static_cast<unsigned>(p.nsplit));
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
