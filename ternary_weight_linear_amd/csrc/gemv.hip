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
    for (int m = 0; m < MR; ++m) atomicAdd(&ws_acc[m * N + n], acc[m]);
    __threadfence();
    uint32_t old = 0;
    if (lane == 0) old = atomicAdd(&ws_cnt[band], 1u);
    old = __shfl(old, 0);
    if (old != static_cast<uint32_t>(nsplit - 1)) return;
    __threadfence();
#pragma unroll
    for (int m = 0; m < MR; ++m) acc[m] = atomicExch(&ws_acc[m * N + n], 0);
    if (lane == 0) atomicExch(&ws_cnt[band], 0u);
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

}  // namespace

hipError_t launch_gemv(const uint32_t* planes, const float* gamma, int M, int64_t K,
                       const void* wpacked, const float* beta, int64_t beta_len, int64_t N,
                       float* y, int32_t* acc_out, int32_t* ws_acc, uint32_t* ws_cnt,
                       hipStream_t s) {
  const int64_t bands = N / 64;
  const int64_t KT = K / 64;
  // Aim for ~2048 workgroups (8 per CU) with at least 16 tiles (4 per wave) each.
  int64_t nsplit = (2048 + bands - 1) / bands;
  nsplit = std::min<int64_t>(nsplit, std::max<int64_t>(1, KT / 16));
  nsplit = std::max<int64_t>(nsplit, 1);
  if (static_cast<int64_t>(M) * N > kAccCap || bands > kMaxCounters) nsplit = 1;
  int64_t tps = (KT + nsplit - 1) / nsplit;
  nsplit = (KT + tps - 1) / tps;
  const dim3 grid(static_cast<unsigned>(bands), static_cast<unsigned>(nsplit));
  const u32x4* W = static_cast<const u32x4*>(wpacked);
#define BL_GEMV_LAUNCH(MR_)                                                                  \
  hipLaunchKernelGGL(gemv_kernel<MR_>, grid, dim3(256), 0, s, planes, gamma, K, W, beta,     \
                     beta_len, N, y, acc_out, ws_acc, ws_cnt, static_cast<int>(tps))
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

}  // namespace bl
