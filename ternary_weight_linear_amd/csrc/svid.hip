// SVID initialisation of a OneBit layer on the GPU.
//
// [onebit] "2. 基于 SVID 初始化量化模型": the weight is split into its sign matrix and its
// magnitude, and the magnitude gets a rank-1 approximation (SVD or NMF); reordering the
// products makes the rank-1 factors the layer's value vectors. Here the rank-1 fit of |W|
// is the leading singular pair found by power iteration,
//     u <- |W| v / ||.||,   v <- |W|^T u / ||.||,   v_0 = 1 / sqrt(K),
// whose vectors stay positive (|W| is nonnegative), and h = sqrt(s) u (one per output),
// g = sqrt(s) v (one per input) with s = || |W|^T u ||, rounded to fp16. Every reduction
// uses a fixed order, so the result is identical from run to run.
#include "bl_internal.h"

namespace bl {
namespace {

constexpr int kColSplits = 32;     // row blocks of the |W|^T u product

// u[n] = sum_k |W[n,k]| v[k]; one wave per row, lanes stride K, then a butterfly.
__global__ __launch_bounds__(256) void absw_rows_kernel(const float* __restrict__ W, int64_t N,
                                                        int64_t K, const float* __restrict__ v,
                                                        float* __restrict__ u) {
  const int lane = threadIdx.x & 63;
  const int64_t n = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (n >= N) return;
  const float4* row = reinterpret_cast<const float4*>(W + n * K);
  const float4* v4 = reinterpret_cast<const float4*>(v);
  float s = 0.0f;
  for (int64_t i = lane; i < K / 4; i += 64) {
    const float4 a = row[i], b = v4[i];
    s += fabsf(a.x) * b.x;
    s += fabsf(a.y) * b.y;
    s += fabsf(a.z) * b.z;
    s += fabsf(a.w) * b.w;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
  if (lane == 0) u[n] = s;
}

// part[r][k] = sum over rows of block r of |W[n,k]| u[n]; thread = column.
__global__ __launch_bounds__(256) void absw_cols_kernel(const float* __restrict__ W, int64_t N,
                                                        int64_t K, const float* __restrict__ u,
                                                        float* __restrict__ part) {
  const int64_t k = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int r = blockIdx.y;
  const int64_t rows = (N + kColSplits - 1) / kColSplits;
  const int64_t n0 = r * rows, n1 = min(N, n0 + rows);
  if (k >= K) return;
  float s = 0.0f;
  for (int64_t n = n0; n < n1; ++n) s += fabsf(W[n * K + k]) * u[n];
  part[r * K + k] = s;
}

__global__ __launch_bounds__(256) void sum_parts_kernel(const float* __restrict__ part, int64_t K,
                                                        float* __restrict__ v) {
  const int64_t k = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (k >= K) return;
  float s = 0.0f;
  for (int r = 0; r < kColSplits; ++r) s += part[r * K + k];
  v[k] = s;
}

// x <- x / ||x||; *norm = ||x||. One workgroup: per-thread strided sums, then a fixed tree.
__global__ __launch_bounds__(1024) void normalize_kernel(float* __restrict__ x, int64_t n,
                                                         float* __restrict__ norm) {
  __shared__ float red[1024];
  float s = 0.0f;
  for (int64_t i = threadIdx.x; i < n; i += 1024) s += x[i] * x[i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  const float nr = sqrtf(red[0]);
  for (int64_t i = threadIdx.x; i < n; i += 1024) x[i] = nr > 0.0f ? x[i] / nr : 0.0f;
  if (threadIdx.x == 0) *norm = nr;
}

__global__ void fill_kernel(float* __restrict__ x, int64_t n, float value) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) x[i] = value;
}

// h = fp16(sqrt(s) u), g = fp16(sqrt(s) v) (round to nearest even); s = *sigma.
__global__ void svid_finish_kernel(const float* __restrict__ u, const float* __restrict__ v,
                                   const float* __restrict__ sigma, int64_t N, int64_t K,
                                   uint16_t* __restrict__ h, uint16_t* __restrict__ g,
                                   float* __restrict__ sigma_out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const float r = sqrtf(*sigma);
  if (i < N) h[i] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(r * u[i]));
  if (i < K) g[i] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(r * v[i]));
  if (i == 0 && sigma_out) *sigma_out = *sigma;
}

inline unsigned blocks(int64_t n, int per) { return static_cast<unsigned>((n + per - 1) / per); }

}  // namespace

size_t svid_scratch_floats(int64_t N, int64_t K) {
  return static_cast<size_t>(N) + K + static_cast<size_t>(kColSplits) * K + 64;
}

hipError_t launch_svid(const float* W, int64_t N, int64_t K, int iters, uint16_t* g, uint16_t* h,
                       float* sigma, float* scratch, hipStream_t s) {
  float* u = scratch;
  float* v = u + N;
  float* part = v + K;
  float* nrm = part + static_cast<size_t>(kColSplits) * K;   // [0] ||u||, [1] ||v||
  hipLaunchKernelGGL(fill_kernel, dim3(blocks(K, 256)), dim3(256), 0, s, v, K,
                     1.0f / sqrtf(static_cast<float>(K)));
  for (int it = 0; it < iters; ++it) {
    hipLaunchKernelGGL(absw_rows_kernel, dim3(blocks(N, 4)), dim3(256), 0, s, W, N, K, v, u);
    hipLaunchKernelGGL(normalize_kernel, dim3(1), dim3(1024), 0, s, u, N, nrm);
    hipLaunchKernelGGL(absw_cols_kernel, dim3(blocks(K, 256), kColSplits), dim3(256), 0, s, W, N,
                       K, u, part);
    hipLaunchKernelGGL(sum_parts_kernel, dim3(blocks(K, 256)), dim3(256), 0, s, part, K, v);
    hipLaunchKernelGGL(normalize_kernel, dim3(1), dim3(1024), 0, s, v, K, nrm + 1);
  }
  hipLaunchKernelGGL(svid_finish_kernel, dim3(blocks(std::max(N, K), 256)), dim3(256), 0, s, u, v,
                     nrm + 1, N, K, h, g, sigma);
  return hipGetLastError();
}

}  // namespace bl
