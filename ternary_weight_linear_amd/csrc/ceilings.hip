// Measured ceilings of the two rooflines the path is held against, built from this source
// (not from the library's kernels): a streaming HBM read and an int8 matrix-core loop. The
// benchmark reports each product kernel as a fraction of both the spec peak and these.
//
//  * bl_ceil_stream_read: every byte of a buffer read once with 16-byte vector loads, eight
//    in flight per thread, grid-strided so consecutive workgroups read consecutive 4 KiB;
//    the loaded words are folded with XOR into one word per workgroup, so no load can be
//    removed. Bytes moved = the buffer size.
//  * bl_ceil_stream_read_slices: the same with each workgroup reading one contiguous slice
//    of bytes / grid (a multiple of 16 KiB) with non-temporal loads, the access pattern of
//    the product kernels' weight streams (a workgroup streams its own bands).
//  * bl_ceil_mfma_i8: v_mfma_i32_16x16x64_i8 on register operands, eight independent
//    accumulators per wave (the matrix-core pipeline never waits on a result), `iters`
//    rounds; the accumulators are stored at the end. Ops = 2 * 16 * 16 * 64 per MFMA.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 8;

__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const u32x4* __restrict__ src,
                                                                    int64_t n16,
                                                                    uint32_t* __restrict__ out) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kReadThreads;
  int64_t i = static_cast<int64_t>(blockIdx.x) * kReadThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kReadUnroll - 1) * stride < n16; i += kReadUnroll * stride) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off);
  if ((threadIdx.x & 63) == 0) atomicXor(out + blockIdx.x, acc);
}

__global__ __launch_bounds__(kReadThreads) void stream_read_slices_kernel(
    const u32x4* __restrict__ src, int64_t per_wg16, uint32_t* __restrict__ out) {
  const u32x4* p = src + static_cast<int64_t>(blockIdx.x) * per_wg16;
  uint32_t acc = 0;
  for (int64_t i = threadIdx.x; i < per_wg16; i += kReadThreads * kReadUnroll) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u)   // per_wg16 is a multiple of 256 * 8: in range
      v[u] = __builtin_nontemporal_load(p + i + kReadThreads * u);
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off);
  if ((threadIdx.x & 63) == 0) atomicXor(out + blockIdx.x, acc);
}

constexpr int kMfmaAcc = 8;

__global__ __launch_bounds__(256) void mfma_i8_kernel(int iters, int seed, i32x4* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const i32x4 a = {lane * 0x01010101 + seed, lane ^ seed, 3 * lane, 0x7F7F7F7F};
  const i32x4 b = {seed, lane * 0x01020304, 0x01010101, lane};
  i32x4 c[kMfmaAcc];
#pragma unroll
  for (int j = 0; j < kMfmaAcc; ++j) c[j] = i32x4{j, 0, 0, 0};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kMfmaAcc; ++j) c[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c[j], 0, 0, 0);
  }
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  i32x4 s = c[0];
#pragma unroll
  for (int j = 1; j < kMfmaAcc; ++j) s += c[j];
  out[t] = s;
}

}  // namespace

extern "C" {

// Streams `bytes` (a multiple of 16) from src; out receives `grid` uint32 words (zeroed by
// the caller). Returns a hipError_t.
__attribute__((visibility("default"))) int bl_ceil_stream_read(const void* src, int64_t bytes,
                                                               uint32_t* out, int grid,
                                                               void* stream) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(kReadThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src), bytes / 16,
                     out);
  return static_cast<int>(hipGetLastError());
}

// The same bytes in `grid` contiguous slices, one per workgroup; bytes must be a multiple of
// grid * 32 KiB. Returns a hipError_t (hipErrorInvalidValue for other sizes).
__attribute__((visibility("default"))) int bl_ceil_stream_read_slices(const void* src,
                                                                      int64_t bytes,
                                                                      uint32_t* out, int grid,
                                                                      void* stream) {
  const int64_t slice = grid > 0 ? bytes / grid : 0;
  if (grid <= 0 || slice * grid != bytes || slice % (kReadThreads * kReadUnroll * 16) != 0)
    return static_cast<int>(hipErrorInvalidValue);
  hipLaunchKernelGGL(stream_read_slices_kernel, dim3(grid), dim3(kReadThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src), slice / 16,
                     out);
  return static_cast<int>(hipGetLastError());
}

// `grid` workgroups of four waves, `iters` rounds of eight MFMAs per wave; out receives
// grid * 256 int32x4 (16 bytes per thread). Returns a hipError_t.
__attribute__((visibility("default"))) int bl_ceil_mfma_i8(int iters, int grid, void* out,
                                                           void* stream) {
  hipLaunchKernelGGL(mfma_i8_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     iters, 1, static_cast<i32x4*>(out));
  return static_cast<int>(hipGetLastError());
}

// int8 operations one bl_ceil_mfma_i8 call performs.
__attribute__((visibility("default"))) double bl_ceil_mfma_i8_ops(int iters, int grid) {
  return 2.0 * 16 * 16 * 64 * kMfmaAcc * static_cast<double>(iters) * grid * 4;
}

}  // extern "C"
