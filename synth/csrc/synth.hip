// GPU twin of synth.ternary_codes: counter-based ternary codes from SplitMix64
// (Steele, Lea and Flood, OOPSLA 2014). Input generation only: none of the layers'
// arithmetic lives here. Code (n, k) of a matrix with key `key` is
//     splitmix64_output(key, n*K + k + 1) mod 3 - 1,
// where the i-th output is the finaliser applied to key + i * 0x9E3779B97F4A7C15.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ __forceinline__ uint64_t splitmix64(uint64_t key, uint64_t i) {
  uint64_t z = key + i * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__global__ void ternary_codes_kernel(int8_t* __restrict__ out, int64_t rows, int64_t K,
                                     uint64_t key, int64_t row0) {
  const int64_t total = rows * K;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / K, k = i % K;
    const uint64_t ctr = static_cast<uint64_t>((row0 + r) * K + k + 1);
    out[i] = static_cast<int8_t>(static_cast<int>(splitmix64(key, ctr) % 3ull) - 1);
  }
}

}  // namespace

extern "C" {

// Writes codes of rows row0 .. row0+rows-1 of a [*, K] matrix into out[rows, K] (device).
// Returns 0 or the HIP error code of the launch.
int syn_ternary_codes(int8_t* out, int64_t rows, int64_t K, uint64_t key, int64_t row0,
                      void* stream) {
  if (!out || rows < 1 || K < 1) return -1;
  const int64_t total = rows * K;
  const int64_t blocks = std::min<int64_t>((total + 255) / 256, 65536);
  hipLaunchKernelGGL(ternary_codes_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), out, rows, K, key, row0);
  return static_cast<int>(hipGetLastError());
}

}  // extern "C"
