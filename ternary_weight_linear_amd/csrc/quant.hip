// Per-token absmax int8 activation quantiser.
//
// [b158] "BitNet b1.58 介绍": activations are scaled per token into [-Q_b, Q_b] with no
// zero point (the [0, Q_b] variant of the original BitNet is dropped). Reading used here:
// Q_b = 127, gamma = max |x| over the token, q = clip(rne(fl32(127 x) / gamma)); 127 x is
// exact in fp32 for fp16 x, so the fp32 division is the only rounding (its correctly rounded
// result decides q; quant_q forms it from a reciprocal and falls back to the IEEE division
// where the two could round apart).
//
// One workgroup per token row. Pass 1 copies the fp16 row into LDS while reducing |x| to
// gamma with wavefront reductions. Pass 2 gives each wave one 64-input tile at a time:
// lane l holds the input whose X8-64 bit position is l, so eight __ballot calls produce
// the eight activation bit planes of the tile directly. When no planes are asked for, a
// second kernel keeps the row in registers instead (below).
#include "bl_internal.h"

namespace bl {
namespace {

template <int BLOCK>
__global__ __launch_bounds__(BLOCK) void quant_act_kernel(const uint16_t* __restrict__ x,
                                                          int64_t K, int8_t* __restrict__ q,
                                                          float* __restrict__ gamma,
                                                          int32_t* __restrict__ rowsum,
                                                          uint32_t* __restrict__ planes) {
  extern __shared__ uint16_t xs[];                 // the row, K halves
  __shared__ float red_max[BLOCK / 64];
  __shared__ int red_bad[BLOCK / 64];
  __shared__ int red_sum[BLOCK / 64];
  const int64_t m = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  constexpr int NW = BLOCK / 64;
  const uint4* row4 = reinterpret_cast<const uint4*>(x + m * K);
  uint4* xs4 = reinterpret_cast<uint4*>(xs);

  float mx = 0.0f;
  int bad = 0;
  for (int64_t i = threadIdx.x; i < K / 8; i += BLOCK) {
    const uint4 v = row4[i];
    xs4[i] = v;
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint16_t lo = static_cast<uint16_t>(w[j] & 0xFFFFu), hi = static_cast<uint16_t>(w[j] >> 16);
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
  if (lane == 0) { red_max[wave] = mx; red_bad[wave] = bad; }
  __syncthreads();
  mx = red_max[0];
  bad = red_bad[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) { mx = fmaxf(mx, red_max[w]); bad |= red_bad[w]; }
  const float g = bad ? __uint_as_float(0x7FC00000u) : mx;
  if (threadIdx.x == 0) gamma[m] = g;
  const bool zero = bad || mx == 0.0f;
  const float rg = __builtin_amdgcn_rcpf(zero ? 1.0f : g);

  // Pass 2. Lane l <-> bit l of the tile's 64-bit plane mask: h = l / 32, bit p = l % 32
  // = 8i + j  <->  input c = 4j + i of half h.
  const int h = lane >> 5, p = lane & 31;
  const int c = 4 * (p & 7) + (p >> 3);
  const int koff = 32 * h + c;
  const int64_t KT = K / 64;
  int sum = 0;
  for (int64_t t = wave; t < KT; t += NW) {
    const int64_t k = 64 * t + koff;
    const int qv = zero ? 0 : quant_q(half_bits_to_float(xs[k]) * 127.0f, g, rg);
    sum += qv;
    if (q) q[m * K + k] = static_cast<int8_t>(qv);
    if (planes) {
      uint32_t mine = 0;
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const unsigned long long mask = __ballot((qv >> b) & 1);
        if ((lane >> 1) == b) mine = (lane & 1) ? static_cast<uint32_t>(mask >> 32) : static_cast<uint32_t>(mask);
      }
      if (lane < 16) planes[(m * KT + t) * 16 + lane] = mine;
    }
  }
  if (rowsum) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
    __syncthreads();
    if (lane == 0) red_sum[wave] = sum;
    __syncthreads();
    if (threadIdx.x == 0) {
      int s = 0;
      for (int w = 0; w < NW; ++w) s += red_sum[w];
      rowsum[m] = s;
    }
  }
}

// Without bit planes the lane order of pass 2 is not needed: each thread quantises the
// (up to NV x 8) inputs it loaded, straight from registers, and stores them as contiguous
// bytes. Same arithmetic per element; one load, two workgroup barriers (gamma, row sum).
template <int BLOCK, int NV>
__global__ __launch_bounds__(BLOCK) void quant_act_regs_kernel(const uint16_t* __restrict__ x,
                                                               int64_t K, int8_t* __restrict__ q,
                                                               float* __restrict__ gamma,
                                                               int32_t* __restrict__ rowsum) {
  __shared__ uint32_t red_max[BLOCK / 64];
  __shared__ int red_sum[BLOCK / 64];
  constexpr int NW = BLOCK / 64;
  const int64_t m = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const uint4* row4 = reinterpret_cast<const uint4*>(x + m * K);
  const int64_t K8 = K / 8;
  uint4 v[NV];
#pragma unroll
  for (int n = 0; n < NV; ++n) v[n] = row4[min<int64_t>(threadIdx.x + BLOCK * n, K8 - 1)];
  // gamma: for finite fp16 the magnitude order is the integer order of the bits with the
  // sign cleared, so this is an integer max (>= 0x7C00 flags NaN/inf)
  uint32_t mb = 0;
#pragma unroll
  for (int n = 0; n < NV; ++n) {
    const uint32_t w[4] = {v[n].x, v[n].y, v[n].z, v[n].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) mb = max(mb, max(w[j] & 0x7FFFu, (w[j] >> 16) & 0x7FFFu));
  }
  mb = wave_max_u32(mb);
  if (lane == 0) red_max[wave] = mb;
  __syncthreads();
  mb = red_max[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) mb = max(mb, red_max[w]);
  const bool bad = mb >= 0x7C00u;
  const float g = bad ? __uint_as_float(0x7FC00000u) : half_bits_to_float(static_cast<uint16_t>(mb));
  if (threadIdx.x == 0) gamma[m] = g;
  const bool zero = bad || mb == 0u;
  const float rg = __builtin_amdgcn_rcpf(zero ? 1.0f : g);

  int sum = 0;
#pragma unroll
  for (int n = 0; n < NV; ++n) {
    const int64_t i = threadIdx.x + BLOCK * n;
    // a guarded body, not a break: with a break the compiler left the loop rolled for NV = 16
    // and indexed v[] in scratch memory (272 bytes per lane)
    if (i >= K8) continue;
    const uint32_t w[4] = {v[n].x, v[n].y, v[n].z, v[n].w};
    float a[8], ge[8], rge[8];
    bool ze[8];
    int qv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = half_bits_to_float(static_cast<uint16_t>((w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu)) * 127.0f;
      ge[e] = g, rge[e] = rg, ze[e] = zero;
    }
    quant_q_n(a, ge, rge, ze, qv);
    uint32_t packed[2] = {0, 0};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sum += qv[e];
      packed[e >> 2] |= (static_cast<uint32_t>(qv[e]) & 0xFFu) << (8 * (e & 3));
    }
    if (q) *reinterpret_cast<uint2*>(q + m * K + 8 * i) = make_uint2(packed[0], packed[1]);
  }
  if (rowsum) {
    sum = wave_sum_i32(sum);
    if (lane == 0) red_sum[wave] = sum;
    __syncthreads();
    if (threadIdx.x == 0) {
      int s = 0;
      for (int w = 0; w < NW; ++w) s += red_sum[w];
      rowsum[m] = s;
    }
  }
}

}  // namespace

hipError_t launch_quant_act(const uint16_t* x, int64_t M, int64_t K, int8_t* q, float* gamma,
                            int32_t* rowsum, uint32_t* planes, hipStream_t s) {
  if (!planes) {
    // one workgroup per row, every input of the row in registers: the smallest build whose
    // BLOCK * NV 16-byte loads cover the row (the loads past it repeat its last piece)
    const int64_t K8 = K / 8;
    const dim3 grid(static_cast<unsigned>(M));
    if (M <= 64) {
      if (K8 <= 1024) hipLaunchKernelGGL((quant_act_regs_kernel<1024, 1>), grid, dim3(1024), 0, s, x, K, q, gamma, rowsum);
      else if (K8 <= 2048) hipLaunchKernelGGL((quant_act_regs_kernel<1024, 2>), grid, dim3(1024), 0, s, x, K, q, gamma, rowsum);
      else hipLaunchKernelGGL((quant_act_regs_kernel<1024, 4>), grid, dim3(1024), 0, s, x, K, q, gamma, rowsum);
    } else {
      if (K8 <= 512) hipLaunchKernelGGL((quant_act_regs_kernel<256, 2>), grid, dim3(256), 0, s, x, K, q, gamma, rowsum);
      else if (K8 <= 1024) hipLaunchKernelGGL((quant_act_regs_kernel<256, 4>), grid, dim3(256), 0, s, x, K, q, gamma, rowsum);
      else if (K8 <= 2048) hipLaunchKernelGGL((quant_act_regs_kernel<256, 8>), grid, dim3(256), 0, s, x, K, q, gamma, rowsum);
      else hipLaunchKernelGGL((quant_act_regs_kernel<256, 16>), grid, dim3(256), 0, s, x, K, q, gamma, rowsum);
    }
    return hipGetLastError();
  }
  const size_t lds = static_cast<size_t>(K) * sizeof(uint16_t);
  if (M <= 64) {
    hipLaunchKernelGGL(quant_act_kernel<1024>, dim3(static_cast<unsigned>(M)), dim3(1024), lds, s,
                       x, K, q, gamma, rowsum, planes);
  } else {
    hipLaunchKernelGGL(quant_act_kernel<256>, dim3(static_cast<unsigned>(M)), dim3(256), lds, s,
                       x, K, q, gamma, rowsum, planes);
  }
  return hipGetLastError();
}

}  // namespace bl
