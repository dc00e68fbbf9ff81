// Residual binarisation as an inference format: W ~ alpha_o ⊙ B_o + alpha_r ⊙ B_r.
//
// [billm] "方法细节", step 2 (binary residual approximation): the weight is binarised once
// and the residual of that approximation is binarised again; the sum of the two scaled sign
// matrices replaces W. Here every group is one output row by the 128 inputs of one S1-128
// tile, each group carrying two fp32 scales, and the two sign planes use the S1-128 layout
// of the OneBit path.
//
// Packing (offline): alpha is the group's mean magnitude, the fp32 value nearest the exact
// mean (one rounding, ties to even; no summation order enters the result). A wave holds one
// group with inputs 2l, 2l+1 in lane l. Each magnitude m * 2^(e-150) (integer m < 2^24) is
// the integer m << (e-1) in units of 2^-149; its pieces in 32-bit limbs at fixed bit
// positions are summed over the wave in 64-bit integers (exact: 128 pieces < 2^32), the
// carries are propagated, and the 288-bit total times 2^-156 (the division by 128) is
// rounded once. The residual R = W -+ alpha_o is one fp32 rounding, and the lanes' sign
// bits are gathered into the row's four S1-128 words with two ballots per plane.
//
// Forward: y[m, n] = sum_b alpha_o[n, b] (x_b . B_o[n, b]) + alpha_r[n, b] (x_b . B_r[n, b]).
// Both group dot products run on fp16 matrix cores with B = +-1.0 built from the packed
// bits (the products x * +-1 are exact); each 128-input tile's two fp32 results are scaled
// by the lane's own column scales and added to the running sum (the shared sign-plane
// kernel of sign_mfma.h, which also serves the OneBit layer).
#include <algorithm>

#include "sign_mfma.h"

namespace bl {
namespace {

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), off);
    const uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), off);
    v += (static_cast<uint64_t>(hi) << 32) | lo;
  }
  return v;
}

// Position of |v| as an integer in units of 2^-149: limb index (32-bit limbs) and the
// significand shifted within its limb (< 2^55, spilling into the next limb).
__device__ __forceinline__ void abs_units(float v, int& limb, uint64_t& shifted) {
  const uint32_t u = __float_as_uint(v) & 0x7FFFFFFFu;
  const int e = static_cast<int>(u >> 23);
  const uint32_t m = e ? ((u & 0x7FFFFFu) | 0x800000u) : u;
  const int p = (e ? e : 1) - 1;
  limb = p >> 5;
  shifted = static_cast<uint64_t>(m) << (p & 31);
}

// The fp32 value nearest the exact mean of |a|, |b| over the wave's 128 values (ties to
// even). NaN anywhere gives NaN, else inf anywhere gives inf. Every lane returns the result.
__device__ float group_abs_mean_exact(float a, float b) {
  const uint32_t ua = __float_as_uint(a) & 0x7FFFFFFFu, ub = __float_as_uint(b) & 0x7FFFFFFFu;
  if (__builtin_amdgcn_ballot_w64(ua > 0x7F800000u || ub > 0x7F800000u))
    return __uint_as_float(0x7FC00000u);
  if (__builtin_amdgcn_ballot_w64(ua == 0x7F800000u || ub == 0x7F800000u))
    return __uint_as_float(0x7F800000u);
  int la, lb;
  uint64_t va, vb;
  abs_units(a, la, va);
  abs_units(b, lb, vb);
  constexpr int L = 9;                               // 288 bits > 2^7 * 2^277
  uint32_t A[L];
  uint64_t carry = 0;
#pragma unroll
  for (int j = 0; j < L; ++j) {
    uint64_t c = (la == j ? (va & 0xFFFFFFFFu) : 0u) + (la + 1 == j ? (va >> 32) : 0u) +
                 (lb == j ? (vb & 0xFFFFFFFFu) : 0u) + (lb + 1 == j ? (vb >> 32) : 0u);
    c = wave_sum_u64(c) + carry;
    A[j] = static_cast<uint32_t>(c);
    carry = c >> 32;
  }
  // mean = A * 2^-156. Keep 24 significant bits (never finer than the subnormal spacing
  // 2^-149 = 2^7 units), round half to even on the dropped bits.
  int top = -1;
#pragma unroll
  for (int j = L - 1; j >= 0; --j)
    if (top < 0 && A[j]) top = 32 * j + 31 - __builtin_clz(A[j]);
  if (top < 0) return 0.0f;
  const int shift = top - 23 > 7 ? top - 23 : 7;
  auto bit = [&](int pos) -> uint32_t { return (A[pos >> 5] >> (pos & 31)) & 1u; };
  uint32_t mant = 0;
  for (int i = 0; i < 24 && shift + i <= top; ++i) mant |= bit(shift + i) << i;
  const uint32_t half = bit(shift - 1);
  bool below = false;
  for (int i = 0; i < shift - 1 && !below; ++i) below = bit(i) != 0;
  if (half && (below || (mant & 1u))) ++mant;
  // value = mant * 2^(shift - 156); for shift = 7 and mant < 2^23 this is the subnormal
  // encoding, otherwise the biased exponent is shift - 6 (a carry to 2^24 bumps it).
  return __uint_as_float((static_cast<uint32_t>(shift - 7) << 23) + mant);
}

// Lane l of the packing wave holds tile inputs 2l, 2l + 1, i.e. c = 32s + 8g + 2q + e with
// l = 16s + 4g + q. The S1-128 word of record g for this row takes bit 4s + q (+16 for the
// odd input) from ballot bit 16s + 4g + q.
__device__ __forceinline__ uint32_t s1_word(uint64_t even, uint64_t odd, int g) {
  uint32_t w = 0;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    w |= static_cast<uint32_t>((even >> (16 * s + 4 * g)) & 0xFu) << (4 * s);
    w |= static_cast<uint32_t>((odd >> (16 * s + 4 * g)) & 0xFu) << (16 + 4 * s);
  }
  return w;
}

__global__ __launch_bounds__(256) void residual_pack_kernel(
    const float* __restrict__ W, int64_t N, int64_t K, uint32_t* __restrict__ Po,
    float* __restrict__ alpha_o, uint32_t* __restrict__ Pr, float* __restrict__ alpha_r) {
  const int lane = threadIdx.x & 63;
  const int64_t KB = K / 128;
  const int64_t item = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (item >= N * KB) return;                           // whole waves leave together
  const int64_t n = item / KB, b = item % KB;
  const float2 w = reinterpret_cast<const float2*>(W + n * K + b * 128)[lane];
  const float ao = group_abs_mean_exact(w.x, w.y);
  const bool n0 = w.x < 0.0f, n1 = w.y < 0.0f;
  const float r0 = w.x - (n0 ? -ao : ao);
  const float r1 = w.y - (n1 ? -ao : ao);
  const float ar = group_abs_mean_exact(r0, r1);
  const uint64_t bo_e = __builtin_amdgcn_ballot_w64(n0), bo_o = __builtin_amdgcn_ballot_w64(n1);
  const uint64_t br_e = __builtin_amdgcn_ballot_w64(r0 < 0.0f);
  const uint64_t br_o = __builtin_amdgcn_ballot_w64(r1 < 0.0f);
  if (lane < 4) {                                        // lane g writes record 16g + u
    const int f = static_cast<int>((n >> 4) & 3), u = static_cast<int>(n & 15);
    const int64_t word = (((n >> 6) * KB + b) * 64 + 16 * lane + u) * 4 + f;
    Po[word] = s1_word(bo_e, bo_o, lane);
    Pr[word] = s1_word(br_e, br_o, lane);
  }
  if (lane == 0) {
    alpha_o[n * KB + b] = ao;
    alpha_r[n * KB + b] = ar;
  }
}

}  // namespace

size_t residual_part_floats(int64_t M, int64_t N, int64_t K) {
  if (N % 64 || K % 128) return 0;
  return sign_mfma_part_floats(M, N, K, true);
}

hipError_t launch_residual_binarize(const float* W, int64_t N, int64_t K, void* planes_o,
                                    float* alpha_o, void* planes_r, float* alpha_r,
                                    hipStream_t s) {
  const int64_t items = N * (K / 128);
  hipLaunchKernelGGL(residual_pack_kernel, dim3(static_cast<unsigned>((items + 3) / 4)), dim3(256),
                     0, s, W, N, K, static_cast<uint32_t*>(planes_o), alpha_o,
                     static_cast<uint32_t*>(planes_r), alpha_r);
  return hipGetLastError();
}

hipError_t launch_residual_linear(const uint16_t* x, const void* planes_o, const float* alpha_o,
                                  const void* planes_r, const float* alpha_r, int64_t M, int64_t N,
                                  int64_t K, float* y, float* ws_part, uint32_t* ws_cnt,
                                  hipStream_t s) {
  SignMfmaArgs a{};
  a.x = x;
  a.p0 = static_cast<const sm_u32x4*>(planes_o);
  a.p1 = static_cast<const sm_u32x4*>(planes_r);
  a.a0 = alpha_o;
  a.a1 = alpha_r;
  a.M = M, a.N = N, a.K = K;
  a.y = y, a.part = ws_part, a.cnt = ws_cnt;
  return launch_sign_mfma<true>(a, s);
}

}  // namespace bl
