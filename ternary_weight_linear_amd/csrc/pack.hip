// Offline weight preparation: T2-PN-64 ternary packing, S1-128 sign packing and the
// exact absmean ternariser, plus the workspace fill kernel.
//
// Ternary weights and their 2-bit storage: [b158] "BitNet b1.58 介绍" (values -1, 0, +1)
// and "实验及结果" (2-bit kernel). Sign-only storage: [onebit] "1. 新的1bit结构" and
// "3. 通过知识蒸馏迁移原模型能力" (only Sign(W) kept for inference).
//
// One thread owns one 16-byte row of one 1 KiB tile, so the packed stream is written with
// fully coalesced 16-byte stores (64 lanes x 16 B = one tile).
#include "bl_internal.h"

namespace bl {
namespace {

// Bit position of input c (0..31) inside a T2-PN-64 / X8-64 word: c = 4j + i -> 8i + j.
__device__ __forceinline__ int t2_bit(int c) { return 8 * (c & 3) + (c >> 2); }

__global__ void fill_zero_kernel(uint4* p16, size_t n16, unsigned char* tail, size_t ntail) {
  size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t j = i; j < n16; j += stride) p16[j] = make_uint4(0, 0, 0, 0);
  if (i < ntail) tail[i] = 0;
}

// codes int8 [N, K] -> T2-PN-64. Thread g <-> (tile = g / 64, row r = g % 64).
__global__ void pack_ternary_kernel(const int8_t* __restrict__ codes, int64_t N, int64_t K,
                                    uint4* __restrict__ out, int32_t* n_invalid) {
  const int64_t KT = K / 64;
  const int64_t g = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (g >= N * KT) return;
  const int64_t tile = g >> 6, r = g & 63;
  const int64_t tn = tile / KT, tk = tile % KT;
  const int64_t n = tn * 64 + r;
  const uint4* src = reinterpret_cast<const uint4*>(codes + n * K + tk * 64);
  uint32_t P[2] = {0, 0}, M[2] = {0, 0};
  int bad = 0;
#pragma unroll
  for (int chunk = 0; chunk < 4; ++chunk) {
    uint4 v = src[chunk];
    uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int b = 0; b < 16; ++b) {
      const int8_t code = static_cast<int8_t>((w4[b >> 2] >> (8 * (b & 3))) & 0xFF);
      const int kk = chunk * 16 + b;         // 0..63 inside the tile
      const int h = kk >> 5, c = kk & 31;
      const uint32_t bit = 1u << t2_bit(c);
      if (code == 1) P[h] |= bit;
      else if (code == -1) M[h] |= bit;
      else if (code != 0) ++bad;
    }
  }
  out[g] = make_uint4(P[0], P[1], M[0], M[1]);
  if (bad && n_invalid) atomicAdd(n_invalid, bad);
}

__global__ void unpack_ternary_kernel(const uint4* __restrict__ in, int64_t N, int64_t K,
                                      int8_t* __restrict__ codes, int32_t* n_invalid) {
  const int64_t KT = K / 64;
  const int64_t g = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (g >= N * KT) return;
  const int64_t tile = g >> 6, r = g & 63;
  const int64_t tn = tile / KT, tk = tile % KT;
  const int64_t n = tn * 64 + r;
  const uint4 w = in[g];
  const uint32_t P[2] = {w.x, w.y}, M[2] = {w.z, w.w};
  int bad = 0;
  uint4* dst = reinterpret_cast<uint4*>(codes + n * K + tk * 64);
#pragma unroll
  for (int chunk = 0; chunk < 4; ++chunk) {
    uint32_t o[4] = {0, 0, 0, 0};
#pragma unroll
    for (int b = 0; b < 16; ++b) {
      const int kk = chunk * 16 + b;
      const int h = kk >> 5, c = kk & 31;
      const int s = t2_bit(c);
      const uint32_t p = (P[h] >> s) & 1u, m = (M[h] >> s) & 1u;
      int code = static_cast<int>(p) - static_cast<int>(m);
      if (p & m) { code = 0; ++bad; }
      o[b >> 2] |= (static_cast<uint32_t>(code) & 0xFFu) << (8 * (b & 3));
    }
    dst[chunk] = make_uint4(o[0], o[1], o[2], o[3]);
  }
  if (bad && n_invalid) atomicAdd(n_invalid, bad);
}

// float W [N, K] -> S1-128. Thread i <-> one 16-byte record: tile i / 64, record L = i % 64
// = 16g + u, holding word f (rows 16f + u) with the signs of tile inputs 32s + 8g + j,
// j = 2q + e, at bit 16e + 4s + q.
// T2-MF64: one thread per 16-byte record of a tile (record 16g + u: word j holds, at bits
// 8i + 2f, the field of row 16f + u, input 16g + 4j + i of the tile: w + 1 for f < 3, w in
// two's complement for f = 3). Invalid codes pack as w = 0 and are counted.
__global__ void pack_ternary_mf_kernel(const int8_t* __restrict__ codes, int64_t N, int64_t K,
                                       uint4* __restrict__ out, int32_t* n_invalid) {
  const int64_t KT = K / 64;
  const int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (idx >= N * KT) return;
  const int64_t tile = idx >> 6;
  const int rec = static_cast<int>(idx & 63), g = rec >> 4, u = rec & 15;
  const int64_t tn = tile / KT, tk = tile % KT;
  uint32_t word[4] = {0, 0, 0, 0};
  int bad = 0;
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const int64_t n = tn * 64 + 16 * f + u;
    const uint4 v = *reinterpret_cast<const uint4*>(codes + n * K + tk * 64 + 16 * g);
    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};   // w4[j] byte i = code of input 16g + 4j + i
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int c = static_cast<int8_t>((w4[j] >> (8 * i)) & 0xFF);
        if (c != 1 && c != 0 && c != -1) {
          c = 0;
          ++bad;
        }
        const uint32_t field = f < 3 ? static_cast<uint32_t>(c + 1) : static_cast<uint32_t>(c) & 3u;
        word[j] |= field << (8 * i + 2 * f);
      }
  }
  out[idx] = make_uint4(word[0], word[1], word[2], word[3]);
  if (bad && n_invalid) atomicAdd(n_invalid, bad);
}

// T2-PN-64 -> T2-MF64, one thread per output record. Input 16g + 4j + i of a tile row is
// bit 8i + 4(g % 2) + j of half g / 2 of the row's P and N words. Per byte the field is
// 1 + p - n for f < 3 (no byte ever borrows: 1 + p >= n) and p | 3n for f = 3 (01 / 11).
// A (P, N) = (1, 1) pair becomes w = 0 and is counted.
__global__ void repack_pn_to_mf_kernel(const uint4* __restrict__ in, int64_t N, int64_t K,
                                       uint4* __restrict__ out, int32_t* n_invalid) {
  const int64_t KT = K / 64;
  const int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (idx >= N * KT) return;
  const int64_t tile = idx >> 6;
  const int rec = static_cast<int>(idx & 63), g = rec >> 4, u = rec & 15;
  uint32_t word[4] = {0, 0, 0, 0};
  int bad = 0;
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const uint4 row = in[tile * 64 + 16 * f + u];
    const uint32_t P = (g >> 1) ? row.y : row.x, Nm = (g >> 1) ? row.w : row.z;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int sh = 4 * (g & 1) + j;
      const uint32_t pb = (P >> sh) & 0x01010101u, nb = (Nm >> sh) & 0x01010101u;
      const uint32_t both = pb & nb;
      bad += __builtin_popcount(both);
      const uint32_t p = pb ^ both, n = nb ^ both;
      const uint32_t field = f < 3 ? (0x01010101u + p) - n : p | (n * 3u);
      word[j] |= field << (2 * f);
    }
  }
  out[idx] = make_uint4(word[0], word[1], word[2], word[3]);
  if (bad && n_invalid) atomicAdd(n_invalid, bad);
}

__global__ void pack_sign_kernel(const float* __restrict__ W, int64_t N, int64_t K,
                                 uint4* __restrict__ out) {
  const int64_t KT = K / 128;
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= N * KT) return;
  const int64_t tile = i >> 6;
  const int L = static_cast<int>(i & 63), g = L >> 4, u = L & 15;
  const int64_t tn = tile / KT, tk = tile % KT;
  uint32_t S[4] = {0, 0, 0, 0};
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const float* row = W + (tn * 64 + 16 * f + u) * K + tk * 128 + 8 * g;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const float4 lo = reinterpret_cast<const float4*>(row + 32 * s)[0];
      const float4 hi = reinterpret_cast<const float4*>(row + 32 * s)[1];
      const float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (v[j] < 0.0f) S[f] |= 1u << (16 * (j & 1) + 4 * s + (j >> 1));
    }
  }
  out[i] = make_uint4(S[0], S[1], S[2], S[3]);
}

__global__ void unpack_sign_kernel(const uint4* __restrict__ in, int64_t N, int64_t K,
                                   int8_t* __restrict__ signs) {
  const int64_t KT = K / 128;
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= N * KT) return;
  const int64_t tile = i >> 6;
  const int L = static_cast<int>(i & 63), g = L >> 4, u = L & 15;
  const int64_t tn = tile / KT, tk = tile % KT;
  const uint4 w = in[i];
  const uint32_t S[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    int8_t* row = signs + (tn * 64 + 16 * f + u) * K + tk * 128 + 8 * g;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint32_t o[2] = {0, 0};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t neg = (S[f] >> (16 * (j & 1) + 4 * s + (j >> 1))) & 1u;
        o[j >> 2] |= (neg ? 0xFFu : 0x01u) << (8 * (j & 3));
      }
      reinterpret_cast<uint2*>(row + 32 * s)[0] = make_uint2(o[0], o[1]);
    }
  }
}

// ---- exact absmean -------------------------------------------------------------------------
// |W| = m * 2^(e - 150) with integer m < 2^24 (subnormals: e = 1, no hidden bit). Integer
// sums of m per exponent field are exact and order-free, so the mean is computed exactly
// and rounded once. Bin 255 counts non-finite values.
__global__ __launch_bounds__(256) void absmean_hist_kernel(const float* __restrict__ W,
                                                           int64_t total,
                                                           unsigned long long* __restrict__ bins) {
  __shared__ unsigned long long hist[4][kAbsmeanBins];
  const int wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < 4 * kAbsmeanBins; i += blockDim.x) (&hist[0][0])[i] = 0;
  __syncthreads();
  const float4* W4 = reinterpret_cast<const float4*>(W);
  const int64_t n4 = total / 4;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n4;
       i += (int64_t)gridDim.x * blockDim.x) {
    const float4 v = W4[i];
    const float e4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t bits = __float_as_uint(e4[u]) & 0x7FFFFFFFu;
      uint32_t e = bits >> 23;
      uint32_t m = bits & 0x7FFFFFu;
      if (e == 255) { atomicAdd(&hist[wave][255], 1ull); continue; }
      if (e) m |= 0x800000u; else e = 1;
      if (m) atomicAdd(&hist[wave][e], (unsigned long long)m);
    }
  }
  __syncthreads();
  for (int b = threadIdx.x; b < kAbsmeanBins; b += blockDim.x)
    bins[blockIdx.x * (int64_t)kAbsmeanBins + b] = hist[0][b] + hist[1][b] + hist[2][b] + hist[3][b];
}

// Round the exact mean (sum of the bins, in units of 2^-149, divided by `count`) to the
// nearest fp32 (ties to even) and write it to *beta.
__global__ __launch_bounds__(256) void absmean_finalize_kernel(
    const unsigned long long* __restrict__ bins, int nblk, uint32_t count, float* beta) {
  __shared__ unsigned long long S[kAbsmeanBins];
  const int e = threadIdx.x;
  unsigned long long s = 0;
  for (int b = 0; b < nblk; ++b) s += bins[b * (int64_t)kAbsmeanBins + e];
  S[e] = s;
  __syncthreads();
  if (threadIdx.x != 0) return;
  if (S[255] != 0) { *beta = __uint_as_float(0x7FC00000u); return; }
  constexpr int L = 12;                      // 384-bit accumulator, units of 2^-149
  uint32_t A[L];
  for (int i = 0; i < L; ++i) A[i] = 0;
  for (int ex = 1; ex < 255; ++ex) {
    const unsigned long long v = S[ex];
    if (!v) continue;
    const int sh = ex - 1, w = sh >> 5, b = sh & 31;
    const unsigned long long lo = v << b;
    const uint32_t hi = b ? static_cast<uint32_t>(v >> (64 - b)) : 0u;
    uint32_t add[3] = {static_cast<uint32_t>(lo), static_cast<uint32_t>(lo >> 32), hi};
    unsigned long long carry = 0;
    for (int i = w; i < L; ++i) {
      const unsigned long long t = (unsigned long long)A[i] + (i - w < 3 ? add[i - w] : 0u) + carry;
      A[i] = static_cast<uint32_t>(t);
      carry = t >> 32;
      if (i - w >= 2 && carry == 0) break;
    }
  }
  // Q = floor(A / count), rem = A mod count
  uint32_t Q[L];
  unsigned long long rem = 0;
  for (int i = L - 1; i >= 0; --i) {
    const unsigned long long cur = (rem << 32) | A[i];
    Q[i] = static_cast<uint32_t>(cur / count);
    rem = cur % count;
  }
  int top = -1;
  for (int i = L - 1; i >= 0; --i) if (Q[i]) { top = i; break; }
  uint32_t bitsout;
  if (top < 0 || (top == 0 && Q[0] < (1u << 24))) {
    // value = (Q + rem/count) * 2^-149 with Q < 2^24: the fp32 encoding of j * 2^-149 is j
    const uint32_t q0 = top < 0 ? 0u : Q[0];
    const unsigned long long twice = 2ull * rem;
    const bool up = twice > count || (twice == count && (q0 & 1u));
    bitsout = q0 + (up ? 1u : 0u);
  } else {
    const int p = 32 * top + 31 - __builtin_clz(Q[top]);   // msb position, >= 24
    int s = p - 23;
    auto bit = [&](int pos) -> uint32_t { return (Q[pos >> 5] >> (pos & 31)) & 1u; };
    uint32_t mant = 0;
    for (int i = 0; i < 24; ++i) mant |= bit(s + i) << i;
    const uint32_t half = bit(s - 1);
    bool below = rem != 0;
    for (int i = 0; i < s - 1 && !below; ++i) below = bit(i) != 0;
    const bool up = half && (below || (mant & 1u));
    mant += up ? 1u : 0u;
    if (mant == (1u << 24)) { mant >>= 1; ++s; }
    bitsout = (static_cast<uint32_t>(s + 1) << 23) | (mant - (1u << 23));
  }
  *beta = __uint_as_float(bitsout);
}

// Codes from beta and pack (and/or write int8 codes). Same thread mapping as the packer.
__global__ void ternarize_pack_kernel(const float* __restrict__ W, int64_t N, int64_t K,
                                      const float* __restrict__ beta_p, int8_t* __restrict__ codes,
                                      uint4* __restrict__ out) {
  const int64_t KT = K / 64;
  const int64_t g = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (g >= N * KT) return;
  const int64_t tile = g >> 6, r = g & 63;
  const int64_t tn = tile / KT, tk = tile % KT;
  const int64_t n = tn * 64 + r;
  const float beta = *beta_p;
  const bool valid = (beta > 0.0f) && (beta <= 3.402823466e38f);   // false for NaN and 0
  const float4* src = reinterpret_cast<const float4*>(W + n * K + tk * 64);
  uint32_t P[2] = {0, 0}, M[2] = {0, 0};
  uint32_t cw[16];
#pragma unroll
  for (int v4 = 0; v4 < 16; ++v4) {
    const float4 v = src[v4];
    const float e[4] = {v.x, v.y, v.z, v.w};
    uint32_t packedc = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int kk = v4 * 4 + u;
      int c = 0;
      if (valid) {
        const float rr = rintf(e[u] / beta);      // IEEE division, round half to even
        c = rr > 0.0f ? 1 : (rr < 0.0f ? -1 : 0);
      }
      const uint32_t bit = 1u << t2_bit(kk & 31);
      if (c == 1) P[kk >> 5] |= bit;
      if (c == -1) M[kk >> 5] |= bit;
      packedc |= (static_cast<uint32_t>(c) & 0xFFu) << (8 * u);
    }
    cw[v4] = packedc;
  }
  if (out) out[g] = make_uint4(P[0], P[1], M[0], M[1]);
  if (codes) {
    uint4* dst = reinterpret_cast<uint4*>(codes + n * K + tk * 64);
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = make_uint4(cw[4 * i], cw[4 * i + 1], cw[4 * i + 2], cw[4 * i + 3]);
  }
}

inline unsigned grid_for(int64_t threads, int block) {
  return static_cast<unsigned>((threads + block - 1) / block);
}

}  // namespace

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
  if (bytes == 0) return hipSuccess;
  unsigned char* base = static_cast<unsigned char*>(p);
  const uintptr_t addr = reinterpret_cast<uintptr_t>(base);
  size_t head = (16 - (addr & 15)) & 15;
  if (head > bytes) head = bytes;
  // head bytes are cleared by the tail path of a second tiny launch
  const size_t n16 = (bytes - head) / 16;
  const size_t ntail = bytes - head - n16 * 16;
  if (n16 || ntail) {
    const size_t blocks = n16 ? std::min<size_t>((n16 + 255) / 256, 4096) : 1;
    hipLaunchKernelGGL(fill_zero_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                       reinterpret_cast<uint4*>(base + head), n16, base + head + n16 * 16, ntail);
  }
  if (head)
    hipLaunchKernelGGL(fill_zero_kernel, dim3(1), dim3(64), 0, s, static_cast<uint4*>(nullptr),
                       size_t(0), base, head);
  return hipGetLastError();
}

hipError_t launch_pack_ternary(const int8_t* codes, int64_t N, int64_t K, void* packed,
                               int32_t* n_invalid, hipStream_t s) {
  const int64_t threads = N * (K / 64);
  hipLaunchKernelGGL(pack_ternary_kernel, dim3(grid_for(threads, 256)), dim3(256), 0, s, codes,
                     N, K, static_cast<uint4*>(packed), n_invalid);
  return hipGetLastError();
}

hipError_t launch_unpack_ternary(const void* packed, int64_t N, int64_t K, int8_t* codes,
                                 int32_t* n_invalid, hipStream_t s) {
  const int64_t threads = N * (K / 64);
  hipLaunchKernelGGL(unpack_ternary_kernel, dim3(grid_for(threads, 256)), dim3(256), 0, s,
                     static_cast<const uint4*>(packed), N, K, codes, n_invalid);
  return hipGetLastError();
}

hipError_t launch_pack_ternary_mf(const int8_t* codes, int64_t N, int64_t K, void* packed,
                                  int32_t* n_invalid, hipStream_t s) {
  const int64_t threads = N * (K / 64);
  hipLaunchKernelGGL(pack_ternary_mf_kernel, dim3(grid_for(threads, 256)), dim3(256), 0, s, codes,
                     N, K, static_cast<uint4*>(packed), n_invalid);
  return hipGetLastError();
}

hipError_t launch_repack_pn_to_mf(const void* pn, int64_t N, int64_t K, void* mf,
                                  int32_t* n_invalid, hipStream_t s) {
  const int64_t threads = N * (K / 64);
  hipLaunchKernelGGL(repack_pn_to_mf_kernel, dim3(grid_for(threads, 256)), dim3(256), 0, s,
                     static_cast<const uint4*>(pn), N, K, static_cast<uint4*>(mf), n_invalid);
  return hipGetLastError();
}

hipError_t launch_pack_sign(const float* W, int64_t N, int64_t K, void* packed, hipStream_t s) {
  const int64_t threads = N * (K / 128);
  hipLaunchKernelGGL(pack_sign_kernel, dim3(grid_for(threads, 256)), dim3(256), 0, s, W, N, K,
                     static_cast<uint4*>(packed));
  return hipGetLastError();
}

hipError_t launch_unpack_sign(const void* packed, int64_t N, int64_t K, int8_t* signs,
                              hipStream_t s) {
  const int64_t threads = N * (K / 128);
  hipLaunchKernelGGL(unpack_sign_kernel, dim3(grid_for(threads, 256)), dim3(256), 0, s,
                     static_cast<const uint4*>(packed), N, K, signs);
  return hipGetLastError();
}

hipError_t launch_ternarize_absmean(const float* W, int64_t N, int64_t K, int8_t* codes,
                                    void* packed, float* beta, unsigned long long* bins,
                                    hipStream_t s) {
  const int64_t total = N * K;
  int64_t want = (total / 4 + 255) / 256;
  const int nblk = static_cast<int>(std::min<int64_t>(std::max<int64_t>(want, 1), kAbsmeanBlocks));
  hipLaunchKernelGGL(absmean_hist_kernel, dim3(nblk), dim3(256), 0, s, W, total, bins);
  hipLaunchKernelGGL(absmean_finalize_kernel, dim3(1), dim3(256), 0, s, bins, nblk,
                     static_cast<uint32_t>(total), beta);
  const int64_t threads = N * (K / 64);
  hipLaunchKernelGGL(ternarize_pack_kernel, dim3(grid_for(threads, 256)), dim3(256), 0, s, W, N,
                     K, beta, codes, static_cast<uint4*>(packed));
  return hipGetLastError();
}

}  // namespace bl
