// Batched / prefill GEMM for ternary weights on int8 matrix cores.
//
// [b158] "实验及结果": b1.58 models serve large batches (Table 3, sequence length 512) and
// the matrix product is an int8 accumulation (Fig. 3). Here the packed T2-PN-64 weights
// are expanded to int8 {-1, 0, +1} tiles in LDS and multiplied with the int8 activations
// by v_mfma_i32_16x16x64_i8 with int32 accumulation, then rescaled in a fused epilogue.
//
// Expansion: for a 32-input word, (X >> j) & 0x01010101 puts the flags of inputs 4j..4j+3
// in bytes 0..3 (the layout's bit order was chosen for this), and
// (P_bytes) + 255 * (N_bytes) turns flags into int8 +1 / -1 bytes (expand_flags).
//
// Batched decode (M <= 64) goes to the weight-streaming kernel of tern_mfma.hip and prefill
// to the register-blocked kernel below. When K is split across workgroups, partial
// accumulators meet in the workspace's split words and the last one applies the epilogue.
#include "bl_internal.h"

namespace bl {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kLd = 64 + 16;   // LDS row pitch in bytes (64 k per tile + pad)

// Per byte: P flag -> 0x01 (+1), N flag -> 0xFF (-1), neither -> 0, i.e. pb + 255 nb. As
// 32-bit arithmetic (pb - nb) + (nb << 8) equals it modulo 2^32 (the borrows cancel), so no
// multiply is needed: one subtraction and one shift-and-add (written out because the
// compiler folds the pair back into a 32-bit multiply).
__device__ __forceinline__ uint32_t expand_flags(uint32_t pb, uint32_t nb) {
  uint32_t o;
  asm("v_lshl_add_u32 %0, %1, 8, %2" : "=v"(o) : "v"(nb), "v"(pb - nb));
  return o;
}

// Register-blocked prefill GEMM. A 256-thread workgroup owns a (4 * 16 FM) x 64 output tile:
// its four waves are stacked along M, each holding a (16 FM) x 64 block of accumulators
// (FM x 4 fragments, 4 FM MFMAs per 64-input k tile). The 64 weight columns (one T2-PN-64
// band) are expanded to int8 once per workgroup and k tile into LDS and read by all four
// waves; the activations go straight from global memory into registers in the MFMA
// operand layout (lane 16g + u: row u of a fragment, inputs 16g .. 16g + 15), so LDS
// carries only the weights: 4 KiB of LDS reads per wave per k tile for 16 FM MFMAs,
// against 1 KiB per MFMA when both operands come from LDS in 32 x 32 wave tiles.
// Raw weight rows and activation fragments are fetched S k tiles ahead into registers,
// weights first (the expansion of tile t + 1 waits for them, and vector loads complete in
// issue order), and every fetch is unconditional with clamped indices.
template <int FM, int S, bool SPLIT>
__global__ __launch_bounds__(256) void gemm_rb_kernel(
    const int8_t* __restrict__ q, const float* __restrict__ gamma, int64_t M, int64_t K,
    const u32x4* __restrict__ W, const float* __restrict__ beta, int64_t beta_len, int64_t N,
    float* __restrict__ y, int32_t* __restrict__ acc_out, uint64_t* __restrict__ ws_acc,
    int tiles_per_split, int MT, int NT) {
  constexpr int WM = 16 * FM;
  constexpr int BM = 4 * WM;
  __shared__ __attribute__((aligned(16))) int8_t Bs[2][64 * kLd];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, u = lane & 15;

  const int nblocks = MT * NT;
  int L = blockIdx.x;
  if ((nblocks & 7) == 0) L = (blockIdx.x & 7) * (nblocks >> 3) + (blockIdx.x >> 3);
  const int mt = L % MT, nt = L / MT;
  const int64_t m0 = static_cast<int64_t>(mt) * BM + wave * WM;
  const int KT = static_cast<int>(K / 64);
  const int t0 = blockIdx.y * tiles_per_split;
  const int t1 = min(KT, t0 + tiles_per_split);

  // activation fragment fm of this lane: row m0 + 16 fm + u (clamped), inputs 16g.. of a tile
  const int8_t* qrow[FM];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
    qrow[fm] = q + min<int64_t>(m0 + 16 * fm + u, M - 1) * K + 16 * g;
  // expansion item of this thread: tile row tid / 4 (column n0 + tid / 4), half hh, quarter qq
  const int brow = tid >> 2, hh = (tid >> 1) & 1, qq = tid & 1;
  const u32x4* wrow = W + static_cast<int64_t>(nt) * KT * 64 + brow;

  u32x4 ra[S][FM];
  u32x4 rb[S];
  auto fetch = [&](int s, int tk) __attribute__((always_inline)) {
    tk = min(tk, t1 - 1);
    rb[s] = wrow[static_cast<int64_t>(tk) * 64];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
      ra[s][fm] = *reinterpret_cast<const u32x4*>(qrow[fm] + static_cast<int64_t>(tk) * 64);
  };
  auto stage = [&](int s, int buf) __attribute__((always_inline)) {
    const uint32_t P = hh ? rb[s].y : rb[s].x, Nm = hh ? rb[s].w : rb[s].z;
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int sh = 4 * qq + j;
      o[j] = expand_flags((P >> sh) & 0x01010101u, (Nm >> sh) & 0x01010101u);
    }
    *reinterpret_cast<u32x4*>(&Bs[buf][brow * kLd + hh * 32 + qq * 16]) = u32x4{o[0], o[1], o[2], o[3]};
  };

  i32x4 acc[FM][4];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = i32x4{0, 0, 0, 0};

  auto compute = [&](int s, int buf) __attribute__((always_inline)) {
    i32x4 b[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      b[j] = *reinterpret_cast<const i32x4*>(&Bs[buf][(16 * j + u) * kLd + 16 * g]);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const i32x4 a = __builtin_bit_cast(i32x4, ra[s][i]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b[j], acc[i][j], 0, 0, 0);
    }
  };

  // tile t (t - t0 = d) sits in register slot d % S and LDS buffer d & 1
#pragma unroll
  for (int s = 0; s < S; ++s) fetch(s, t0 + s);
  stage(0, 0);
  __syncthreads();
  for (int kb = t0; kb < t1; kb += S) {
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int tk = kb + s;
      const int ns = (s + 1) % S;
      if (tk < t1) compute(s, (tk - t0) & 1);
      if (tk + 1 < t1) stage(ns, (tk + 1 - t0) & 1);
      fetch(s, tk + S);   // unconditional (clamped): loads behind a branch cost exact waits
      __syncthreads();
    }
  }

  // D layout of a 16x16 fragment: lane l holds rows 4*(l/16) + r, column l % 16. With K
  // split, each row tile's 16 outputs of a lane meet the other splits in two batches of 8
  // adds in flight.
  const int nsplit = gridDim.y;
  const int64_t n0 = static_cast<int64_t>(nt) * 64;
  if constexpr (!SPLIT) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t row = m0 + 16 * i + 4 * g + r;
          const int64_t col = n0 + 16 * j + u;
          if (row >= M) continue;
          // written once, not read back here: non-temporal stores
          if (acc_out) __builtin_nontemporal_store(acc[i][j][r], &acc_out[row * N + col]);
          if (y)
            __builtin_nontemporal_store(static_cast<float>(acc[i][j][r]) * (gamma[row] / 127.0f) *
                                            beta[beta_len == 1 ? 0 : col],
                                        &y[row * N + col]);
        }
  } else {
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      int32_t v[8];
      uint32_t active = 0;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int j = 2 * half + k / 4, r = k % 4;
        v[k] = acc[i][j][r];
        if (m0 + 16 * i + 4 * g + r < M) active |= 1u << k;
      }
      auto word = [&](int k) __attribute__((always_inline)) {
        const int j = 2 * half + k / 4, r = k % 4;
        return ws_acc + min<int64_t>(m0 + 16 * i + 4 * g + r, M - 1) * N + n0 + 16 * j + u;
      };
      const uint32_t done = split_arrive_batch<8>(word, v, active, nsplit);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if (!((done >> k) & 1u)) continue;
        const int j = 2 * half + k / 4, r = k % 4;
        const int64_t row = m0 + 16 * i + 4 * g + r;
        const int64_t col = n0 + 16 * j + u;
        if (acc_out) acc_out[row * N + col] = v[k];
        if (y) y[row * N + col] = static_cast<float>(v[k]) * (gamma[row] / 127.0f) *
                                  beta[beta_len == 1 ? 0 : col];
      }
    }
  }
}

// Workgroups the register-blocked kernel aims for before it splits K: one per CU.
constexpr int64_t kGemmRbTarget = 256;

template <int FM, int S = 3>
hipError_t launch_rb(const int8_t* q, const float* gamma, int64_t M, int64_t K, const u32x4* W,
                     const float* beta, int64_t beta_len, int64_t N, float* y, int32_t* acc_out,
                     uint64_t* ws_acc, hipStream_t s) {
  constexpr int BM = 64 * FM;
  const int MT = static_cast<int>((M + BM - 1) / BM), NT = static_cast<int>(N / 64);
  const int KT = static_cast<int>(K / 64);
  const int64_t tiles = static_cast<int64_t>(MT) * NT;
  const int64_t target = kGemmRbTarget;
  int nsplit = static_cast<int>(std::min<int64_t>((target + tiles - 1) / tiles, std::max(1, KT / 8)));
  nsplit = std::max(nsplit, 1);
  if (M * N > kAccCap || K > kMaxIntSplitK) nsplit = 1;
  nsplit = std::min(nsplit, kMaxIntSplits);
  const int tps = (KT + nsplit - 1) / nsplit;
  nsplit = (KT + tps - 1) / tps;
  // the split hand-off lives in its own instantiation: its registers would otherwise lower
  // the occupancy of the common unsplit kernel
  if (nsplit > 1)
    hipLaunchKernelGGL((gemm_rb_kernel<FM, S, true>), dim3(static_cast<unsigned>(tiles), nsplit),
                       dim3(256), 0, s, q, gamma, M, K, W, beta, beta_len, N, y, acc_out, ws_acc,
                       tps, MT, NT);
  else
    hipLaunchKernelGGL((gemm_rb_kernel<FM, S, false>), dim3(static_cast<unsigned>(tiles), 1),
                       dim3(256), 0, s, q, gamma, M, K, W, beta, beta_len, N, y, acc_out, ws_acc,
                       tps, MT, NT);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const int8_t* q, const float* gamma, int64_t M, int64_t K,
                       const void* wpacked, const float* beta, int64_t beta_len, int64_t N,
                       float* y, int32_t* acc_out, uint64_t* ws_acc, hipStream_t s) {
  const u32x4* W = static_cast<const u32x4*>(wpacked);
  // Batched decode: weights streamed into registers and expanded there (tern_mfma.hip);
  // measured 1.1-2.2x faster than LDS tiles for M <= 64 on the 70B-shaped linears.
  if (M <= 64) return launch_tern_mfma(q, gamma, M, K, wpacked, beta, beta_len, N, y, acc_out, ws_acc, s);
  // Prefill: 64 x 64 output tiles with the four waves stacked along M, activations straight
  // into registers, weights expanded once per tile into LDS (measured on the 3B shapes at
  // M = 512: 5 % faster over the set than 64 x 64 tiles with both operands in LDS; deeper
  // register tiles, 128 x 64 and 256 x 64, were slower: too few waves per SIMD to hide the
  // per-k-tile latencies).
  return launch_rb<1>(q, gamma, M, K, W, beta, beta_len, N, y, acc_out, ws_acc, s);
}

}  // namespace bl
