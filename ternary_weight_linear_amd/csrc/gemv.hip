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

#include <type_traits>

namespace bl {
namespace {

constexpr int kWaves = 4;
constexpr int kUnroll = 8;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

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
      w[u] = tt < t1 ? __builtin_nontemporal_load(&wp[static_cast<int64_t>(tt) * 64]) : u32x4{0, 0, 0, 0};
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
            A[m][b] = static_cast<int>(bcnt_acc((x0 & w[u].x) | (~x0 & w[u].z), static_cast<uint32_t>(A[m][b])));
            A[m][b] = static_cast<int>(bcnt_acc((x1 & w[u].y) | (~x1 & w[u].w), static_cast<uint32_t>(A[m][b])));
          }
        }
        cn = static_cast<int>(bcnt_acc(w[u].w, bcnt_acc(w[u].z, static_cast<uint32_t>(cn))));
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
// inside the kernel instead of read from X8-64 memory. A workgroup owns kFW consecutive
// 64-row bands (one per wave) and one K range, processed in chunks of up to kChunk tiles:
//  1. loads are issued at once: first this thread's share of the row for gamma and the x
//     values its wave quantises in the first chunk, then the wave's first weight batch, so
//     HBM streaming runs through steps 2-3 (vector loads complete in issue order, so the
//     x-dependent steps never wait for weights); the ring's other batches follow between
//     the tiles of step 3, one per tile;
//  2. gamma: every workgroup reduces |x| over the whole row. For finite fp16 the magnitude
//     order equals the integer order of the bits with the sign cleared, so this is an
//     integer max over masked bit patterns (no conversions); a maximum >= 0x7C00 flags
//     NaN/inf;
//  3. each wave quantises every kFW-th tile of the chunk (lane l takes the input whose plane
//     bit is l; eight wave ballots give the tile's planes) into LDS, then one barrier;
//  4. each wave runs the select + popcount loop over the chunk for its own band with a ring
//     of kRing register batches, each slot refilled with the batch kRing ahead as soon as
//     it is reduced, planes read from LDS as wave-uniform broadcasts.
// Weights are read through a buffer resource that spans the wave's band over the
// workgroup's K range: loads past the range return zero without a memory access, so the
// stream is issued ahead unconditionally (no clamped re-reads at the end of a range).
// The integer results are identical to bl_quant_act_int8 followed by the GEMV.
constexpr int kBatch = 2;                   // tiles per register batch
constexpr int kRing = 8;                    // register batches per wave
constexpr int kChunk = 64;                  // tiles whose planes sit in LDS at once
constexpr int kFW = 4;                      // waves (bands) per workgroup

constexpr int kPerWave = kChunk / kFW;      // tiles each wave quantises per chunk
constexpr int kMinSplitTiles = 4;           // a K split of the fused kernel spans >= 4 tiles
// Ring shape and issue order, measured on MI355X (70B-shaped decode pass at M = 1, A/B runs
// of the whole pass on one box): with four 4-tile batches, all of them before gamma 4.82 ms,
// one per quantised tile 4.34 ms, one per 2 / 3 / 4 tiles 4.30 / 4.29 / 4.33 ms, none before
// gamma 4.40 ms (weight requests issued sooner queue ahead of the x reads that gamma and the
// quantiser wait on); eight 2-tile batches, one before gamma and one per quantised tile, 4.24
// against 4.28 ms for the best 4 x 4 order (finer batches: the loop waits for two tiles at a
// time, and the ring is refilled in smaller steps); eight 4-tile batches 4.84 ms, sixteen
// 1-tile ones 4.38 ms; of the eight 2-tile batches, one / two / three before gamma (then one
// per quantised tile) 4.28 / 4.25 / 4.34 ms, two before gamma and two per tile 4.33 ms.
constexpr int kPreGamma = 2;        // ring batches issued before gamma; then one per tile
static_assert(kChunk % (kRing * kBatch) == 0, "a chunk holds whole ring turns");
constexpr int kRsrcWord3 = 0x00020000;      // raw buffer resource, 32-bit elements
// Weights are read once per pass: non-temporal loads (the nt cache policy) keep them from
// displacing what is reused (x, the split words, outputs). Measured on MI355X, 70B-shaped
// decode pass at M = 1: 4.64 -> 4.43 ms (the sc0 and sc1 bits changed nothing).
constexpr int kLoadNT = 2;


template <int MR, int GL>
__global__ __launch_bounds__(64 * kFW) void gemv_fused_kernel(
    const uint16_t* __restrict__ x, int64_t K, const u32x4* __restrict__ W,
    const float* __restrict__ beta, int64_t beta_len, int64_t N, float* __restrict__ y,
    uint64_t* __restrict__ ws_acc, uint32_t* __restrict__ ws_cnt, int tiles_per_split) {
  __shared__ __attribute__((aligned(16))) uint32_t pl[kChunk][MR][16];
  __shared__ uint32_t red_max[kFW][MR];
  const int64_t nbands = N / 64;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t band = static_cast<int64_t>(blockIdx.x) * kFW + wave;
  const bool active = band < nbands;
  const int split = blockIdx.y;
  const int nsplit = gridDim.y;
  const int KT = static_cast<int>(K / 64);
  const int t0 = split * tiles_per_split;
  const int t1 = min(KT, t0 + tiles_per_split);
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<u32x4*>(W + ((active ? band : 0) * KT + t0) * 64), 0,
      active && t1 > t0 ? (t1 - t0) * 1024 : 0, kRsrcWord3);
  // lane l <-> plane bit l of a tile: half h = l / 32, bit p = l % 32 = 8i + j <-> c = 4j + i
  const int koff = 32 * (lane >> 5) + 4 * (lane & 7) + ((lane & 31) >> 3);

  // All loads below are unconditional (x indices past the range are clamped, weight tiles
  // past it read as zero): branch-free code lets the compiler wait for exactly the loads a
  // step needs instead of for every load in flight.
  u32x4 w[kRing][kBatch];
  auto load_batch = [&](u32x4 (&dst)[kBatch], int rel) {   // tiles t0 + rel .. + kBatch - 1
#pragma unroll
    for (int u = 0; u < kBatch; ++u)   // streamed once: non-temporal (aux bit 1, nt)
      dst[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                             wr, (rel + u) * 1024 + lane * 16, 0, kLoadNT));
    // keep each batch where it is issued: the scheduler would otherwise interleave or sink
    // batches, and the waits for one batch would then cover the next as well
    __builtin_amdgcn_sched_barrier(0);
  };
  auto load_x = [&](uint16_t (&xq)[kPerWave][MR], int c0, int c1) {
#pragma unroll
    for (int j = 0; j < kPerWave; ++j) {
      const int tt = min(c0 + wave + kFW * j, c1 - 1);
#pragma unroll
      for (int m = 0; m < MR; ++m) xq[j][m] = x[m * K + 64 * tt + koff];
    }
  };
  // Vector loads complete in issue order, so everything that waits only on x is issued
  // before the weights: this thread's share of the row for gamma (GL loads per row when
  // GL > 0, i.e. K <= 2048 GL) and the x values it quantises in the first chunk.
  const u32x4* const row4 = reinterpret_cast<const u32x4*>(x);
  const int64_t K8 = K / 8;
  u32x4 gx[MR][GL > 0 ? GL : 1];
  if constexpr (GL > 0) {
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      // row m through a buffer resource of its own: loads past the row read zero, which
      // leaves the maximum unchanged, and the offset needs no clamp
      const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(x + static_cast<int64_t>(m) * K), 0, static_cast<int>(K * 2),
          kRsrcWord3);
#pragma unroll
      for (int i = 0; i < GL; ++i)
        gx[m][i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 xr, (threadIdx.x + 64 * kFW * i) * 16, 0, 0));
    }
  }
  uint16_t xq[kPerWave][MR];
  load_x(xq, t0, min(t1, t0 + kChunk));
  // the first kPreGamma batches; the rest of the ring is issued between the quantised tiles: a
  // wave issues its loads in order, and the vector memory path takes ~16 cycles per 1 KiB
  // load, so issuing them here would hold the gamma fold back
#pragma unroll
  for (int r = 0; r < kPreGamma; ++r) load_batch(w[r], r * kBatch);

  // gamma_m = max |x_m| over the whole row (NaN if the row holds NaN/inf)
  float g[MR], rg[MR];
  bool zero[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    // both halves at once (packed 16-bit max), then the wave maximum through DPP
    u16x2 m2 = {0, 0};
    auto fold = [&](const u32x4& v) {
      const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j)
        m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2, w4[j] & 0x7FFF7FFFu));
    };
    if constexpr (GL > 0) {
#pragma unroll
      for (int i = 0; i < GL; ++i) fold(gx[m][i]);
    } else {
#pragma unroll 4
      for (int64_t i = threadIdx.x; i < K8; i += 64 * kFW) fold(row4[m * K8 + i]);
    }
    const uint32_t mb = wave_max_u32(max(static_cast<uint32_t>(m2.x), static_cast<uint32_t>(m2.y)));
    if (lane == 0) red_max[wave][m] = mb;
  }
  __syncthreads();
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    uint32_t mb = red_max[0][m];
#pragma unroll
    for (int w2 = 1; w2 < kFW; ++w2) mb = max(mb, red_max[w2][m]);
    const bool bad = mb >= 0x7C00u;
    g[m] = bad ? __uint_as_float(0x7FC00000u) : half_bits_to_float(static_cast<uint16_t>(mb));
    zero[m] = bad || mb == 0u;
    rg[m] = __builtin_amdgcn_rcpf(zero[m] ? 1.0f : g[m]);
  }

  int A[MR][8];
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int b = 0; b < 8; ++b) A[m][b] = 0;
  int cn = 0;

  // quantise tiles c0 + wave + kFW j of a chunk into LDS; in the first chunk, the ring's
  // remaining batches are issued between the tiles
  auto quantise = [&](int c0, int c1, auto first) {
#pragma unroll
    for (int j = 0; j < kPerWave; ++j) {
      if constexpr (decltype(first)::value) {
        if (j + kPreGamma < kRing) load_batch(w[j + kPreGamma], (j + kPreGamma) * kBatch);
      }
      const int tt = c0 + wave + kFW * j;
      if (tt < c1) {
#pragma unroll
        for (int m = 0; m < MR; ++m) {
          const int qv = zero[m] ? 0 : quant_q(half_bits_to_float(xq[j][m]) * 127.0f, g[m], rg[m]);
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
  };
  static_assert(kRing - kPreGamma <= kPerWave, "the ring is issued within the first chunk");
  for (int c0 = t0; c0 < t1; c0 += kChunk) {
    const int c1 = min(t1, c0 + kChunk);
    if (c0 == t0) {
      quantise(c0, c1, std::true_type{});
    } else {
      __syncthreads();                    // the previous chunk's planes are consumed
      load_x(xq, c0, c1);                 // (this chunk's first batches are already in flight)
      quantise(c0, c1, std::false_type{});
    }
    __syncthreads();
    if (active) {
      // batch i of the range sits in ring slot i % kRing; once reduced, the slot is refilled
      // with batch i + kRing (unconditionally: past the range it reads zero for free)
      for (int tb = c0; tb < c1; tb += kRing * kBatch) {
#pragma unroll
        for (int r = 0; r < kRing; ++r) {
          const int tr = tb + r * kBatch;
          if (tr < c1) {
            // every tile of the batch unconditionally (tiles past the range hold zero weights
            // and add nothing; their plane index is clamped into the array), so the scheduler
            // can read the next tile's planes while this one is reduced
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
              {
                const u32x4 wc = w[r][u];
                const int pt = min(tr + u - c0, kChunk - 1);
#pragma unroll
                for (int m = 0; m < MR; ++m) {
                  const u32x4* X4 = reinterpret_cast<const u32x4*>(&pl[pt][m][0]);
                  const u32x4 p0 = X4[0], p1 = X4[1], p2 = X4[2], p3 = X4[3];
                  const uint32_t X[16] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w,
                                          p2.x, p2.y, p2.z, p2.w, p3.x, p3.y, p3.z, p3.w};
#pragma unroll
                  for (int b = 0; b < 8; ++b) {
                    const uint32_t x0 = X[2 * b], x1 = X[2 * b + 1];
                    A[m][b] = static_cast<int>(bcnt_acc((x0 & wc.x) | (~x0 & wc.z), static_cast<uint32_t>(A[m][b])));
                    A[m][b] = static_cast<int>(bcnt_acc((x1 & wc.y) | (~x1 & wc.w), static_cast<uint32_t>(A[m][b])));
                  }
                }
                cn = static_cast<int>(bcnt_acc(wc.w, bcnt_acc(wc.z, static_cast<uint32_t>(cn))));
              }
            }
          }
          load_batch(w[r], tr - t0 + kRing * kBatch);
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

struct GemvFusedPlan { int64_t groups, nsplit, tps; };

GemvFusedPlan plan_gemv_fused(int M, int64_t N, int64_t K) {
  const int64_t bands = N / 64;
  const int64_t groups = (bands + kFW - 1) / kFW;
  const int64_t KT = K / 64;
  // measured on MI355X: narrow outputs do best with fewer, longer workgroups (every
  // workgroup reads the whole row for gamma), wide ones with more
  const int64_t target = bands < 512 ? 256 : 512;
  int64_t nsplit = target / groups;   // never above the target: a partial extra wave of
                                      // workgroups would run after all the others
  nsplit = std::min<int64_t>(nsplit, std::max<int64_t>(1, KT / kMinSplitTiles));
  nsplit = std::max<int64_t>(nsplit, 1);
  if (static_cast<int64_t>(M) * N > kAccCap || K > kMaxIntSplitK) nsplit = 1;
  nsplit = std::min<int64_t>(nsplit, kMaxIntSplits);
  const int64_t tps = (KT + nsplit - 1) / nsplit;
  return {groups, (KT + tps - 1) / tps, tps};
}

struct GemvPlan { int64_t nsplit, tps; };

GemvPlan plan_gemv(int M, int64_t N, int64_t K) {
  const int64_t bands = N / 64;
  const int64_t KT = K / 64;
  // Split K so the launch has about `target` workgroups (measured on MI355X: ~512 suit
  // narrow outputs, ~1024 wide ones), keeping at least 8 tiles (2 per wave) per workgroup.
  const int64_t target = bands < 256 ? 512 : 1024;
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
#define BL_GEMVF_LAUNCH(MR_, GL_)                                                            \
  hipLaunchKernelGGL((gemv_fused_kernel<MR_, GL_>), grid, dim3(64 * kFW), 0, s, x, K, W, beta, \
                     beta_len, N, y, ws_acc, ws_cnt, static_cast<int>(p.tps))
  // gamma loads unrolled per thread: K <= 512 kFW GL (row loads in registers); longer rows loop
  const int64_t gl = (K / 8 + 64 * kFW - 1) / (64 * kFW);
  switch (M) {
    case 1:
      if (gl <= 2) BL_GEMVF_LAUNCH(1, 2);
      else if (gl <= 4) BL_GEMVF_LAUNCH(1, 4);
      else if (gl <= 8) BL_GEMVF_LAUNCH(1, 8);
      else BL_GEMVF_LAUNCH(1, 16);   // the entry point takes K <= 28672: gl <= 14
      break;
    case 2:
      if (gl <= 2) BL_GEMVF_LAUNCH(2, 2);
      else if (gl <= 4) BL_GEMVF_LAUNCH(2, 4);
      else if (gl <= 8) BL_GEMVF_LAUNCH(2, 8);
      else BL_GEMVF_LAUNCH(2, 0);
      break;
    case 3: BL_GEMVF_LAUNCH(3, 0); break;
    case 4: BL_GEMVF_LAUNCH(4, 0); break;
    default: return hipErrorInvalidValue;
  }
#undef BL_GEMVF_LAUNCH
  return hipGetLastError();
}

}  // namespace bl
