// Ternary GEMM on int8 matrix cores with weights streamed straight into registers.
//
// [b158] "实验及结果": b1.58 models serve batches (Table 3, sequence length 512) and the
// matrix product is an int8 accumulation (Fig. 3). acc[m, n] = sum_k q[m, k] w[n, k] with
// q the int8 activations and w in {-1, 0, +1} from T2-PN-64, multiplied exactly by
// v_mfma_i32_16x16x64_i8 (A = 16 rows of q, B = 16 weight rows expanded to int8).
//
// Expansion in registers: lane 16g + u needs, for weight row r = 16f + u of a 64-input tile,
// the int8 values of inputs 16g .. 16g + 15. They sit in half h = g / 2 of the row's
// T2-PN-64 words (P_h, N_h) at bit positions 8i + j with
// j = 4(g % 2) .. 4(g % 2) + 3, so ((P_h >> j) & 0x01010101) gives the +1 flags of inputs
// 4j .. 4j + 3 as bytes. Either flags_p + 255 flags_n (tern_expand) turns each word into
// four int8 values for one MFMA, or the +1 and -1 flag bytes go to two MFMAs whose results
// are subtracted.
//
// Mapping (the weight-streaming counterpart of the LDS-tiled GEMM, used for batched decode,
// M <= 64, where the weights dominate the bytes): a workgroup of four waves owns one
// 64-column band, FM 16-row tiles of q and a range of 64-input tiles. The waves take the
// range's tiles in turn (wave w: tiles w, w + 4, ...) with kTernDepth - 1 tiles of loads in
// flight (weights and q of a tile issued together, unconditionally: loads past a range are
// clamped into it and never used), and meet in LDS with exact int32 sums. K splits across
// workgroups meet in the 64-bit split words of the workspace (split_arrive), also exact.
#include <algorithm>

#include "bl_internal.h"

namespace bl {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kTernDepth = 2;   // tile sets per wave (depth - 1 in flight)

__device__ __forceinline__ uint32_t tern_expand(uint32_t pb, uint32_t nb) {
  // pb + 255 nb per byte as (pb - nb) + (nb << 8) (exact modulo 2^32: the borrows cancel);
  // written out because the compiler folds the pair back into a 32-bit multiply
  uint32_t o;
  asm("v_lshl_add_u32 %0, %1, 8, %2" : "=v"(o) : "v"(nb), "v"(pb - nb));
  return o;
}

template <int FM>
struct TernTile {
  u32x4 w[4];            // T2-PN-64 row 16f + u of the tile: P0, P1, N0, N1; f = 0..3
  u32x4 a[FM];           // q[m0 + 16fm + u, 64t + 16g .. +15]
};

struct TernArgs {
  const int8_t* q;           // int8 [M, K]
  const float* gamma;        // fp32 [M]
  const u32x4* W;            // T2-PN-64 [N, K]
  const float* beta;
  int64_t beta_len, M, N, K;
  float* y;                  // fp32 [M, N] (may be null)
  int32_t* acc_out;          // int32 [M, N] (may be null)
  uint64_t* ws_acc;          // split words [M, N] (nsplit > 1)
  int tiles_per_split;
};

template <int FM>
__device__ __forceinline__ void tern_load(TernTile<FM>& T, const TernArgs& a, int64_t band,
                                          const uint32_t (&qoff)[FM], uint32_t woff, int t,
                                          int KT) {
  // woff = 16 u: row u of the tile (one 16-byte load per fragment; fewer, wider loads
  // beat loading only the two words a lane uses)
  const char* wt = reinterpret_cast<const char*>(a.W) + ((band * KT + t) << 10);
#pragma unroll
  for (int f = 0; f < 4; ++f) T.w[f] = *reinterpret_cast<const u32x4*>(wt + 256 * f + woff);
  const char* qt = reinterpret_cast<const char*>(a.q) + static_cast<int64_t>(t) * 64;
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) T.a[fm] = *reinterpret_cast<const u32x4*>(qt + qoff[fm]);
}

// Epilogue shared by both kernels (wave 0, after the LDS reduction): per 16-row tile fm,
// the 16 outputs of this lane meet the other K splits with all 16 adds in flight at once
// (split_arrive_batch; one round trip measured faster here than two batches of 8 with
// fewer registers), and y / acc are written. T2-MF64 (rowsum given): fragment f's sums are
// shifted right by 2f first, and rowsum is taken away from fragments f < 3.
// D layout: lane l holds rows 4*(l/16) + i of the q tile, column l % 16 of fragment f.
template <int FM>
__device__ __forceinline__ void tern_epilogue(const TernArgs& a, const i32x4 (&acc)[FM][4],
                                              const int (&red)[3][FM * 16][64], int lane,
                                              int64_t band, int64_t m0, int nsplit,
                                              const int32_t* rowsum) {
  const int g = lane >> 4, u = lane & 15;
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    // output k = 4 f + i: row m0 + 16 fm + 4g + i, column band * 64 + 16 f + u
    int32_t v[16];
    uint32_t active = 0;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int f = k / 4, i = k % 4, e = (fm * 4 + f) * 4 + i;
      v[k] = acc[fm][f][i] + red[0][e][lane] + red[1][e][lane] + red[2][e][lane];
      if (rowsum) v[k] >>= 2 * f;   // exact: a multiple of 4^f
      if (m0 + 16 * fm + 4 * g + i < a.M) active |= 1u << k;
    }
    auto word = [&](int k) __attribute__((always_inline)) {
      const int64_t row = min<int64_t>(m0 + 16 * fm + 4 * g + k % 4, a.M - 1);
      return a.ws_acc + row * a.N + band * 64 + 16 * (k / 4) + u;
    };
    const uint32_t done = nsplit > 1 ? split_arrive_batch<16>(word, v, active, nsplit) : active;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      if (!((done >> k) & 1u)) continue;
      const int64_t row = m0 + 16 * fm + 4 * g + k % 4;
      const int64_t col = band * 64 + 16 * (k / 4) + u;
      int r = v[k];
      if (rowsum && k / 4 < 3) r -= rowsum[row];
      if (a.acc_out) a.acc_out[row * a.N + col] = r;
      if (a.y)
        a.y[row * a.N + col] = static_cast<float>(r) * (a.gamma[row] / 127.0f) *
                               a.beta[a.beta_len == 1 ? 0 : col];
    }
  }
}

// SPLIT: multiply the +1 flags and the -1 flags separately (two MFMAs, acc = accP - accN,
// four VALU ops per 16 weights); otherwise expand to int8 first (one MFMA, six VALU ops).
// The first suits few rows of q (VALU-bound), the second many (matrix-core-bound).
template <int FM, bool SPLIT>
__device__ __forceinline__ void tern_compute(const TernTile<FM>& T, i32x4 (&acc)[FM][4],
                                             i32x4 (&accn)[SPLIT ? FM : 1][4], const int (&js)[4],
                                             bool hi) {
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const uint32_t Pw = hi ? T.w[f].y : T.w[f].x, Nw = hi ? T.w[f].w : T.w[f].z;
    i32x4 bp, bn;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const uint32_t pb = (Pw >> js[jj]) & 0x01010101u, nb = (Nw >> js[jj]) & 0x01010101u;
      if constexpr (SPLIT) {
        bp[jj] = static_cast<int>(pb);
        bn[jj] = static_cast<int>(nb);
      } else {
        bp[jj] = static_cast<int>(tern_expand(pb, nb));
      }
    }
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      const i32x4 av = __builtin_bit_cast(i32x4, T.a[fm]);
      acc[fm][f] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, bp, acc[fm][f], 0, 0, 0);
      if constexpr (SPLIT)
        accn[fm][f] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, bn, accn[fm][f], 0, 0, 0);
    }
  }
}

template <int FM, bool SPLIT>
__global__ __launch_bounds__(256) void tern_mfma_kernel(const TernArgs a) {
  constexpr int P = kTernDepth;
  constexpr int kRows = 16 * FM;
  __shared__ int red[3][FM * 16][64];                   // waves 1..3, (fm, f, i), lane
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, u = lane & 15;
  const int64_t band = blockIdx.x;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * kRows;
  const int split = blockIdx.z, nsplit = gridDim.z;
  const int KT = static_cast<int>(a.K / 64);
  const int t0 = split * a.tiles_per_split;
  const int t1 = min(KT, t0 + a.tiles_per_split);
  // q rows past M are clamped to row M - 1: they only reach outputs that are never stored
  uint32_t qoff[FM];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    const int64_t row = min<int64_t>(m0 + 16 * fm + u, a.M - 1);
    qoff[fm] = static_cast<uint32_t>(row * a.K + 16 * g);   // M*K < 2^31 (checked on the host)
  }
  const uint32_t woff = 16u * u;
  const bool hi = g >= 2;                               // half h = g / 2 of the row
  int js[4];                                            // bit offsets 4(g % 2) + jj
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) js[jj] = 4 * (g & 1) + jj;

  i32x4 acc[FM][4], accn[SPLIT ? FM : 1][4];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int f = 0; f < 4; ++f) acc[fm][f] = i32x4{0, 0, 0, 0};
#pragma unroll
  for (int fm = 0; fm < (SPLIT ? FM : 1); ++fm)
#pragma unroll
    for (int f = 0; f < 4; ++f) accn[fm][f] = i32x4{0, 0, 0, 0};

  // this wave's tiles: j = 0..n-1 at first + 4j; loads past the end are clamped to the last
  const int first = t0 + wave;
  const int n = first < t1 ? (t1 - first + 3) / 4 : 0;
  const int last = n > 0 ? first + 4 * (n - 1) : t1 - 1;
  TernTile<FM> T[P];
#pragma unroll
  for (int d = 0; d < P - 1; ++d) tern_load<FM>(T[d], a, band, qoff, woff, min(first + 4 * d, last), KT);
  for (int j0 = 0; j0 < n; j0 += P) {
#pragma unroll
    for (int d = 0; d < P; ++d) {
      const int j = j0 + d;
      tern_load<FM>(T[(d + P - 1) % P], a, band, qoff, woff, min(first + 4 * (j + P - 1), last), KT);
      // keep the loads where they are: the scheduler would otherwise sink them towards
      // their use and the tiles in flight would collapse to one
      __builtin_amdgcn_sched_barrier(0);
      if (j < n) tern_compute<FM, SPLIT>(T[d], acc, accn, js, hi);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if constexpr (SPLIT) {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int f = 0; f < 4; ++f) acc[fm][f] -= accn[fm][f];
  }

  // waves 1..3 hand their sums to wave 0 through LDS (exact int32)
  if (wave > 0) {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wave - 1][(fm * 4 + f) * 4 + i][lane] = acc[fm][f][i];
  }
  __syncthreads();
  if (wave > 0) return;
  tern_epilogue<FM>(a, acc, red, lane, band, m0, nsplit, nullptr);
}

// ---- T2-MF64 weights -------------------------------------------------------------------
// The second ternary layout stores, for each lane 16g + u of a wave, the 16 bytes its four
// fragments need: word j holds, at bits 8i + 2f, the field of weight row 16f + u, input
// 16g + 4j + i (w + 1 for f < 3, w in two's complement for f = 3). So a tile costs one
// 16-byte load per lane (no lane loads bytes another lane also loads) and fragment f's
// operand dword j is one AND, word j & (0x03030303 << 2f): bytes 4^f (w + 1) for f < 3 and,
// as signed bytes, 64 w for f = 3 (four ALU ops per fragment). One MFMA per fragment then
// accumulates 4^f sum q (w + 1), resp. 64 sum q w; shifting right by 2f is exact, and for
// f < 3 the final writer takes away sum_k q[m, k] (from the quantiser), which makes the
// integers those of q . w exactly. A split's shifted partial |sum q (w + 1)| <= 254 * 64 *
// tiles stays below the split words' 2^23 bias as long as a split spans at most
// kMfMaxSplitTiles tiles; unshifted, 16 * 254 * K and 64 * 127 * K stay below 2^31 for
// K <= 65536.
constexpr int kMfDepth = 3;
constexpr int kMfMaxSplitTiles = ((1 << 23) - 1) / (254 * 64);   // 516

template <int FM>
struct MfTile {
  u32x4 w;               // record 16g + u of the tile: words f = 0..3
  u32x4 a[FM];           // q[m0 + 16fm + u, 64t + 16g .. +15]
};

template <int FM>
__device__ __forceinline__ void mf_load(MfTile<FM>& T, const TernArgs& a, int64_t band,
                                        const uint32_t (&qoff)[FM], int lane, int t, int KT) {
  T.w = a.W[(band * KT + t) * 64 + lane];
  const char* qt = reinterpret_cast<const char*>(a.q) + static_cast<int64_t>(t) * 64;
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) T.a[fm] = *reinterpret_cast<const u32x4*>(qt + qoff[fm]);
}

template <int FM>
__device__ __forceinline__ void mf_compute(const MfTile<FM>& T, i32x4 (&acc)[FM][4]) {
  const uint32_t w4[4] = {T.w.x, T.w.y, T.w.z, T.w.w};
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    i32x4 b;
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = static_cast<int>(w4[j] & (0x03030303u << (2 * f)));
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
      acc[fm][f] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, T.a[fm]), b,
                                                         acc[fm][f], 0, 0, 0);
  }
}

// Same mapping as tern_mfma_kernel: a workgroup owns one 64-column band, FM 16-row tiles of
// q and a K range whose tiles its four waves take in turn (kMfDepth - 1 in flight, loads
// clamped and unconditional), meeting in LDS with exact int32 sums.
template <int FM>
__global__ __launch_bounds__(256) void tern_mf_kernel(const TernArgs a,
                                                      const int32_t* __restrict__ rowsum) {
  constexpr int P = kMfDepth;
  constexpr int kRows = 16 * FM;
  __shared__ int red[3][FM * 16][64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, u = lane & 15;
  const int64_t band = blockIdx.x;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * kRows;
  const int split = blockIdx.z, nsplit = gridDim.z;
  const int KT = static_cast<int>(a.K / 64);
  const int t0 = split * a.tiles_per_split;
  const int t1 = min(KT, t0 + a.tiles_per_split);
  uint32_t qoff[FM];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    const int64_t row = min<int64_t>(m0 + 16 * fm + u, a.M - 1);
    qoff[fm] = static_cast<uint32_t>(row * a.K + 16 * g);   // M*K < 2^31 (checked on the host)
  }
  i32x4 acc[FM][4];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int f = 0; f < 4; ++f) acc[fm][f] = i32x4{0, 0, 0, 0};

  const int first = t0 + wave;
  const int n = first < t1 ? (t1 - first + 3) / 4 : 0;
  const int last = n > 0 ? first + 4 * (n - 1) : t1 - 1;
  MfTile<FM> T[P];
#pragma unroll
  for (int d = 0; d < P - 1; ++d) mf_load<FM>(T[d], a, band, qoff, lane, min(first + 4 * d, last), KT);
  for (int j0 = 0; j0 < n; j0 += P) {
#pragma unroll
    for (int d = 0; d < P; ++d) {
      const int j = j0 + d;
      mf_load<FM>(T[(d + P - 1) % P], a, band, qoff, lane, min(first + 4 * (j + P - 1), last), KT);
      __builtin_amdgcn_sched_barrier(0);
      if (j < n) mf_compute<FM>(T[d], acc);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  if (wave > 0) {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wave - 1][(fm * 4 + f) * 4 + i][lane] = acc[fm][f][i];
  }
  __syncthreads();
  if (wave > 0) return;
  tern_epilogue<FM>(a, acc, red, lane, band, m0, nsplit, rowsum);
}

// ---- T2-MF64 with q staged in LDS (batched decode, prefill) -----------------------------
// A workgroup of four waves owns four consecutive bands (one per wave), 16 FM rows of q
// (FM = 1, 2 or 3; more rows take more workgroups) and a K range. For each chunk of kQC tiles the
// workgroup copies q[rows, chunk] into LDS once; each wave decodes its own weight tile once
// (16 ALU ops) and runs FM x 4 MFMAs with A fragments read from LDS, so neither the q bytes
// nor the decoding are repeated per 16 rows. Weights come through a buffer resource over
// the wave's band and K range: past the range a load returns zero without a memory access,
// and a zero code adds nothing to sum q (w + 1), so the ring of R chunks is refilled
// unconditionally as soon as a slot is consumed. A chunk's q is loaded into registers
// together with its weights (R chunks ahead) and stored to LDS the step before its use:
// vector loads complete in issue order, so loading it later would make the store wait for
// the whole ring. Staged rows are kQC * 64 + 16 bytes apart: the copy and the fragment
// reads are both free of LDS bank conflicts.
constexpr int kQC = 4;                     // tiles per q chunk and per weight batch
constexpr int kQPitch = kQC * 64 + 16;     // bytes per staged row of q
constexpr int kStRow = 68;                 // ints per staged result row (64 + 4)
constexpr int kQRing = 4;                  // chunks in flight per wave (16- and 32-row tiles)
constexpr int kQRing3 = 2;                 // 48-row tiles: two, so that three waves fit per SIMD
constexpr int kRsrcWord3 = 0x00020000;     // raw buffer resource, 32-bit elements

// 48-row tiles are held to 168 VGPRs (three workgroups per CU instead of two): a 3B-shaped
// prefill then runs its work items in one round instead of one and a half.
// BW = 2 or 1: a work item is BW bands, and each band's K range is split in 4 / BW parts taken
// by as many waves (wave w + BW p takes part p of band w, with its own q chunks in LDS); the
// parts' sums meet in LDS in part order. 4 / BW times the work items of BW = 4 without split
// words, for row tiles that would otherwise split K across workgroups.
template <int FM, int BW>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(FM == 3 ? 3 : 1)))
void tern_mfq_kernel(const TernArgs a, const int32_t* __restrict__ rowsum) {
  constexpr int kRows = 16 * FM;
  constexpr int R = FM == 3 ? kQRing3 : kQRing;
  constexpr int KS = 4 / BW;                       // K halves per band
  constexpr int kHT = 256 / KS;                    // threads per half
  constexpr int kSegs = kRows * kQC * 4 / kHT;     // 16-byte pieces of q per thread per chunk
  static_assert(BW == 4 || BW == 2 || BW == 1, "four bands, or fewer with K in 4 / BW parts");
  static_assert(kSegs >= 1 && (kRows * kQC * 4) % kHT == 0, "q chunk copy");
  constexpr int kQBuf = kRows * kQPitch;           // one staged chunk of q
  constexpr int kStBytes = 4 * 16 * kStRow * 4;    // result rows of the epilogue
  constexpr int kRedBytes = (KS - 1) * BW * FM * 16 * 64 * 4;   // the other parts' sums
  constexpr int kLds = 2 * KS * kQBuf > kStBytes + kRedBytes ? 2 * KS * kQBuf : kStBytes + kRedBytes;
  __shared__ __attribute__((aligned(16))) int8_t lds[kLds];   // q chunks, then results
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane((tid >> 6) % BW);   // band within the item
  const int half = KS > 1 ? __builtin_amdgcn_readfirstlane(tid / kHT) : 0;
  const int htid = tid % kHT;                                        // thread within the half
  auto qs = [&](int buf) __attribute__((always_inline)) { return lds + (half * 2 + buf) * kQBuf; };
  const int g = lane >> 4, u = lane & 15;
  const int64_t bands = a.N / 64;
  const int KT = static_cast<int>(a.K / 64);
  // Work item of this workgroup. Dispatch ids are dealt round-robin over the 8 XCDs (id i
  // runs on XCD i % 8); each XCD takes a contiguous range of work items, ordered split,
  // band group, row group (fastest), so the row groups of a band group run side by side on
  // one XCD and read its weights through that XCD's L2 once instead of once per row group.
  const int groups = static_cast<int>((bands + BW - 1) / BW);
  const int mgroups = static_cast<int>((a.M + kRows - 1) / kRows);
  const int nsplit = (KT + a.tiles_per_split - 1) / a.tiles_per_split;
  const int nwork = groups * mgroups * nsplit;
  const int per_xcd = (nwork + 7) / 8;
  const int wk = static_cast<int>(blockIdx.x & 7) * per_xcd + static_cast<int>(blockIdx.x >> 3);
  if (wk >= nwork) return;   // the grid is rounded up to 8 per_xcd
  const int mg = wk % mgroups;
  const int grp = (wk / mgroups) % groups;
  const int split = wk / (mgroups * groups);
  const int64_t band = static_cast<int64_t>(grp) * BW + wave;
  const bool active = band < bands;
  const int64_t m0 = static_cast<int64_t>(mg) * kRows;
  const int s0 = split * a.tiles_per_split;
  const int s1 = min(KT, s0 + a.tiles_per_split);
  // this half's chunks: [half * nchh, (half + 1) * nchh) of the item's; both halves run nchh
  // steps in lockstep (a half with fewer chunks multiplies zero weights)
  const int nchh = ((s1 - s0 + kQC - 1) / kQC + KS - 1) / KS;
  const int t0 = min(s1, s0 + half * nchh * kQC);
  const int t1 = min(s1, t0 + nchh * kQC);
  const int nch = (t1 - t0 + kQC - 1) / kQC;

  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<u32x4*>(a.W + ((active ? band : 0) * KT + t0) * 64), 0,
      active ? (t1 - t0) * 1024 : 0, kRsrcWord3);
  u32x4 w[R][kQC];
  auto load_w = [&](u32x4 (&dst)[kQC], int chunk) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < kQC; ++t)
      dst[t] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                             wr, (chunk * kQC + t) * 1024 + lane * 16, 0, 0));
    __builtin_amdgcn_sched_barrier(0);   // keep each batch where it is issued
  };
  // q piece s = htid + kHT i of a chunk: row s / (4 kQC), tile (s / 4) % kQC, 16 bytes s % 4.
  // Rows past M and tiles past K are clamped into q (their products are never stored or
  // meet zero weights).
  u32x4 qr[R][kSegs];
  auto load_q = [&](u32x4 (&dst)[kSegs], int chunk) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kSegs; ++i) {
      const int sg = htid + kHT * i;
      const int64_t row = min<int64_t>(m0 + sg / (4 * kQC), a.M - 1);
      const int tile = min(t0 + chunk * kQC + (sg / 4) % kQC, KT - 1);
      dst[i] = *reinterpret_cast<const u32x4*>(a.q + row * a.K + tile * 64 + (sg % 4) * 16);
    }
  };
  auto store_q = [&](const u32x4 (&src)[kSegs], int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kSegs; ++i) {
      const int sg = htid + kHT * i;
      *reinterpret_cast<u32x4*>(qs(buf) + (sg / (4 * kQC)) * kQPitch + ((sg / 4) % kQC) * 64 +
                                (sg % 4) * 16) = src[i];
    }
  };

  i32x4 acc[FM][4];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int f = 0; f < 4; ++f) acc[fm][f] = i32x4{0, 0, 0, 0};
  // The A fragments of tile t + 1 are read from LDS while tile t's products run (read just
  // before use, every fragment's LDS latency sat in front of its MFMAs; measured on MI355X,
  // 3B-shaped prefill: down 908 -> 1040 TOPS, the set 1153 -> 1197).
  auto compute = [&](const u32x4 (&wb)[kQC], int buf) __attribute__((always_inline)) {
    i32x4 avb[2][FM];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
      avb[0][fm] = *reinterpret_cast<const i32x4*>(qs(buf) + (16 * fm + u) * kQPitch + g * 16);
#pragma unroll
    for (int t = 0; t < kQC; ++t) {
      if (t + 1 < kQC) {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
          avb[(t + 1) & 1][fm] = *reinterpret_cast<const i32x4*>(
              qs(buf) + (16 * fm + u) * kQPitch + (t + 1) * 64 + g * 16);
      }
      const uint32_t w4[4] = {wb[t].x, wb[t].y, wb[t].z, wb[t].w};
      i32x4 b[4];
#pragma unroll
      for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int j = 0; j < 4; ++j) b[f][j] = static_cast<int>(w4[j] & (0x03030303u << (2 * f)));
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        const i32x4 av = avb[t & 1][fm];
#pragma unroll
        for (int f = 0; f < 4; ++f)
          acc[fm][f] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, b[f], acc[fm][f], 0, 0, 0);
      }
    }
  };

#pragma unroll
  for (int r = 0; r < R; ++r) {
    load_q(qr[r], r);
    load_w(w[r], r);
  }
  store_q(qr[0], 0);
  __syncthreads();
  // chunk c: weights and q registers in ring slot c % R, q in LDS buffer c % 2. Step c
  // reduces chunk c, reloads its slot with chunk c + R, stores chunk c + 1's q, one barrier.
  for (int c0 = 0; c0 < nchh; c0 += R) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int c = c0 + r;
      if (c < nch) compute(w[r], c & 1);
      load_q(qr[r], c + R);
      load_w(w[r], c + R);
      store_q(qr[(r + 1) % R], (c + 1) & 1);
      __syncthreads();
    }
  }
  if constexpr (KS > 1) {
    // the later parts' sums join the first part's, lane for lane, in part order
    __syncthreads();                        // every wave is done with the q chunks
    int* red = reinterpret_cast<int*>(lds + kStBytes);
    auto slot = [&](int part) __attribute__((always_inline)) {
      return red + ((part - 1) * BW + wave) * FM * 16 * 64;
    };
    if (half) {
      int* dst = slot(half);
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int f = 0; f < 4; ++f)
#pragma unroll
          for (int i = 0; i < 4; ++i) dst[((fm * 4 + f) * 4 + i) * 64 + lane] = acc[fm][f][i];
    }
    __syncthreads();
    if (!half) {
#pragma unroll
      for (int part = 1; part < KS; ++part) {
        const int* src = slot(part);
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
          for (int f = 0; f < 4; ++f)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[fm][f][i] += src[((fm * 4 + f) * 4 + i) * 64 + lane];
      }
    }
  }
  // Without a K split the integers leave through LDS as whole rows: each wave stages its
  // 16 x 64 slice of row tile fm (rows kStRow ints apart: conflict-free both ways), then
  // writes it back row by row, lane = column, so every store covers 256 contiguous bytes
  // (from the MFMA layout directly, a store covers four 64-byte pieces of four rows).
  if (nsplit == 1) {
    __syncthreads();                        // every wave is done with the q chunks
    int* st = reinterpret_cast<int*>(lds) + wave * 16 * kStRow;
    const int64_t col = band * 64 + lane;
    const float bcol = (a.y != nullptr && active) ? a.beta[a.beta_len == 1 ? 0 : col] : 0.0f;
    // row sums and scales of the workgroup's rows, lane l holding row m0 + l (clamped), read
    // by every row below as a wave-uniform value
    const int64_t rl = min<int64_t>(m0 + lane, a.M - 1);
    const int rs_l = rowsum[rl];
    const float gs_l = a.y != nullptr ? a.gamma[rl] / 127.0f : 0.0f;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      if (!half) {
#pragma unroll
        for (int k = 0; k < 16; ++k)   // output k: row 4g + k % 4, column 16 (k / 4) + u
          st[(4 * g + k % 4) * kStRow + 16 * (k / 4) + u] = acc[fm][k / 4][k % 4] >> (2 * (k / 4));
      }
      __syncthreads();
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rr = 16 * fm + r;
        const int rsv = __builtin_amdgcn_readlane(rs_l, rr);
        const int v = st[r * kStRow + lane] - (lane < 48 ? rsv : 0);   // fragments f < 3
        const float gs = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gs_l), rr));
        const int64_t row = m0 + rr;
        // outputs are written once and not read back here: non-temporal stores (measured on
        // MI355X, 3B-shaped prefill at M = 512: the four products 1195 -> 1262 TOPS)
        if (!half && active && row < a.M) {
          if (a.acc_out) __builtin_nontemporal_store(v, &a.acc_out[row * a.N + col]);
          if (a.y) __builtin_nontemporal_store(static_cast<float>(v) * gs * bcol, &a.y[row * a.N + col]);
        }
      }
      __syncthreads();
    }
    return;
  }
  if (half || !active) return;

  // output k = 4 f + i of row tile fm: row m0 + 16 fm + 4g + i, column band * 64 + 16 f + u
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    int32_t v[16];
    uint32_t live = 0;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      v[k] = acc[fm][k / 4][k % 4] >> (2 * (k / 4));
      if (m0 + 16 * fm + 4 * g + k % 4 < a.M) live |= 1u << k;
    }
    uint32_t done = live;
    if (nsplit > 1 && nsplit <= kMaxPairSplits) {
      // rows 4g + 2p and 4g + 2p + 1 of column 16f + u share one split word (pair e = 2f + p
      // holds outputs k = 2e, 2e + 1), word row = first row / 2
      uint32_t plive = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (m0 + 16 * fm + 4 * g + 2 * (e & 1) < a.M) plive |= 1u << e;
      auto pword = [&](int e) __attribute__((always_inline)) {
        const int64_t r0 = min<int64_t>(m0 + 16 * fm + 4 * g + 2 * (e & 1), a.M - 1);
        return a.ws_acc + (r0 / 2) * a.N + band * 64 + 16 * (e >> 1) + u;
      };
      const uint32_t pd = split_arrive_pairs<8>(pword, v, plive, nsplit);
      done = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if ((pd >> e) & 1u) done |= 3u << (2 * e);
      done &= live;
    } else if (nsplit > 1) {
      auto word = [&](int k) __attribute__((always_inline)) {
        const int64_t row = min<int64_t>(m0 + 16 * fm + 4 * g + k % 4, a.M - 1);
        return a.ws_acc + row * a.N + band * 64 + 16 * (k / 4) + u;
      };
      done = split_arrive_batch<16>(word, v, live, nsplit);
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      if (!((done >> k) & 1u)) continue;
      const int64_t row = m0 + 16 * fm + 4 * g + k % 4;
      const int64_t col = band * 64 + 16 * (k / 4) + u;
      const int r = v[k] - (k / 4 < 3 ? rowsum[row] : 0);
      if (a.acc_out) a.acc_out[row * a.N + col] = r;
      if (a.y)
        a.y[row * a.N + col] = static_cast<float>(r) * (a.gamma[row] / 127.0f) *
                               a.beta[a.beta_len == 1 ? 0 : col];
    }
  }
}

struct TernPlan { int64_t bands, mgroups, nsplit, tps; int fm; bool split; };

}  // namespace

namespace {

TernPlan plan_tern(int64_t M, int64_t N, int64_t K) {
  const int64_t KT = K / 64, bands = N / 64;
  // measured on MI355X (70B-shaped decode at M = 8..64): one 16-row tile of q per wave
  // (more workgroups, each weight tile re-read per 16 rows from L2) except for very wide
  // outputs, where two
  const int fm = M > 16 && bands >= 512 ? 2 : 1;
  const int64_t mgroups = (M + 16 * fm - 1) / (16 * fm);
  const int64_t target = 512;
  int64_t nsplit = (target + bands * mgroups - 1) / (bands * mgroups);
  nsplit = std::min<int64_t>(nsplit, std::max<int64_t>(1, KT / 8));   // >= 2 tiles per wave
  nsplit = std::max<int64_t>(nsplit, 1);
  if (M * N > kAccCap || K > kMaxIntSplitK) nsplit = 1;
  nsplit = std::min<int64_t>(nsplit, kMaxIntSplits);
  const int64_t tps = (KT + nsplit - 1) / nsplit;
  const bool split = fm <= 2;   // VALU-bound at few rows
  return {bands, mgroups, (KT + tps - 1) / tps, tps, fm, split};
}

}  // namespace

namespace {

TernArgs mf_args(const int8_t* q, const float* gamma, const void* wmf, const float* beta,
                 int64_t beta_len, int64_t M, int64_t N, int64_t K, float* y, int32_t* acc_out,
                 uint64_t* ws_acc, int64_t tps) {
  return TernArgs{q, gamma, static_cast<const u32x4*>(wmf), beta, beta_len, M, N, K, y,
                  acc_out, ws_acc, static_cast<int>(tps)};
}

// Per-band kernel: one 16-row tile of q per workgroup, K split until ~512 workgroups.
hipError_t launch_mf_band(const int8_t* q, const float* gamma, const int32_t* rowsum, int64_t M,
                          int64_t K, const void* wmf, const float* beta, int64_t beta_len,
                          int64_t N, float* y, int32_t* acc_out, uint64_t* ws_acc,
                          hipStream_t s) {
  const int64_t KT = K / 64, bands = N / 64;
  const int64_t mgroups = (M + 15) / 16;
  const int64_t target = 512;
  int64_t nsplit = (target + bands * mgroups - 1) / (bands * mgroups);
  nsplit = std::min<int64_t>(nsplit, std::max<int64_t>(1, KT / 8));
  nsplit = std::max<int64_t>(nsplit, (KT + kMfMaxSplitTiles - 1) / kMfMaxSplitTiles);
  if (M * N > kAccCap) nsplit = 1;
  nsplit = std::min<int64_t>(nsplit, kMaxIntSplits);
  int64_t tps = (KT + nsplit - 1) / nsplit;
  nsplit = (KT + tps - 1) / tps;
  if (nsplit == 1) tps = KT;   // no split words: sum q (w + 1) fits int32 for K <= 65536
  const TernArgs a = mf_args(q, gamma, wmf, beta, beta_len, M, N, K, y, acc_out, ws_acc, tps);
  const dim3 grid(static_cast<unsigned>(bands), static_cast<unsigned>(mgroups),
                  static_cast<unsigned>(nsplit));
  hipLaunchKernelGGL((tern_mf_kernel<1>), grid, dim3(256), 0, s, a, rowsum);
  return hipGetLastError();
}

// Row tile of the staged-q kernel (16 fm rows per workgroup), measured on MI355X
// (70B-shaped batched decode, 3B-shaped prefill): 32 rows for 17..64 rows of q where that
// still gives >= 192 workgroups (the decoded weights serve more rows), else 16 (row groups
// of a band group share its weights through one XCD's L2, and more workgroups win).
int mfq_fm(int64_t M, int64_t groups) {
  // measured on MI355X: 48-row tiles for prefill-sized M over >= 32 band groups (3B at
  // M = 512: gate|up 34.2 vs 46.3 us with 16-row tiles, q|k|v 26.8 vs 28.0 us; o and down,
  // 13 groups, too few work items, were slower; 64-row tiles were slower everywhere),
  // 32-row tiles for 17-64 rows where they still give enough work items, else 16
  if (M >= 256 && groups >= 32) return 3;
  return (M > 16 && M <= 64 && groups * ((M + 31) / 32) >= 192) ? 2 : 1;
}

struct QuadPlan { int fm, bw; int64_t groups, mgroups, nsplit, tps; };

QuadPlan plan_mf_quad(int64_t M, int64_t N, int64_t K) {
  const int64_t KT = K / 64, bands = N / 64;
  int64_t groups = (bands + 3) / 4;
  const int fm = mfq_fm(M, groups);
  const int64_t mgroups = (M + 16 * fm - 1) / (16 * fm);
  // K is split until about `target` workgroups; a split spans whole ring turns where the
  // range allows (no padded chunks) and at most kMfMaxSplitTiles tiles (split word bias)
  const int64_t target = 256;
  // Where 16-row items of four bands would split K, more than 16 rows take items of two bands
  // (each band's range in two halves met in LDS), or of one band (four quarters) where even
  // those would split, and need fewer splits (measured on MI355X, 70B-shaped batched decode:
  // at M = 64 o 17.4 -> 12.6 us, down 32.2 -> 30.1 us, the pass 10.20 -> 9.50 ms; at M = 32,
  // one-band o and down, the pass 8.11 -> 7.85 -> 7.51 ms; q|k|v at M = 64, not split, was
  // slower as 320 two-band items, 17.9 against 16.7 us; at M = 16 slower)
  const int bw = (fm == 1 && M > 16 && 2 * groups * mgroups <= target)
                     ? (4 * groups * mgroups <= target ? 1 : 2) : 4;
  groups = (bands + bw - 1) / bw;
  int64_t nsplit = std::max<int64_t>(1, target / (groups * mgroups));
  const int64_t turn = kQC * kQRing;
  int64_t tps = (KT + nsplit - 1) / nsplit;
  tps = std::min<int64_t>((tps + turn - 1) / turn * turn, kMfMaxSplitTiles / turn * turn);
  nsplit = (KT + tps - 1) / tps;
  if (M * N > kAccCap) nsplit = 1;
  if (nsplit == 1) tps = KT;   // no split words: sum q (w + 1) fits int32 for K <= 65536
  // (nsplit <= KT / 12 <= 86 < kMaxIntSplits: a split word never overflows its count)
  return {fm, bw, groups, mgroups, nsplit, tps};
}

// Staged-q kernel: four bands and 16 fm rows per workgroup.
hipError_t launch_mf_quad(const int8_t* q, const float* gamma, const int32_t* rowsum, int64_t M,
                          int64_t K, const void* wmf, const float* beta, int64_t beta_len,
                          int64_t N, float* y, int32_t* acc_out, uint64_t* ws_acc,
                          hipStream_t s) {
  const QuadPlan p = plan_mf_quad(M, N, K);
  const int fm = p.fm;
  const int64_t groups = p.groups, mgroups = p.mgroups, nsplit = p.nsplit;
  const TernArgs a = mf_args(q, gamma, wmf, beta, beta_len, M, N, K, y, acc_out, ws_acc, p.tps);
  const int64_t nwork = groups * mgroups * nsplit;   // one workgroup per item, 8 | grid
  const dim3 grid(static_cast<unsigned>((nwork + 7) / 8 * 8));
  if (fm == 1 && p.bw == 1)
    hipLaunchKernelGGL((tern_mfq_kernel<1, 1>), grid, dim3(256), 0, s, a, rowsum);
  else if (fm == 1 && p.bw == 2)
    hipLaunchKernelGGL((tern_mfq_kernel<1, 2>), grid, dim3(256), 0, s, a, rowsum);
  else if (fm == 1)
    hipLaunchKernelGGL((tern_mfq_kernel<1, 4>), grid, dim3(256), 0, s, a, rowsum);
  else if (fm == 2)
    hipLaunchKernelGGL((tern_mfq_kernel<2, 4>), grid, dim3(256), 0, s, a, rowsum);
  else
    hipLaunchKernelGGL((tern_mfq_kernel<3, 4>), grid, dim3(256), 0, s, a, rowsum);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_tern_mf(const int8_t* q, const float* gamma, const int32_t* rowsum, int64_t M,
                          int64_t K, const void* wmf, const float* beta, int64_t beta_len,
                          int64_t N, float* y, int32_t* acc_out, uint64_t* ws_acc, hipStream_t s) {
  // up to eight rows of narrow outputs: the four-band kernel with q of a whole K range in
  // LDS (measured on MI355X, 70B-shaped, us: M = 8 q|k|v 11.4 / o 11.0 / down 17.4
  // against 13.3 / 12.2 / 19.6 here; M = 1 down 13.3 against 16.0; wide outputs and M = 16
  // were slower, e.g. gate|up at M = 8 27.6 against 23.9)
  if (M <= 8 && N / 64 < 512 && mf_qgemv_fits(M, N, K))
    return launch_mf_qgemv(q, gamma, rowsum, static_cast<int>(M), K, wmf, beta, beta_len, N, y,
                           acc_out, ws_acc, s);
  // otherwise (measured on MI355X, 70B-shaped decode at M = 8..64, 3B-shaped prefill at
  // M = 512) the staged-q kernel wherever its work items (four-band groups x row tiles)
  // number >= 160, so that it fills the GPU without splitting K (e.g. gate|up at M = 64:
  // 42 us against 91 us per band; every 3B GEMM at M = 512), and with fewer where at most
  // eight K splits meet in split words shared by two rows (M = 64: down 35.3 against 46.7
  // us per band, q|k|v 18.4 both; M = 32: down 25.1 against 31.4, q|k|v 16.1 against 19.4;
  // M = 16: down 20.5 against 22.7); more splits would cost M x N split-word atomics per
  // split, more than the per-band kernel's repeated weight reads
  const QuadPlan qp = plan_mf_quad(M, N, K);
  const bool quad = qp.groups * qp.mgroups >= 160 || qp.nsplit <= kMaxPairSplits;
  return quad ? launch_mf_quad(q, gamma, rowsum, M, K, wmf, beta, beta_len, N, y, acc_out,
                               ws_acc, s)
              : launch_mf_band(q, gamma, rowsum, M, K, wmf, beta, beta_len, N, y, acc_out,
                               ws_acc, s);
}

hipError_t launch_tern_mfma(const int8_t* q, const float* gamma, int64_t M, int64_t K,
                            const void* wpacked, const float* beta, int64_t beta_len, int64_t N,
                            float* y, int32_t* acc_out, uint64_t* ws_acc, hipStream_t s) {
  const TernPlan p = plan_tern(M, N, K);
  TernArgs a{q, gamma, static_cast<const u32x4*>(wpacked), beta, beta_len, M, N, K, y, acc_out,
             ws_acc, static_cast<int>(p.tps)};
  const dim3 grid(static_cast<unsigned>(p.bands), static_cast<unsigned>(p.mgroups),
                  static_cast<unsigned>(p.nsplit));
#define BL_TERN_LAUNCH(FM_, SPLIT_) \
  hipLaunchKernelGGL((tern_mfma_kernel<FM_, SPLIT_>), grid, dim3(256), 0, s, a)
  switch (p.fm * 2 + (p.split ? 1 : 0)) {
    case 2: BL_TERN_LAUNCH(1, false); break;
    case 3: BL_TERN_LAUNCH(1, true); break;
    case 4: BL_TERN_LAUNCH(2, false); break;
    case 5: BL_TERN_LAUNCH(2, true); break;
    case 9: BL_TERN_LAUNCH(4, true); break;
    default: BL_TERN_LAUNCH(4, false); break;
  }
#undef BL_TERN_LAUNCH
  return hipGetLastError();
}

}  // namespace bl
