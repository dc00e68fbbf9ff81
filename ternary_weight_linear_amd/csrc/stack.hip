// Whole-stack decode: a list of BitLinear layers in one persistent launch.
//
// [b158] "实验及结果", Table 3: the 70B model's decode throughput is a sweep over all of its
// linears, one token at a time; Fig. 3: each product is int8 additions. Launched one layer
// at a time, every GEMV pays a fixed cost of several microseconds: the launch, the ramp-up of
// its memory stream, gamma and the first chunk's quantisation before any weight is reduced,
// and the tail of its last workgroups. Here one grid of resident workgroups walks the whole
// list. Weights never depend on activations, so a workgroup keeps its weight loads running
// across the boundary between linears: the first weights of its share of linear l + 1 are in
// flight while it waits for linear l to finish.
//
// Order: linear l reads its x only after every workgroup has finished linears 0 .. l - 1.
// Arrivals go up a two-level counter tree in the workspace; a workgroup arrives for linear l
// only after it has seen linear l released, so the counts of a level reach (l + 1) times
// their members exactly when every workgroup below has finished linear l. The result is
// that of separate calls in order, also when a y overlaps a later x (read after write) or an
// earlier x (write after read): y is written with agent-scope stores, performed at the
// device coherence point instead of being left in one XCD's L2, and a linear whose x
// overlaps an earlier y loads x with agent-scope loads. (Outputs overlapping each other,
// weights or scales are rejected when the plan is made.)
//
// Work split: linear l has T = groups * KT "group tiles" (a group is four 64-row bands, one
// per wave of a workgroup; a group tile is those bands' tiles at one 64-input position).
// Workgroup w of the G_l taking part gets group tiles [w T / G_l, (w + 1) T / G_l): shares
// equal to one tile whatever the shape. A share may start or end inside a group; the
// workgroups sharing a group combine exact int32 partial sums with the one-atomic split
// hand-off, so the integers are those of one sum.
//
// Per tile the arithmetic is the fused GEMV's: gamma = max |x| over the row (integer max of
// the fp16 bit patterns with the sign cleared; >= 0x7C00 flags NaN/inf), q = rne(127 x /
// gamma) clipped to +-127 in fp32, eight wave ballots make a tile's bit planes, and per
// 32-input word and plane one select and one popcount; acc = sum_b c_b A_b + popcount(N).
#include <atomic>
#include <cstdlib>
#include <cstring>
#include <type_traits>
#include <vector>

#include "bl_internal.h"

namespace bl {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Pointers read from the plan carry no address space; global ones let the compiler use
// global (not flat) memory instructions, whose completion it can count precisely.
#define BL_GLOBAL __attribute__((address_space(1)))
template <class T>
__device__ __forceinline__ const BL_GLOBAL T* gptr(const T* p) {
  return (const BL_GLOBAL T*)(p);
}
template <class T>
__device__ __forceinline__ BL_GLOBAL T* gptr_mut(T* p) {
  return (BL_GLOBAL T*)(p);
}

// One workgroup of 8 waves per CU (measured on MI355X, 70B-shaped pass at M = 1: 5.74 ms
// against 6.18 ms with three 4-wave workgroups per CU; 16 waves, 5.65 ms, leave too few
// registers for M = 3, 4). The waves of a workgroup meet at every chunk barrier, so no lone
// late workgroup is left on a CU at the end of a linear.
constexpr int kSW = 8;                    // waves per workgroup, one 64-row band each
constexpr int kSB = 4;                    // tiles per register batch; the ring holds two
constexpr int kSChunk = 64;               // tiles whose planes sit in LDS at once
constexpr int kSPerWave = kSChunk / kSW;  // tiles each wave quantises per chunk
constexpr int kSGX = 4;                   // 16-byte x loads per thread per gamma round
// Workgroups sharing one group at most (<= kMaxIntSplits - 1 so a split word never
// overflows its count).
constexpr int64_t kSMaxContrib = 254;
static_assert(kSMaxContrib <= kMaxIntSplits - 1, "split word count");
constexpr uint32_t kStackMagic = 0x4B435453u;
// Bound of one grid-wide wait: 2 s of the 100 MHz real-time counter.
constexpr uint64_t kWaitTicks = 200000000ull;
// Grid-wide wait: a two-level tree (measured on MI355X: one counter for 1024 workgroups
// takes ~13 us per wait, groups of 32 ~2.5 us). Slots are 256 bytes apart: group counters,
// then the root counter, then one release word per group.
constexpr int kBarGroup = 32;
constexpr int kBarPad = 64;                              // uint32 per slot
constexpr int kMaxStackGrid = 4096;                      // <= 128 groups
constexpr int kBarGroups = kMaxStackGrid / kBarGroup;
constexpr int kBarWords = (2 * kBarGroups + 1) * kBarPad;

struct StackEntry {
  const uint16_t* x;
  const u32x4* W;
  const float* beta;
  float* y;
  int64_t beta_len, N, K;
  uint32_t raw;   // x overlaps the y of an earlier linear: load it at agent scope
  uint32_t pad;
};
struct StackHeader {
  uint32_t magic, count, M, status;
  uint32_t pad[12];
};
static_assert(sizeof(StackEntry) == 64, "plan entry layout");
static_assert(sizeof(StackHeader) == 64, "plan header layout");

// The part of linear (N, K) that workgroups of a grid of `grid` take. Every count fits 32
// bits (N <= 4194304, K <= 65536); products of two of them are taken in 64 bits.
struct LinSplit {
  int KT;      // 64-input tiles per row
  int bands;   // 64-row bands
  int T;       // group tiles
  int G;       // workgroups taking part (0 .. G - 1)
};
__device__ __forceinline__ LinSplit lin_split(int64_t N, int64_t K, int grid) {
  LinSplit s;
  s.KT = static_cast<int>(K / 64);
  s.bands = static_cast<int>(N / 64);
  const int groups = (s.bands + kSW - 1) / kSW;
  s.T = groups * s.KT;
  s.G = static_cast<int>(min<int64_t>(grid, min<int64_t>(s.T, kSMaxContrib * groups)));
  return s;
}
// Workgroup whose share holds group tile a.
__device__ __forceinline__ int lin_cover(const LinSplit& s, int a) {
  return static_cast<int>((static_cast<int64_t>(a + 1) * s.G - 1) / s.T);
}
// First group tile of workgroup w's share (w = G: the end of the last share).
__device__ __forceinline__ int lin_start(const LinSplit& s, int w) {
  return static_cast<int>(static_cast<int64_t>(w) * s.T / s.G);
}

// Position of one workgroup in its sequence of (linear, group, chunk, batch). Every value
// is the same in all waves of the workgroup.
struct Cursor {
  int l;               // linear; == count once past the end
  int end;             // end of this workgroup's share of linear l (group tiles)
  int g;               // current group
  int t, cs, cend, send;   // tile within group g; start and end of the current chunk; end
                           // of the segment (this workgroup's part of group g)
  LinSplit sp;
  const StackEntry* e;
};

__device__ __forceinline__ bool has_work(const StackEntry* ent, int l, int w, int grid) {
  return w < lin_split(ent[l].N, ent[l].K, grid).G;
}

// Places c at the start of this workgroup's share of linear l (which must have work).
__device__ __forceinline__ void cursor_enter(Cursor& c, const StackEntry* ent, int l, int w,
                                             int grid) {
  c.l = l;
  c.e = ent + l;
  c.sp = lin_split(c.e->N, c.e->K, grid);
  const int s = lin_start(c.sp, w);
  c.end = lin_start(c.sp, w + 1);
  c.g = s / c.sp.KT;
  c.t = s - c.g * c.sp.KT;
  c.send = min(c.sp.KT, c.end - c.g * c.sp.KT);
  c.cs = c.t;
  c.cend = min(c.send, c.t + kSChunk);
}

// What finished when a cursor moved past a batch.
enum : int { kStepChunk = 1, kStepSegment = 2, kStepLinear = 4 };

// Moves c to the next batch; returns which boundaries it crossed. Past the last linear
// c.l == count (the other fields keep their last values).
__device__ __forceinline__ int cursor_next(Cursor& c, const StackEntry* ent, int count, int w,
                                           int grid) {
  c.t += kSB;
  if (c.t < c.cend) return 0;
  if (c.cend < c.send) {
    c.t = c.cend;
    c.cs = c.t;
    c.cend = min(c.send, c.t + kSChunk);
    return kStepChunk;
  }
  const int pos = c.g * c.sp.KT + c.send;
  if (pos < c.end) {   // the share goes on in the next group, from its first tile
    c.g += 1;
    c.t = 0;
    c.cs = 0;
    c.send = min(c.sp.KT, c.end - c.g * c.sp.KT);
    c.cend = min(c.send, kSChunk);
    return kStepChunk | kStepSegment;
  }
  int l = c.l + 1;
  while (l < count && !has_work(ent, l, w, grid)) ++l;
  if (l < count) {
    cursor_enter(c, ent, l, w, grid);
  } else {
    c.l = count;
  }
  return kStepChunk | kStepSegment | kStepLinear;
}

template <int MR>
__global__ __launch_bounds__(64 * kSW) void gemv_stack_kernel(StackHeader* __restrict__ hdr,
                                                              uint32_t* __restrict__ bar,
                                                              uint64_t* __restrict__ ws_acc,
                                                              int count) {
  __shared__ __attribute__((aligned(16))) uint32_t pl[kSChunk][MR][16];
  __shared__ uint32_t red_max[kSW][MR];
  __shared__ int wait_ok;
  const StackEntry* ent = reinterpret_cast<const StackEntry*>(hdr + 1);
  if (hdr->magic != kStackMagic || static_cast<int>(hdr->count) != count || hdr->M != MR) {
    if (blockIdx.x == 0 && threadIdx.x == 0)
      __hip_atomic_store(&hdr->status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int w = blockIdx.x;
  const int grid = gridDim.x;
  // barrier tree: this workgroup's group counter and release word, the root counter
  const int ngrp = (grid + kBarGroup - 1) / kBarGroup;
  const int grp = w / kBarGroup;
  const uint32_t members = static_cast<uint32_t>(min(kBarGroup, grid - grp * kBarGroup));
  uint32_t* const gcnt = bar + grp * kBarPad;
  uint32_t* const root = bar + kBarGroups * kBarPad;
  uint32_t* const rel0 = bar + (kBarGroups + 1) * kBarPad;
  // lane l <-> plane bit l of a tile: half h = l / 32, bit p = l % 32 = 8i + j <-> c = 4j + i
  const int koff = 32 * (lane >> 5) + 4 * (lane & 7) + ((lane & 31) >> 3);

  // Grid-wide wait for linear l: every workgroup has finished linears 0 .. l - 1, i.e. the
  // release word of this workgroup's group holds l.
  auto grid_wait = [&](int l) __attribute__((always_inline)) -> bool {
    if (l == 0) return true;
    if (threadIdx.x == 0) {
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      int ok = 1;
      while (__hip_atomic_load(rel0 + grp * kBarPad, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
             static_cast<uint32_t>(l)) {
        __builtin_amdgcn_s_sleep(1);
        if (__builtin_amdgcn_s_memrealtime() - t0 > kWaitTicks) {
          __hip_atomic_store(&hdr->status, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          ok = 0;
          break;
        }
      }
      wait_ok = ok;
    }
    __syncthreads();
    return wait_ok != 0;
  };
  // Arrival for finished linear l, after this workgroup's outputs are complete. The last
  // arrival of a group goes on to the root; the last root arrival releases every group (or,
  // after the last linear, when nobody waits any more, zeroes the tree for the next launch).
  auto arrive = [&](int l) __attribute__((always_inline)) {
    wait_own_memory_ops();
    __syncthreads();
    if (threadIdx.x == 0) {
      const uint32_t done = static_cast<uint32_t>(l + 1);
      if (__hip_atomic_fetch_add(gcnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1 ==
              done * members &&
          __hip_atomic_fetch_add(root, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1 ==
              done * static_cast<uint32_t>(ngrp)) {
        if (l + 1 == count) {
          for (int g = 0; g < ngrp; ++g) {
            __hip_atomic_store(bar + g * kBarPad, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(rel0 + g * kBarPad, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
          __hip_atomic_store(root, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
          for (int g = 0; g < ngrp; ++g)
            __hip_atomic_store(rel0 + g * kBarPad, done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
  };
  // Linears this workgroup has no share of still take part in the order.
  auto pass_through = [&](int from, int to) __attribute__((always_inline)) -> bool {
    for (int l = from; l < to; ++l) {
      if (!grid_wait(l)) return false;
      arrive(l);
    }
    return true;
  };

  // first linear with a share for this workgroup; the ones before it are passed through
  // (once: every workgroup arrives exactly once per linear) after the first weight loads
  int l0 = 0;
  while (l0 < count && !has_work(ent, l0, w, grid)) ++l0;
  if (l0 == count) {
    pass_through(0, count);
    return;
  }

  Cursor C, L;
  cursor_enter(C, ent, l0, w, grid);
  L = C;

  // weight pointer of the load cursor: this wave's band of the current group (clamped to
  // the last band; a wave past the last band loads and discards)
  auto band_ptr = [&](const Cursor& c) __attribute__((always_inline)) {
    const int64_t band = min(c.g * kSW + wave, c.sp.bands - 1);
    return gptr(c.e->W) + band * c.sp.KT * 64 + lane;
  };
  u32x4 ring[2][kSB];
  auto issue = [&](u32x4 (&dst)[kSB], const Cursor& c) __attribute__((always_inline)) {
    const auto wp = band_ptr(c);
#pragma unroll
    for (int u = 0; u < kSB; ++u)   // weights are read once: non-temporal
      dst[u] = __builtin_nontemporal_load(&wp[static_cast<int64_t>(min(c.t + u, c.cend - 1)) * 64]);
  };

  float gam[MR];
  bool zero[MR];
  int A[MR][8];
  int cn = 0;
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int b = 0; b < 8; ++b) A[m][b] = 0;

  // gamma of linear C.l (after its grid-wide wait): every workgroup reduces the whole row
  auto gamma_of = [&](const StackEntry* e) __attribute__((always_inline)) {
    const int64_t K = e->K;
    const int64_t K8 = K / 8;
    const bool raw = e->raw != 0;
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      uint32_t mb = 0;
      auto fold = [&](uint32_t v) __attribute__((always_inline)) { mb = max(mb, max(v & 0x7FFFu, (v >> 16) & 0x7FFFu)); };
      if (!raw) {
        const BL_GLOBAL u32x4* row4 = gptr(reinterpret_cast<const u32x4*>(e->x + m * K));
        for (int64_t i0 = 0; i0 < K8; i0 += 64 * kSW * kSGX) {
          u32x4 v[kSGX];
#pragma unroll
          for (int i = 0; i < kSGX; ++i)   // repeated elements do not change the maximum
            v[i] = row4[min<int64_t>(i0 + threadIdx.x + 64 * kSW * i, K8 - 1)];
#pragma unroll
          for (int i = 0; i < kSGX; ++i) {
            fold(v[i].x); fold(v[i].y); fold(v[i].z); fold(v[i].w);
          }
        }
      } else {
        const BL_GLOBAL uint32_t* row = gptr(reinterpret_cast<const uint32_t*>(e->x + m * K));
        for (int64_t i = threadIdx.x; i < K / 2; i += 64 * kSW)
          fold(__hip_atomic_load(row + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) mb = max(mb, static_cast<uint32_t>(__shfl_xor(mb, off)));
      if (lane == 0) red_max[wave][m] = mb;
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      uint32_t mb = red_max[0][m];
#pragma unroll
      for (int w2 = 1; w2 < kSW; ++w2) mb = max(mb, red_max[w2][m]);
      const bool bad = mb >= 0x7C00u;
      gam[m] = bad ? __uint_as_float(0x7FC00000u) : half_bits_to_float(static_cast<uint16_t>(mb));
      zero[m] = bad || mb == 0u;
    }
  };

  // the x values this wave quantises in the chunk [c.t, c.cend) of linear c.l (issued before
  // gamma's loads at a linear's start, so both arrive in one round trip)
  uint16_t xq[kSPerWave][MR];
  auto load_chunk_x = [&](const Cursor& c) __attribute__((always_inline)) {
    const StackEntry* e = c.e;
    const int64_t K = e->K;
    const BL_GLOBAL uint16_t* xg = gptr(e->x);
    const BL_GLOBAL uint32_t* xg32 = gptr(reinterpret_cast<const uint32_t*>(e->x));
    if (e->raw == 0) {
#pragma unroll
      for (int j = 0; j < kSPerWave; ++j) {
        const int tt = min(c.t + wave + kSW * j, c.cend - 1);
#pragma unroll
        for (int m = 0; m < MR; ++m) xq[j][m] = xg[m * K + 64 * tt + koff];
      }
    } else {
#pragma unroll
      for (int j = 0; j < kSPerWave; ++j) {
        const int tt = min(c.t + wave + kSW * j, c.cend - 1);
#pragma unroll
        for (int m = 0; m < MR; ++m) {
          const int64_t k = m * K + 64 * tt + koff;
          const uint32_t v = __hip_atomic_load(xg32 + (k >> 1), __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
          xq[j][m] = static_cast<uint16_t>((k & 1) ? (v >> 16) : v);
        }
      }
    }
  };
  // planes of the chunk [c.t, c.cend) into LDS from xq (the caller syncs before and after)
  auto quantise_chunk = [&](const Cursor& c) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kSPerWave; ++j) {
      const int tt = c.t + wave + kSW * j;
      if (tt < c.cend) {
#pragma unroll
        for (int m = 0; m < MR; ++m) {
          const int qv = zero[m] ? 0 : quant_q(half_bits_to_float(xq[j][m]) * 127.0f, gam[m],
                                               __builtin_amdgcn_rcpf(gam[m]));
          uint32_t mine = 0;
#pragma unroll
          for (int b = 0; b < 8; ++b) {
            const unsigned long long mask = __ballot((qv >> b) & 1);
            if ((lane >> 1) == b) mine = (lane & 1) ? static_cast<uint32_t>(mask >> 32) : static_cast<uint32_t>(mask);
          }
          if (lane < 16) pl[tt - c.cs][m][lane] = mine;
        }
      }
    }
  };

  // end of this workgroup's part of group C.g: combine with the other workgroups sharing it
  auto finish_group = [&](const Cursor& c) __attribute__((always_inline)) {
    const StackEntry* e = c.e;
    const int64_t band = c.g * kSW + wave;
    const int a0 = c.g * c.sp.KT;
    const int nsplit = lin_cover(c.sp, a0 + c.sp.KT - 1) - lin_cover(c.sp, a0) + 1;
    if (band < c.sp.bands) {
      const int64_t N = e->N;
      const int64_t n = band * 64 + lane;
      const float b = gptr(e->beta)[e->beta_len == 1 ? 0 : n];
      BL_GLOBAL float* yg = gptr_mut(e->y);
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        const int acc = A[m][0] + 2 * A[m][1] + 4 * A[m][2] + 8 * A[m][3] + 16 * A[m][4] +
                        32 * A[m][5] + 64 * A[m][6] - 128 * A[m][7] + cn;
        int total = acc;
        if (nsplit > 1 && !split_arrive(&ws_acc[m * N + n], acc, nsplit, &total)) continue;
        __hip_atomic_store(yg + (m * N + n), static_cast<float>(total) * (gam[m] / 127.0f) * b,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
      for (int b = 0; b < 8; ++b) A[m][b] = 0;
    cn = 0;
  };

  // select + popcount over the tiles of one batch (planes of the current chunk in LDS)
  auto reduce_batch = [&](const u32x4 (&wb)[kSB], const Cursor& c) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kSB; ++u) {
      if (c.t + u < c.cend) {
        const u32x4 wc = wb[u];
        const int pt = c.t + u - c.cs;
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
  };

  // One step: (at a chunk start: wait / gamma, quantise) issue the load cursor's batch into
  // the free ring slot, reduce the compute cursor's batch from slot S, move on. The ring
  // slot of a batch alternates, so the loop body holds two steps with constant slots.
  bool chunk_start = true, lin_start = true;
  auto step = [&](auto slot) __attribute__((always_inline)) -> bool {
    constexpr int S = decltype(slot)::value;
    if (chunk_start) {
      if (lin_start) {
        if (!grid_wait(C.l)) return false;   // includes a barrier of the workgroup
        load_chunk_x(C);
        gamma_of(C.e);
      } else {
        __syncthreads();                    // every wave is done with the previous planes
        load_chunk_x(C);
      }
      quantise_chunk(C);
      __syncthreads();
    }
    __builtin_amdgcn_sched_barrier(0);
    issue(ring[1 - S], L);
    __builtin_amdgcn_sched_barrier(0);
    if (L.l < count) cursor_next(L, ent, count, w, grid);
    reduce_batch(ring[S], C);
    const Cursor Cp = C;
    const int crossed = cursor_next(C, ent, count, w, grid);
    chunk_start = crossed != 0;
    lin_start = (crossed & kStepLinear) != 0;
    if (crossed & kStepSegment) finish_group(Cp);
    if (crossed & kStepLinear) {
      arrive(Cp.l);
      if (!pass_through(Cp.l + 1, C.l)) return false;
      if (C.l == count) return false;
    }
    return true;
  };

  issue(ring[0], L);
  cursor_next(L, ent, count, w, grid);
  if (!pass_through(0, l0)) return;
  while (step(std::integral_constant<int, 0>{}) && step(std::integral_constant<int, 1>{})) {
  }
}

}  // namespace

size_t stack_plan_bytes(int64_t count) {
  return sizeof(StackHeader) + static_cast<size_t>(count) * sizeof(StackEntry);
}

hipError_t stack_write_plan(const bl_linear_desc* d, int64_t count, int64_t M, void* plan,
                            hipStream_t s) {
  std::vector<unsigned char> buf(stack_plan_bytes(count), 0);
  StackHeader h{};
  h.magic = kStackMagic;
  h.count = static_cast<uint32_t>(count);
  h.M = static_cast<uint32_t>(M);
  h.status = 0;
  std::memcpy(buf.data(), &h, sizeof h);
  for (int64_t l = 0; l < count; ++l) {
    StackEntry e{};
    e.x = d[l].x;
    e.W = static_cast<const u32x4*>(d[l].wpacked);
    e.beta = d[l].beta;
    e.y = d[l].y;
    e.beta_len = d[l].beta_len;
    e.N = d[l].N;
    e.K = d[l].K;
    const uintptr_t xa = reinterpret_cast<uintptr_t>(d[l].x);
    const uintptr_t xb = xa + static_cast<uintptr_t>(M * d[l].K * 2);
    for (int64_t j = 0; j < l && !e.raw; ++j) {
      const uintptr_t ya = reinterpret_cast<uintptr_t>(d[j].y);
      const uintptr_t yb = ya + static_cast<uintptr_t>(M * d[j].N * 4);
      if (ya < xb && xa < yb) e.raw = 1;
    }
    std::memcpy(buf.data() + sizeof(StackHeader) + l * sizeof(StackEntry), &e, sizeof e);
  }
  hipError_t err = hipMemcpyAsync(plan, buf.data(), buf.size(), hipMemcpyHostToDevice, s);
  if (err != hipSuccess) return err;
  return hipStreamSynchronize(s);
}

namespace {
template <int MR>
hipError_t launch_stack_mr(const void* plan, int count, uint32_t* bar, uint64_t* ws_acc,
                           hipStream_t s) {
  // persistent grid: every workgroup must be resident at once (cooperative launch); one per
  // CU, or BL_STACK_GRID workgroups if that is set and smaller
  // grid per device, computed once; calling threads may race to fill a slot, and every one
  // of them computes the same value, so relaxed atomics suffice
  static std::atomic<int> cached[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  int grid = (dev >= 0 && dev < 64) ? cached[dev].load(std::memory_order_relaxed) : 0;
  if (grid == 0) {
    int cus = 0, per_cu = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &per_cu, reinterpret_cast<const void*>(&gemv_stack_kernel<MR>), 64 * kSW, 0);
    if (e != hipSuccess) return e;
    if (per_cu < 1 || cus < 1) return hipErrorCooperativeLaunchTooLarge;
    grid = cus;   // per_cu >= 1: one workgroup per CU is resident
    if (dev >= 0 && dev < 64) cached[dev].store(grid, std::memory_order_relaxed);
  }
  grid = std::min(grid, kMaxStackGrid);
  if (const char* env = std::getenv("BL_STACK_GRID")) {
    const long v = std::strtol(env, nullptr, 10);
    if (v > 0 && v < grid) grid = static_cast<int>(v);
  }
  StackHeader* hdr = static_cast<StackHeader*>(const_cast<void*>(plan));
  void* args[] = {&hdr, &bar, &ws_acc, &count};
  return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&gemv_stack_kernel<MR>),
                                    dim3(static_cast<unsigned>(grid)), dim3(64 * kSW), args, 0, s);
}
}  // namespace

size_t stack_barrier_words() { return kBarWords; }

hipError_t launch_gemv_stack(const void* plan, int64_t count, int64_t M, uint32_t* bar,
                             uint64_t* ws_acc, hipStream_t s) {
  const int c = static_cast<int>(count);
  switch (M) {
    case 1: return launch_stack_mr<1>(plan, c, bar, ws_acc, s);
    case 2: return launch_stack_mr<2>(plan, c, bar, ws_acc, s);
    case 3: return launch_stack_mr<3>(plan, c, bar, ws_acc, s);
    case 4: return launch_stack_mr<4>(plan, c, bar, ws_acc, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t stack_read_status(const void* plan, uint32_t* status, hipStream_t s) {
  const StackHeader* hdr = static_cast<const StackHeader*>(plan);
  hipError_t e = hipMemcpyAsync(status, &hdr->status, 4, hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return e;
  return hipStreamSynchronize(s);
}

}  // namespace bl
