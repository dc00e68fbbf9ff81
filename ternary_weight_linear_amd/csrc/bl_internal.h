// Internal declarations shared by the libbitlinear translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "libbitlinear.h"

namespace bl {

constexpr int kQb = 127;               // activation range [-127, 127]
constexpr int kAbsmeanBlocks = 1024;   // partial histograms of the exact absmean sum
constexpr int kAbsmeanBins = 256;      // one bin per fp32 exponent field value

// Carve-up of the caller's workspace. Every region starts 256-byte aligned.
// cnt and acc sit at fixed offsets for every shape, must be zero on entry and are left
// zero by every call; the regions after them are scratch that any call may overwrite.
// Fixed positions keep one shape's scratch from ever landing on another shape's
// zero-maintained region when a workspace is shared.
constexpr int64_t kMaxCounters = 65536;          // completion counters (256 KiB)
constexpr int64_t kAccCap = int64_t(64) * 65536; // 64-bit split-K words (32 MiB)
constexpr int32_t kSplitOffset = int32_t(1) << 23;  // bias that keeps split partials >= 0
// Integer split-K is used only when every partial fits |p| < kSplitOffset (127 * K below
// this bound) and at most kMaxIntSplits partials meet in one word.
constexpr int64_t kMaxIntSplitK = (int64_t(1) << 23) / 127;
constexpr int kMaxIntSplits = 255;
struct WsLayout {
  size_t cnt_off, cnt_bytes;       // uint32 completion counters, one per output tile
  size_t acc_off, acc_bytes;       // uint64 [M, N] split-K words (see split_arrive)
  size_t part_off, part_bytes;     // fp32 [KS, M, N] split-K partial sums (fp16-input paths)
  size_t bins_off, bins_bytes;     // uint64 [kAbsmeanBlocks, 256] + flag (absmean)
  size_t q_off, q_bytes;           // int8 [M, K] activations (forward)
  size_t planes_off, planes_bytes; // X8-64 planes [M*K bytes] (forward)
  size_t gamma_off, gamma_bytes;   // fp32 [M] (forward)
  size_t rowsum_off, rowsum_bytes; // int32 [M] (forward from T2-MF64 weights)
  size_t svid_off, svid_bytes;     // fp32 power-iteration vectors (SVID)
  size_t total;
};
WsLayout ws_layout(int64_t M, int64_t N, int64_t K);

// fp32 split-K partials of the OneBit forward for a shape (fix the workspace size).
size_t onebit_part_floats(int64_t M, int64_t N, int64_t K);
// fp32 split-K partials of the residual-binarisation forward for a shape.
size_t residual_part_floats(int64_t M, int64_t N, int64_t K);

// ---- launchers (all asynchronous on `s`) -----------------------------------------------
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);

hipError_t launch_pack_ternary(const int8_t* codes, int64_t N, int64_t K, void* packed,
                               int32_t* n_invalid, hipStream_t s);
hipError_t launch_unpack_ternary(const void* packed, int64_t N, int64_t K, int8_t* codes,
                                 int32_t* n_invalid, hipStream_t s);
// T2-MF64 (the matrix-core layout) from codes, or from T2-PN-64 bytes.
hipError_t launch_pack_ternary_mf(const int8_t* codes, int64_t N, int64_t K, void* packed,
                                  int32_t* n_invalid, hipStream_t s);
hipError_t launch_repack_pn_to_mf(const void* pn, int64_t N, int64_t K, void* mf,
                                  int32_t* n_invalid, hipStream_t s);
hipError_t launch_pack_sign(const float* W, int64_t N, int64_t K, void* packed, hipStream_t s);
hipError_t launch_unpack_sign(const void* packed, int64_t N, int64_t K, int8_t* signs,
                              hipStream_t s);
hipError_t launch_ternarize_absmean(const float* W, int64_t N, int64_t K, int8_t* codes,
                                    void* packed, float* beta, unsigned long long* bins,
                                    hipStream_t s);

hipError_t launch_quant_act(const uint16_t* x, int64_t M, int64_t K, int8_t* q, float* gamma,
                            int32_t* rowsum, uint32_t* planes, hipStream_t s);

// y != nullptr: fp32 epilogue into y; acc_out != nullptr: raw int32 accumulators.
hipError_t launch_gemv(const uint32_t* planes, const float* gamma, int M, int64_t K,
                       const void* wpacked, const float* beta, int64_t beta_len, int64_t N,
                       float* y, int32_t* acc_out, uint64_t* ws_acc, uint32_t* ws_cnt,
                       hipStream_t s);
// SVID: rank-1 power iteration on |W| (scratch = svid_scratch_floats(N, K) floats).
size_t svid_scratch_floats(int64_t N, int64_t K);
hipError_t launch_svid(const float* W, int64_t N, int64_t K, int iters, uint16_t* g, uint16_t* h,
                       float* sigma, float* scratch, hipStream_t s);

// Quantise fp16 x inside the GEMV (no separate quantiser launch); M <= 4.
hipError_t launch_gemv_fused(const uint16_t* x, int M, int64_t K, const void* wpacked,
                             const float* beta, int64_t beta_len, int64_t N, float* y,
                             uint64_t* ws_acc, uint32_t* ws_cnt, hipStream_t s);
hipError_t launch_gemm(const int8_t* q, const float* gamma, int64_t M, int64_t K,
                       const void* wpacked, const float* beta, int64_t beta_len, int64_t N,
                       float* y, int32_t* acc_out, uint64_t* ws_acc, hipStream_t s);
// Residual binarisation: two S1-128 sign planes plus fp32 scales [N, K/128] per plane.
hipError_t launch_residual_binarize(const float* W, int64_t N, int64_t K, void* planes_o,
                                    float* alpha_o, void* planes_r, float* alpha_r,
                                    hipStream_t s);
hipError_t launch_residual_linear(const uint16_t* x, const void* planes_o, const float* alpha_o,
                                  const void* planes_r, const float* alpha_r, int64_t M, int64_t N,
                                  int64_t K, float* y, float* ws_part, uint32_t* ws_cnt,
                                  hipStream_t s);
// Weight-streaming ternary GEMM (int8 matrix cores, expansion in registers); M * K < 2^31.
hipError_t launch_tern_mfma(const int8_t* q, const float* gamma, int64_t M, int64_t K,
                            const void* wpacked, const float* beta, int64_t beta_len, int64_t N,
                            float* y, int32_t* acc_out, uint64_t* ws_acc, hipStream_t s);
// Whole-stack decode (stack.hip): the device plan of a list of linears, its persistent
// launch (barrier = a zero-maintained counter, ws_acc the split words) and its status word.
size_t stack_plan_bytes(int64_t count);
hipError_t stack_write_plan(const bl_linear_desc* linears, int64_t count, int64_t M, void* plan,
                            hipStream_t s);
hipError_t launch_gemv_stack(const void* plan, int64_t count, int64_t M, uint32_t* bar,
                             uint64_t* ws_acc, hipStream_t s);
size_t stack_barrier_words();   // zero-maintained uint32 words of the grid-wide wait
hipError_t stack_read_status(const void* plan, uint32_t* status, hipStream_t s);
// Ternary GEMM from T2-MF64 weights (int8 matrix cores; rowsum = sum_k q[m, k]); any M,
// built for M <= 64; M * K < 2^31, K <= 65536.
hipError_t launch_tern_mf(const int8_t* q, const float* gamma, const int32_t* rowsum, int64_t M,
                          int64_t K, const void* wmf, const float* beta, int64_t beta_len,
                          int64_t N, float* y, int32_t* acc_out, uint64_t* ws_acc, hipStream_t s);
// Fused quantise + product from T2-MF64 weights for M <= 16 (K <= 32768) where
// mf_decode_fits (a workgroup's K range must fit in LDS).
bool mf_decode_fits(int64_t M, int64_t N, int64_t K);
hipError_t launch_mf_decode(const uint16_t* x, int M, int64_t K, const void* wmf,
                            const float* beta, int64_t beta_len, int64_t N, float* y,
                            uint64_t* ws_acc, hipStream_t s);
// The same product from q given (quantiser outputs), M <= 16 where mf_decode_fits; raw int32
// outputs into acc_out and/or the fp32 epilogue into y.
bool mf_qgemv_fits(int64_t M, int64_t N, int64_t K);
hipError_t launch_mf_qgemv(const int8_t* q, const float* gamma, const int32_t* rowsum, int M,
                           int64_t K, const void* wmf, const float* beta, int64_t beta_len,
                           int64_t N, float* y, int32_t* acc_out, uint64_t* ws_acc,
                           hipStream_t s);
hipError_t launch_onebit(const uint16_t* x, const uint16_t* g, const void* spacked,
                         const uint16_t* h, int64_t M, int64_t N, int64_t K, float* y,
                         float* ws_part, uint32_t* ws_cnt, hipStream_t s);

// ---- device helpers ---------------------------------------------------------------------
__device__ __forceinline__ float half_bits_to_float(uint16_t b) {
  return static_cast<float>(__builtin_bit_cast(_Float16, b));
}

// q = rint(a / g) for a = x * 127 (exact in fp32) and |a| <= 127 g, decided on the correctly
// rounded fp32 quotient. d = a * rcp(g) is within 3.1e-5 of that quotient (rcp 1 ulp, product
// 0.5 ulp, |a / g| <= 127), so the two round to the same integer unless a half-integer lies
// within that distance of d; such inputs (fractional part within 2^-12 of 1/2) take the IEEE
// division instead (behind a wave-uniform test, so that the common case skips it).
__device__ __forceinline__ int quant_q(float a, float g, float rg) {
  float d = a * rg;
  const bool near = fabsf(__builtin_amdgcn_fractf(d) - 0.5f) < 0x1p-12f;
  if (__ballot(near) != 0) {
    float gv = g;
    asm volatile("" : "+v"(gv));   // keeps the division inside the branch (no speculation)
    const float e = a / gv;
    d = near ? e : d;
  }
  return static_cast<int>(__builtin_amdgcn_fmed3f(rintf(d), -127.0f, 127.0f));
}

// quant_q for N inputs at once (input e of row gamma g[e], rg[e] = rcp(g[e]); zero[e]: the
// row's gamma is 0 or not finite, q = 0). The distances of the N quotients from the nearest
// half-integer are folded into one minimum, so one compare and one wave-uniform test cover
// them all and the common case is straight-line VALU code (quant_q per input under a
// per-row select compiles into a masked branch per input). A zero row clamps to [0, 0]
// (med3 of a NaN and two zeros is zero). Same results as quant_q input by input.
template <int N>
__device__ __forceinline__ void quant_q_n(const float (&a)[N], const float (&g)[N],
                                          const float (&rg)[N], const bool (&zero)[N],
                                          int (&q)[N]) {
  float d[N], t[N];
#pragma unroll
  for (int e = 0; e < N; ++e) {
    d[e] = a[e] * rg[e];
    t[e] = fabsf(__builtin_amdgcn_fractf(d[e]) - 0.5f);
  }
  float tmin = t[0];
#pragma unroll
  for (int e = 1; e < N; ++e) tmin = fminf(tmin, t[e]);
  if (__ballot(tmin < 0x1p-12f) != 0) {
#pragma unroll
    for (int e = 0; e < N; ++e) {
      float gv = g[e];
      asm volatile("" : "+v"(gv));   // keeps the division inside the branch
      const float div = a[e] / gv;
      d[e] = t[e] < 0x1p-12f ? div : d[e];
    }
  }
#pragma unroll
  for (int e = 0; e < N; ++e) {
    const float lim = zero[e] ? 0.0f : 127.0f;
    q[e] = static_cast<int>(__builtin_amdgcn_fmed3f(rintf(d[e]), -lim, lim));
  }
}

// Maximum over the 64 lanes of a wave, returned to every lane: DPP steps within quads,
// half rows and rows, then the row broadcasts (lane 15 -> row 1 and 3, lane 31 -> rows 2
// and 3), leaving the maximum in lane 63. Lanes a step does not write keep their own value.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  auto step = [](uint32_t a, uint32_t b) { return a > b ? a : b; };
  v = step(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(v), static_cast<int>(v), 0xB1, 0xF, 0xF, false)));
  v = step(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(v), static_cast<int>(v), 0x4E, 0xF, 0xF, false)));
  v = step(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(v), static_cast<int>(v), 0x141, 0xF, 0xF, false)));
  v = step(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(v), static_cast<int>(v), 0x140, 0xF, 0xF, false)));
  v = step(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(v), static_cast<int>(v), 0x142, 0xA, 0xF, false)));
  v = step(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(v), static_cast<int>(v), 0x143, 0xC, 0xF, false)));
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63));
}

// Sum over each group of eight lanes 8k .. 8k + 7, returned to every lane of the group
// (DPP: pairs, quads, then the mirrored half row).
__device__ __forceinline__ int group8_sum_i32(int v) {
  v += __builtin_amdgcn_update_dpp(v, v, 0xB1, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(v, v, 0x4E, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(v, v, 0x141, 0xF, 0xF, false);
  return v;
}

// Sum over the 64 lanes of a wave, returned to every lane: the eight-lane sums, then the
// mirrored row, then the row broadcasts into lanes of rows 1, 3 and 2, 3 (lanes a broadcast
// does not write add 0), leaving the total in lane 63.
__device__ __forceinline__ int wave_sum_i32(int v) {
  v = group8_sum_i32(v);
  v += __builtin_amdgcn_update_dpp(v, v, 0x140, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);
  return __builtin_amdgcn_readlane(v, 63);
}

// popcount(x) + acc in one v_bcnt_u32_b32 (its second operand accumulates). Written out:
// the compiler sums pairs of popcounts with a three-input add instead, one more VALU op
// per pair in the add-only loops.
__device__ __forceinline__ uint32_t bcnt_acc(uint32_t x, uint32_t acc) {
  uint32_t r;
  asm("v_bcnt_u32_b32 %0, %1, %2" : "=v"(r) : "v"(x), "v"(acc));
  return r;
}

// Split-K hand-off between workgroups without cache write-back fences.
// Partial results move only through agent-scope atomics, which the hardware performs at
// the device-wide coherence point rather than in one XCD's L2, so no L2 write-back or
// invalidate is needed (a __threadfence() here costs tens of microseconds per launch).
// A workgroup waits for its own atomics to complete (s_waitcnt 0) before it increments
// the tile's completion counter; the workgroup that sees count == nsplit - 1 reads the
// totals back with atomic exchanges, which also restore the workspace to zero.
__device__ __forceinline__ void atomic_add_agent(int32_t* p, int32_t v) {
  __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void atomic_store_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float atomic_load_agent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t atomic_take_agent(int32_t* p) {
  return __hip_atomic_exchange(p, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// One-round-trip split-K reduction of one int32 output element. The workspace word holds
// (number of arrivals << 32) + sum of (partial + kSplitOffset); each contributor adds its
// share with one returning atomic at the device coherence point. The contributor whose
// add brings the count to nsplit is the last one: it alone gets true, reads the exact total
// from the returned value (no further round trip, no fence) and clears the word.
__device__ __forceinline__ bool split_arrive(uint64_t* word, int32_t partial, int nsplit,
                                             int32_t* total) {
  const uint64_t add = (uint64_t(1) << 32) + static_cast<uint32_t>(partial + kSplitOffset);
  const uint64_t now =
      __hip_atomic_fetch_add(word, add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + add;
  if ((now >> 32) != static_cast<uint64_t>(nsplit)) return false;
  *total = static_cast<int32_t>(static_cast<uint32_t>(now) -
                                static_cast<uint32_t>(nsplit) * static_cast<uint32_t>(kSplitOffset));
  __hip_atomic_store(word, uint64_t(0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

// split_arrive for kN outputs of one lane with one round trip: every add is issued before
// any returned word is examined (testing each result before the next add would serialise
// the round trips). word(e) gives element e's split word (called again for the reset, so
// no pointers stay live); element e takes part iff bit e of `active`, and word(e) must be a
// valid split word either way (an inactive element adds 0, which changes nothing, so that
// no add sits behind a branch of its own). The result has bit e set where this lane
// brought the count to nsplit, v[e] then holding the exact total (and the word cleared).
template <int kN, class WordFn>
__device__ __forceinline__ uint32_t split_arrive_batch(WordFn word, int32_t (&v)[kN],
                                                       uint32_t active, int nsplit) {
  if (active == 0) return 0;
  uint64_t now[kN];
#pragma unroll
  for (int e = 0; e < kN; ++e) {
    const uint64_t add = ((active >> e) & 1u)
                             ? (uint64_t(1) << 32) + static_cast<uint32_t>(v[e] + kSplitOffset)
                             : uint64_t(0);
    now[e] = __hip_atomic_fetch_add(word(e), add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + add;
  }
  uint32_t last = 0;
#pragma unroll
  for (int e = 0; e < kN; ++e) {
    if (((active >> e) & 1u) && (now[e] >> 32) == static_cast<uint64_t>(nsplit)) {
      v[e] = static_cast<int32_t>(static_cast<uint32_t>(now[e]) -
                                  static_cast<uint32_t>(nsplit) * static_cast<uint32_t>(kSplitOffset));
      __hip_atomic_store(word(e), uint64_t(0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      last |= 1u << e;
    }
  }
  return last;
}

// split_arrive_batch for two outputs per word (output pair e = elements 2e, 2e + 1 of v), for
// at most kMaxPairSplits partials of |p| < kSplitOffset: the word holds the arrival count
// in bits 54.., and the two sums of (partial + kSplitOffset) in bits 27..53 and 0..26 (each
// below 8 * 2^24 = 2^27, so neither carries into the next field). Half the atomics of one
// word per output, still one round trip. Bit e of `active`: pair e takes part (both of its
// elements are added; an unused second element adds a bias nobody reads); word(e) must be
// valid for every e. Returns bit e set where this lane completed pair e, v[2e] and v[2e + 1]
// then holding the exact totals (and the word cleared).
constexpr int kMaxPairSplits = 8;
template <int kP, class WordFn>
__device__ __forceinline__ uint32_t split_arrive_pairs(WordFn word, int32_t (&v)[2 * kP],
                                                       uint32_t active, int nsplit) {
  if (active == 0) return 0;
  constexpr uint64_t kField = (uint64_t(1) << 27) - 1;
  uint64_t now[kP];
#pragma unroll
  for (int e = 0; e < kP; ++e) {
    const uint64_t add =
        ((active >> e) & 1u)
            ? (uint64_t(1) << 54) |
                  (static_cast<uint64_t>(static_cast<uint32_t>(v[2 * e + 1] + kSplitOffset)) << 27) |
                  static_cast<uint64_t>(static_cast<uint32_t>(v[2 * e] + kSplitOffset))
            : uint64_t(0);
    now[e] = __hip_atomic_fetch_add(word(e), add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + add;
  }
  uint32_t last = 0;
  const uint32_t bias = static_cast<uint32_t>(nsplit) * static_cast<uint32_t>(kSplitOffset);
#pragma unroll
  for (int e = 0; e < kP; ++e) {
    if (((active >> e) & 1u) && (now[e] >> 54) == static_cast<uint64_t>(nsplit)) {
      v[2 * e] = static_cast<int32_t>(static_cast<uint32_t>(now[e] & kField) - bias);
      v[2 * e + 1] = static_cast<int32_t>(static_cast<uint32_t>((now[e] >> 27) & kField) - bias);
      __hip_atomic_store(word(e), uint64_t(0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      last |= 1u << e;
    }
  }
  return last;
}

// Wait until every memory operation this thread issued has completed, and keep the
// compiler from moving memory operations across the wait.
__device__ __forceinline__ void wait_own_memory_ops() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
// Increment a completion counter; returns the previous count.
__device__ __forceinline__ uint32_t arrive_agent(uint32_t* cnt) {
  return __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void reset_agent(uint32_t* cnt) {
  __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace bl
