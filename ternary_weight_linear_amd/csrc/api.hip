// The C ABI of libbitlinear: host-side argument checks, workspace carve-up and dispatch.
// Every check runs before anything is queued; see include/libbitlinear.h for the contract.
#include <algorithm>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "bl_internal.h"

namespace bl {
namespace {

thread_local char g_last_error[256] = "";

int hip_fail(hipError_t e, const char* where) {
  std::snprintf(g_last_error, sizeof(g_last_error), "%s: %s (%d)", where, hipGetErrorString(e),
                static_cast<int>(e));
  return BL_ERR_HIP;
}

inline int check_launch(hipError_t e, const char* where) {
  return e == hipSuccess ? BL_OK : hip_fail(e, where);
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline size_t round256(size_t b) { return (b + 255) & ~size_t(255); }

// Half-open byte ranges [a, a + na) and [b, b + nb) intersect.
inline bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || !na || !nb) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

constexpr int64_t kMaxDim = int64_t(1) << 30;
constexpr int64_t kMaxMtiles = 65535;     // 16-row tiles of x along the grid's y dimension
constexpr int64_t kMaxSignK = int64_t(1) << 26;   // fp16-input kernels use 32-bit row offsets
constexpr int64_t kMaxStack = 4096;               // linears in one stack plan

inline bool dims_ok(int64_t M, int64_t N, int64_t K) {
  return M >= 1 && N >= 1 && K >= 1 && M <= kMaxDim && N <= kMaxDim && K <= kMaxDim;
}

}  // namespace

WsLayout ws_layout(int64_t M, int64_t N, int64_t K) {
  WsLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes, size_t& o, size_t& b) {
    o = off;
    b = round256(bytes);
    off += b;
  };
  take(static_cast<size_t>(kMaxCounters) * 4, L.cnt_off, L.cnt_bytes);
  take(static_cast<size_t>(kAccCap) * 8, L.acc_off, L.acc_bytes);
  take(std::max(onebit_part_floats(M, N, K), residual_part_floats(M, N, K)) * 4, L.part_off,
       L.part_bytes);
  take(static_cast<size_t>(kAbsmeanBlocks) * kAbsmeanBins * 8, L.bins_off, L.bins_bytes);
  take(static_cast<size_t>(M) * K, L.q_off, L.q_bytes);
  take(static_cast<size_t>(M) * K, L.planes_off, L.planes_bytes);
  take(static_cast<size_t>(M) * 4, L.gamma_off, L.gamma_bytes);
  take(static_cast<size_t>(M) * 4, L.rowsum_off, L.rowsum_bytes);
  take(svid_scratch_floats(N, K) * 4, L.svid_off, L.svid_bytes);
  L.total = off;
  return L;
}

}  // namespace bl

using namespace bl;

namespace {

// Common checks of the ternary product entry points. Returns BL_OK or a status.
int check_ternary_product(int64_t M, int64_t K, const void* wpacked, int64_t N,
                          const float* gamma, void* ws, size_t ws_bytes) {
  if (!wpacked || !gamma) return BL_ERR_NULL;
  if (!dims_ok(M, N, K) || N % 64 || K % 64 || 127 * K >= (int64_t(1) << 31)) return BL_ERR_SHAPE;
  if (!aligned16(wpacked)) return BL_ERR_ALIGN;
  if (!ws || ws_bytes < ws_layout(M, N, K).total) return BL_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return BL_ERR_ALIGN;
  return BL_OK;
}

int check_beta(const float* beta, int64_t beta_len, int64_t N) {
  if (!beta) return BL_ERR_NULL;
  if (beta_len != 1 && beta_len != N) return BL_ERR_ARG;
  return BL_OK;
}

// ---- library-owned scratch for callers that cannot allocate --------------------------
// The split-K words of the fused decode GEMV (one uint64 per output, zero between calls)
// for bl_bitlinear_forward_gemv_noalloc. Each GPU holds its own copy of the array; host code
// must use the device address that hipGetSymbolAddress returns, never the array's name.
constexpr int64_t kScratchWords = int64_t(1) << 18;   // M * N <= 262144 outputs, 2 MiB
static __device__ __align__(256) uint64_t scratch[kScratchWords];
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
uint64_t* g_scratch_ptr[kScratchDevices] = {};

// Device address of the current device's scratch. The first call on a device looks the
// address up and queues one zero fill on `s` (every call leaves the words zero again).
int scratch_words(hipStream_t s, uint64_t** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "bl_bitlinear_forward_gemv_noalloc (hipGetDevice)");
  if (dev < 0 || dev >= kScratchDevices) return BL_ERR_ARG;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol,
                      "bl_bitlinear_forward_gemv_noalloc (hipGetSymbolAddress)");
    e = launch_fill_zero(p, sizeof(uint64_t) * kScratchWords, s);
    if (e != hipSuccess) return hip_fail(e, "bl_bitlinear_forward_gemv_noalloc (clear)");
    g_scratch_ptr[dev] = static_cast<uint64_t*>(p);
  }
  *out = g_scratch_ptr[dev];
  return BL_OK;
}

}  // namespace

extern "C" {

const char* bl_status_string(int status) {
  switch (status) {
    case BL_OK: return "ok";
    case BL_ERR_NULL: return "a required pointer is NULL";
    case BL_ERR_SHAPE: return "a size is out of range or not a multiple its layout needs";
    case BL_ERR_ALIGN: return "a pointer lacks the alignment its loads need";
    case BL_ERR_ALIAS: return "an output buffer overlaps another buffer";
    case BL_ERR_WORKSPACE: return "workspace missing or smaller than bl_workspace_bytes()";
    case BL_ERR_HIP: return "a HIP call failed (see bl_last_error)";
    case BL_ERR_ARG: return "invalid argument";
    case BL_ERR_CAPACITY:
      return "the shape exceeds the fixed capacity of the library's own scratch (M * N <= 262144)";
    default: return "unknown status";
  }
}

const char* bl_last_error(void) { return g_last_error; }

int bl_version(void) { return 10000; }

size_t bl_ternary_packed_bytes(int64_t N, int64_t K) {
  if (!dims_ok(1, N, K) || N % 64 || K % 64) return 0;
  return static_cast<size_t>(N) * K / 4;
}

size_t bl_sign_packed_bytes(int64_t N, int64_t K) {
  if (!dims_ok(1, N, K) || N % 64 || K % 128) return 0;
  return static_cast<size_t>(N) * K / 8;
}

size_t bl_act_planes_bytes(int64_t M, int64_t K) {
  if (!dims_ok(M, 1, K) || K % 64) return 0;
  return static_cast<size_t>(M) * K;
}

size_t bl_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (!dims_ok(M, N, K)) return 0;
  return ws_layout(M, N, K).total;
}

int bl_workspace_clear(void* ws, size_t bytes, void* stream) {
  if (!ws) return BL_ERR_NULL;
  return check_launch(launch_fill_zero(ws, bytes, static_cast<hipStream_t>(stream)),
                      "bl_workspace_clear");
}

int bl_ternarize_absmean(const float* W, int64_t N, int64_t K, int8_t* codes, void* packed,
                         float* beta, void* ws, size_t ws_bytes, void* stream) {
  if (!W || !beta || (!codes && !packed)) return BL_ERR_NULL;
  if (!dims_ok(1, N, K) || N % 64 || K % 64 || N * K >= (int64_t(1) << 32)) return BL_ERR_SHAPE;
  if (!aligned16(W) || (codes && !aligned16(codes)) || (packed && !aligned16(packed)))
    return BL_ERR_ALIGN;
  const WsLayout L = ws_layout(1, N, K);
  if (!ws || ws_bytes < L.total) return BL_ERR_WORKSPACE;
  const size_t wb = static_cast<size_t>(N) * K * 4;
  if (overlap(codes, N * K, W, wb) || overlap(packed, N * K / 4, W, wb) ||
      overlap(codes, N * K, packed, N * K / 4) || overlap(beta, 4, W, wb) ||
      overlap(beta, 4, codes, N * K) || overlap(beta, 4, packed, N * K / 4))
    return BL_ERR_ALIAS;
  auto* bins = reinterpret_cast<unsigned long long*>(static_cast<char*>(ws) + L.bins_off);
  return check_launch(launch_ternarize_absmean(W, N, K, codes, packed, beta, bins,
                                               static_cast<hipStream_t>(stream)),
                      "bl_ternarize_absmean");
}

int bl_pack_ternary(const int8_t* codes, int64_t N, int64_t K, void* packed, int32_t* n_invalid,
                    void* stream) {
  if (!codes || !packed) return BL_ERR_NULL;
  if (!dims_ok(1, N, K) || N % 64 || K % 64) return BL_ERR_SHAPE;
  if (!aligned16(codes) || !aligned16(packed)) return BL_ERR_ALIGN;
  if (overlap(codes, N * K, packed, N * K / 4) || overlap(n_invalid, 4, packed, N * K / 4))
    return BL_ERR_ALIAS;
  return check_launch(launch_pack_ternary(codes, N, K, packed, n_invalid,
                                          static_cast<hipStream_t>(stream)),
                      "bl_pack_ternary");
}

int bl_unpack_ternary(const void* packed, int64_t N, int64_t K, int8_t* codes, int32_t* n_invalid,
                      void* stream) {
  if (!codes || !packed) return BL_ERR_NULL;
  if (!dims_ok(1, N, K) || N % 64 || K % 64) return BL_ERR_SHAPE;
  if (!aligned16(codes) || !aligned16(packed)) return BL_ERR_ALIGN;
  if (overlap(codes, N * K, packed, N * K / 4) || overlap(n_invalid, 4, codes, N * K))
    return BL_ERR_ALIAS;
  return check_launch(launch_unpack_ternary(packed, N, K, codes, n_invalid,
                                            static_cast<hipStream_t>(stream)),
                      "bl_unpack_ternary");
}

int bl_pack_ternary_mf(const int8_t* codes, int64_t N, int64_t K, void* packed,
                       int32_t* n_invalid, void* stream) {
  if (!codes || !packed) return BL_ERR_NULL;
  if (!dims_ok(1, N, K) || N % 64 || K % 64) return BL_ERR_SHAPE;
  if (!aligned16(codes) || !aligned16(packed)) return BL_ERR_ALIGN;
  if (overlap(codes, N * K, packed, N * K / 4) || overlap(n_invalid, 4, packed, N * K / 4))
    return BL_ERR_ALIAS;
  return check_launch(launch_pack_ternary_mf(codes, N, K, packed, n_invalid,
                                             static_cast<hipStream_t>(stream)),
                      "bl_pack_ternary_mf");
}

int bl_repack_ternary_mf(const void* t2pn, int64_t N, int64_t K, void* mf, int32_t* n_invalid,
                         void* stream) {
  if (!t2pn || !mf) return BL_ERR_NULL;
  if (!dims_ok(1, N, K) || N % 64 || K % 64) return BL_ERR_SHAPE;
  if (!aligned16(t2pn) || !aligned16(mf)) return BL_ERR_ALIGN;
  if (overlap(t2pn, N * K / 4, mf, N * K / 4) || overlap(n_invalid, 4, mf, N * K / 4))
    return BL_ERR_ALIAS;
  return check_launch(launch_repack_pn_to_mf(t2pn, N, K, mf, n_invalid,
                                             static_cast<hipStream_t>(stream)),
                      "bl_repack_ternary_mf");
}

int bl_pack_sign(const float* W, int64_t N, int64_t K, void* packed, void* stream) {
  if (!W || !packed) return BL_ERR_NULL;
  if (!dims_ok(1, N, K) || N % 64 || K % 128) return BL_ERR_SHAPE;
  if (!aligned16(W) || !aligned16(packed)) return BL_ERR_ALIGN;
  if (overlap(W, static_cast<size_t>(N) * K * 4, packed, N * K / 8)) return BL_ERR_ALIAS;
  return check_launch(launch_pack_sign(W, N, K, packed, static_cast<hipStream_t>(stream)),
                      "bl_pack_sign");
}

int bl_unpack_sign(const void* packed, int64_t N, int64_t K, int8_t* signs, void* stream) {
  if (!signs || !packed) return BL_ERR_NULL;
  if (!dims_ok(1, N, K) || N % 64 || K % 128) return BL_ERR_SHAPE;
  if (!aligned16(signs) || !aligned16(packed)) return BL_ERR_ALIGN;
  if (overlap(signs, N * K, packed, N * K / 8)) return BL_ERR_ALIAS;
  return check_launch(launch_unpack_sign(packed, N, K, signs, static_cast<hipStream_t>(stream)),
                      "bl_unpack_sign");
}

int bl_quant_act_int8(const uint16_t* x, int64_t M, int64_t K, int8_t* q, float* gamma,
                      int32_t* rowsum, uint32_t* planes, void* stream) {
  if (!x || !gamma || (!q && !planes)) return BL_ERR_NULL;
  if (!dims_ok(M, 1, K) || K % 64 || K > 28672 || M > (int64_t(1) << 24)) return BL_ERR_SHAPE;
  if (!aligned16(x) || (q && !aligned16(q)) || (planes && !aligned16(planes))) return BL_ERR_ALIGN;
  const size_t xb = static_cast<size_t>(M) * K * 2, qb = static_cast<size_t>(M) * K;
  const void* outs[4] = {q, gamma, rowsum, planes};
  const size_t outb[4] = {qb, static_cast<size_t>(M) * 4, static_cast<size_t>(M) * 4, qb};
  for (int i = 0; i < 4; ++i) {
    if (overlap(outs[i], outb[i], x, xb)) return BL_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outb[i], outs[j], outb[j])) return BL_ERR_ALIAS;
  }
  return check_launch(launch_quant_act(x, M, K, q, gamma, rowsum, planes,
                                       static_cast<hipStream_t>(stream)),
                      "bl_quant_act_int8");
}

int bl_bitlinear_gemv(const uint32_t* planes, const float* gamma, int64_t M, int64_t K,
                      const void* wpacked, const float* beta, int64_t beta_len, int64_t N,
                      float* y, void* ws, size_t ws_bytes, void* stream) {
  if (!planes || !y) return BL_ERR_NULL;
  if (M > 4) return BL_ERR_SHAPE;
  int st = check_ternary_product(M, K, wpacked, N, gamma, ws, ws_bytes);
  if (st) return st;
  if ((st = check_beta(beta, beta_len, N))) return st;
  if (!aligned16(planes)) return BL_ERR_ALIGN;
  const size_t yb = static_cast<size_t>(M) * N * 4;
  if (overlap(y, yb, planes, M * K) || overlap(y, yb, wpacked, N * K / 4) ||
      overlap(y, yb, gamma, M * 4) || overlap(y, yb, beta, beta_len * 4) ||
      overlap(y, yb, ws, ws_bytes))
    return BL_ERR_ALIAS;
  const WsLayout L = ws_layout(M, N, K);
  char* w = static_cast<char*>(ws);
  return check_launch(launch_gemv(planes, gamma, static_cast<int>(M), K, wpacked, beta, beta_len,
                                  N, y, nullptr, reinterpret_cast<uint64_t*>(w + L.acc_off),
                                  reinterpret_cast<uint32_t*>(w + L.cnt_off),
                                  static_cast<hipStream_t>(stream)),
                      "bl_bitlinear_gemv");
}

int bl_bitlinear_gemm(const int8_t* q, const float* gamma, int64_t M, int64_t K,
                      const void* wpacked, const float* beta, int64_t beta_len, int64_t N,
                      float* y, void* ws, size_t ws_bytes, void* stream) {
  if (!q || !y) return BL_ERR_NULL;
  int st = check_ternary_product(M, K, wpacked, N, gamma, ws, ws_bytes);
  if (st) return st;
  if ((st = check_beta(beta, beta_len, N))) return st;
  if (!aligned16(q)) return BL_ERR_ALIGN;
  const size_t yb = static_cast<size_t>(M) * N * 4;
  if (overlap(y, yb, q, M * K) || overlap(y, yb, wpacked, N * K / 4) ||
      overlap(y, yb, gamma, M * 4) || overlap(y, yb, beta, beta_len * 4) ||
      overlap(y, yb, ws, ws_bytes))
    return BL_ERR_ALIAS;
  const WsLayout L = ws_layout(M, N, K);
  char* w = static_cast<char*>(ws);
  return check_launch(launch_gemm(q, gamma, M, K, wpacked, beta, beta_len, N, y, nullptr,
                                  reinterpret_cast<uint64_t*>(w + L.acc_off),
                                  static_cast<hipStream_t>(stream)),
                      "bl_bitlinear_gemm");
}

int bl_bitlinear_gemm_mf(const int8_t* q, const float* gamma, const int32_t* rowsum, int64_t M,
                         int64_t K, const void* wmf, const float* beta, int64_t beta_len,
                         int64_t N, float* y, int32_t* acc, void* ws, size_t ws_bytes,
                         void* stream) {
  if (!q || !rowsum || !wmf || (!y && !acc)) return BL_ERR_NULL;
  if (!dims_ok(M, N, K) || N % 64 || K % 64 || K > 65536 || M * K >= (int64_t(1) << 31))
    return BL_ERR_SHAPE;
  int st;
  if (y) {
    if (!gamma) return BL_ERR_NULL;
    if ((st = check_beta(beta, beta_len, N))) return st;
  }
  if (!aligned16(q) || !aligned16(wmf)) return BL_ERR_ALIGN;
  const WsLayout L = ws_layout(M, N, K);
  if (!ws || ws_bytes < L.total) return BL_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return BL_ERR_ALIGN;
  const size_t ob = static_cast<size_t>(M) * N * 4;
  for (const void* out : {static_cast<const void*>(y), static_cast<const void*>(acc)}) {
    if (!out) continue;
    if (overlap(out, ob, q, M * K) || overlap(out, ob, wmf, N * K / 4) ||
        overlap(out, ob, gamma, gamma ? M * 4 : 0) || overlap(out, ob, rowsum, M * 4) ||
        overlap(out, ob, beta, y ? beta_len * 4 : 0) || overlap(out, ob, ws, ws_bytes))
      return BL_ERR_ALIAS;
  }
  if (y && acc && overlap(y, ob, acc, ob)) return BL_ERR_ALIAS;
  char* w = static_cast<char*>(ws);
  return check_launch(launch_tern_mf(q, gamma, rowsum, M, K, wmf, beta, beta_len, N, y, acc,
                                     reinterpret_cast<uint64_t*>(w + L.acc_off),
                                     static_cast<hipStream_t>(stream)),
                      "bl_bitlinear_gemm_mf");
}

int bl_bitlinear_forward_mf(const uint16_t* x, int64_t M, int64_t K, const void* wmf,
                            const float* beta, int64_t beta_len, int64_t N, float* y, void* ws,
                            size_t ws_bytes, void* stream) {
  if (!x || !y || !wmf) return BL_ERR_NULL;
  if (!dims_ok(M, N, K) || N % 64 || K % 64 || K > 28672 || M * K >= (int64_t(1) << 31))
    return BL_ERR_SHAPE;
  int st = check_beta(beta, beta_len, N);
  if (st) return st;
  if (!aligned16(x) || !aligned16(wmf)) return BL_ERR_ALIGN;
  const WsLayout L = ws_layout(M, N, K);
  if (!ws || ws_bytes < L.total) return BL_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return BL_ERR_ALIGN;
  const size_t yb = static_cast<size_t>(M) * N * 4;
  if (overlap(y, yb, x, M * K * 2) || overlap(y, yb, wmf, N * K / 4) ||
      overlap(y, yb, beta, beta_len * 4) || overlap(y, yb, ws, ws_bytes))
    return BL_ERR_ALIAS;
  char* w = static_cast<char*>(ws);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  // decode: one launch quantises and multiplies. Each workgroup quantises its K range of
  // every row itself, so beyond four rows that pays only for narrow outputs of short rows
  // (measured on MI355X, 70B-shaped linears, us per call: M = 4 all four shapes fused, e.g.
  // down 18.7 against 20.0 for quantiser + product; M = 8 q|k|v 13.1 / o 12.3 fused against
  // 14.6 / 14.4, gate|up 32.3 against 27.7, down 23.4 against 23.0; M = 16 q|k|v and o
  // 19.6 / 18.5 against 19.6 / 17.8, down 45.8 against 28.3)
  if (mf_decode_fits(M, N, K) && (M <= 4 || (K <= 8192 && N / 64 < 512)))
    return check_launch(launch_mf_decode(x, static_cast<int>(M), K, wmf, beta, beta_len, N, y,
                                         reinterpret_cast<uint64_t*>(w + L.acc_off), s),
                        "bl_bitlinear_forward_mf");
  auto* qbuf = reinterpret_cast<int8_t*>(w + L.q_off);
  auto* gbuf = reinterpret_cast<float*>(w + L.gamma_off);
  auto* rbuf = reinterpret_cast<int32_t*>(w + L.rowsum_off);
  hipError_t e = launch_quant_act(x, M, K, qbuf, gbuf, rbuf, nullptr, s);
  if (e != hipSuccess) return hip_fail(e, "bl_bitlinear_forward_mf (quantise)");
  return check_launch(launch_tern_mf(qbuf, gbuf, rbuf, M, K, wmf, beta, beta_len, N, y, nullptr,
                                     reinterpret_cast<uint64_t*>(w + L.acc_off), s),
                      "bl_bitlinear_forward_mf");
}

int bl_bitlinear_acc_i32(const int8_t* q, const uint32_t* planes, int64_t M, int64_t K,
                         const void* wpacked, int64_t N, int32_t* acc, int path, void* ws,
                         size_t ws_bytes, void* stream) {
  if (!acc || !wpacked) return BL_ERR_NULL;
  if (!dims_ok(M, N, K) || N % 64 || K % 64 || 127 * K >= (int64_t(1) << 31)) return BL_ERR_SHAPE;
  if (path == BL_PATH_AUTO) path = (M <= 2 && planes) ? BL_PATH_GEMV : BL_PATH_GEMM;
  if (path != BL_PATH_GEMV && path != BL_PATH_GEMM) return BL_ERR_ARG;
  if (path == BL_PATH_GEMV && !planes) return BL_ERR_NULL;
  if (path == BL_PATH_GEMM && !q) return BL_ERR_NULL;
  if (path == BL_PATH_GEMV && M > 4) return BL_ERR_SHAPE;
  if (!aligned16(wpacked) || (q && !aligned16(q)) || (planes && !aligned16(planes)))
    return BL_ERR_ALIGN;
  const WsLayout L = ws_layout(M, N, K);
  if (!ws || ws_bytes < L.total) return BL_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return BL_ERR_ALIGN;
  const size_t ab = static_cast<size_t>(M) * N * 4;
  if (overlap(acc, ab, q, M * K) || overlap(acc, ab, planes, M * K) ||
      overlap(acc, ab, wpacked, N * K / 4) || overlap(acc, ab, ws, ws_bytes))
    return BL_ERR_ALIAS;
  char* w = static_cast<char*>(ws);
  auto* wsacc = reinterpret_cast<uint64_t*>(w + L.acc_off);
  auto* wscnt = reinterpret_cast<uint32_t*>(w + L.cnt_off);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (path == BL_PATH_GEMV)
    return check_launch(launch_gemv(planes, nullptr, static_cast<int>(M), K, wpacked, nullptr, 1,
                                    N, nullptr, acc, wsacc, wscnt, s),
                        "bl_bitlinear_acc_i32");
  return check_launch(launch_gemm(q, nullptr, M, K, wpacked, nullptr, 1, N, nullptr, acc, wsacc,
                                  s),
                      "bl_bitlinear_acc_i32");
}

int bl_bitlinear_forward(const uint16_t* x, int64_t M, int64_t K, const void* wpacked,
                         const float* beta, int64_t beta_len, int64_t N, float* y, int path,
                         void* ws, size_t ws_bytes, void* stream) {
  if (!x || !y || !wpacked) return BL_ERR_NULL;
  if (!dims_ok(M, N, K) || N % 64 || K % 64 || K > 28672) return BL_ERR_SHAPE;
  int st = check_beta(beta, beta_len, N);
  if (st) return st;
  if (path == BL_PATH_AUTO) path = M <= 2 ? BL_PATH_GEMV : BL_PATH_GEMM;
  if (path != BL_PATH_GEMV && path != BL_PATH_GEMM) return BL_ERR_ARG;
  if (path == BL_PATH_GEMV && M > 4) return BL_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(wpacked)) return BL_ERR_ALIGN;
  const WsLayout L = ws_layout(M, N, K);
  if (!ws || ws_bytes < L.total) return BL_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return BL_ERR_ALIGN;
  const size_t yb = static_cast<size_t>(M) * N * 4;
  if (overlap(y, yb, x, M * K * 2) || overlap(y, yb, wpacked, N * K / 4) ||
      overlap(y, yb, beta, beta_len * 4) || overlap(y, yb, ws, ws_bytes))
    return BL_ERR_ALIAS;
  char* w = static_cast<char*>(ws);
  auto* wsacc = reinterpret_cast<uint64_t*>(w + L.acc_off);
  auto* wscnt = reinterpret_cast<uint32_t*>(w + L.cnt_off);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (path == BL_PATH_GEMV) {
    e = launch_gemv_fused(x, static_cast<int>(M), K, wpacked, beta, beta_len, N, y, wsacc, wscnt, s);
  } else {
    auto* qbuf = reinterpret_cast<int8_t*>(w + L.q_off);
    auto* gbuf = reinterpret_cast<float*>(w + L.gamma_off);
    e = launch_quant_act(x, M, K, qbuf, gbuf, nullptr, nullptr, s);
    if (e != hipSuccess) return hip_fail(e, "bl_bitlinear_forward (quantise)");
    e = launch_gemm(qbuf, gbuf, M, K, wpacked, beta, beta_len, N, y, nullptr, wsacc, s);
  }
  return check_launch(e, "bl_bitlinear_forward");
}

int bl_bitlinear_forward_gemv_noalloc(const uint16_t* x, int64_t M, int64_t K, const void* wpacked,
                                      const float* beta, int64_t beta_len, int64_t N, float* y,
                                      void* stream) {
  if (!x || !y || !wpacked) return BL_ERR_NULL;
  if (!dims_ok(M, N, K) || N % 64 || K % 64 || K > 28672 || M > 4) return BL_ERR_SHAPE;
  if (M * N > kScratchWords) return BL_ERR_CAPACITY;
  int st = check_beta(beta, beta_len, N);
  if (st) return st;
  if (!aligned16(x) || !aligned16(wpacked)) return BL_ERR_ALIGN;
  const size_t yb = static_cast<size_t>(M) * N * 4;
  if (overlap(y, yb, x, M * K * 2) || overlap(y, yb, wpacked, N * K / 4) ||
      overlap(y, yb, beta, beta_len * 4))
    return BL_ERR_ALIAS;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  uint64_t* words = nullptr;
  st = scratch_words(s, &words);
  if (st) return st;
  return check_launch(launch_gemv_fused(x, static_cast<int>(M), K, wpacked, beta, beta_len, N, y,
                                        words, nullptr, s),
                      "bl_bitlinear_forward_gemv_noalloc");
}

size_t bl_stack_plan_bytes(int64_t count) {
  return count >= 1 && count <= kMaxStack ? stack_plan_bytes(count) : 0;
}

int bl_stack_prepare(const bl_linear_desc* linears, int64_t count, int64_t M, void* plan,
                     size_t plan_bytes, void* stream) {
  if (!linears || !plan) return BL_ERR_NULL;
  if (count < 1 || count > kMaxStack || M < 1 || M > 4) return BL_ERR_SHAPE;
  if (plan_bytes < stack_plan_bytes(count)) return BL_ERR_ARG;
  if (!aligned16(plan)) return BL_ERR_ALIGN;
  const size_t pb = stack_plan_bytes(count);
  for (int64_t l = 0; l < count; ++l) {
    const bl_linear_desc& d = linears[l];
    if (!d.x || !d.wpacked || !d.beta || !d.y) return BL_ERR_NULL;
    if (!dims_ok(M, d.N, d.K) || d.N % 64 || d.K % 64 || d.K > 65536 || M * d.N > kAccCap)
      return BL_ERR_SHAPE;
    const int st = check_beta(d.beta, d.beta_len, d.N);
    if (st) return st;
    if (d.reserved != 0) return BL_ERR_ARG;
    if (!aligned16(d.x) || !aligned16(d.wpacked)) return BL_ERR_ALIGN;
  }
  for (int64_t l = 0; l < count; ++l) {
    const bl_linear_desc& d = linears[l];
    const size_t yb = static_cast<size_t>(M * d.N) * 4;
    if (overlap(d.y, yb, d.x, static_cast<size_t>(M * d.K) * 2) || overlap(d.y, yb, plan, pb))
      return BL_ERR_ALIAS;
    for (int64_t j = 0; j < count; ++j) {
      const bl_linear_desc& o = linears[j];
      if (overlap(d.y, yb, o.wpacked, static_cast<size_t>(o.N * o.K / 4)) ||
          overlap(d.y, yb, o.beta, static_cast<size_t>(o.beta_len) * 4) ||
          (j != l && overlap(d.y, yb, o.y, static_cast<size_t>(M * o.N) * 4)))
        return BL_ERR_ALIAS;
    }
  }
  return check_launch(stack_write_plan(linears, count, M, plan, static_cast<hipStream_t>(stream)),
                      "bl_stack_prepare");
}

int bl_bitlinear_forward_stack(const void* plan, int64_t count, int64_t M, void* ws,
                               size_t ws_bytes, void* stream) {
  if (!plan) return BL_ERR_NULL;
  if (count < 1 || count > kMaxStack || M < 1 || M > 4) return BL_ERR_SHAPE;
  if (!aligned16(plan)) return BL_ERR_ALIGN;
  const WsLayout L = ws_layout(M, 64, 128);
  if (!ws || ws_bytes < L.acc_off + L.acc_bytes) return BL_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return BL_ERR_ALIGN;
  char* w = static_cast<char*>(ws);
  auto* wsacc = reinterpret_cast<uint64_t*>(w + L.acc_off);
  // the grid-wide wait uses the last words of the (zero-maintained) counter region
  auto* bar = reinterpret_cast<uint32_t*>(w + L.cnt_off) + (kMaxCounters - stack_barrier_words());
  return check_launch(launch_gemv_stack(plan, count, M, bar, wsacc,
                                        static_cast<hipStream_t>(stream)),
                      "bl_bitlinear_forward_stack");
}

int bl_stack_status(const void* plan, void* stream) {
  if (!plan) return -1;
  uint32_t st = 0;
  const hipError_t e = stack_read_status(plan, &st, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    hip_fail(e, "bl_stack_status");
    return -1;
  }
  return static_cast<int>(st);
}

int bl_svid_rank1(const float* W, int64_t N, int64_t K, int iters, void* spacked, uint16_t* g,
                  uint16_t* h, float* sigma, void* ws, size_t ws_bytes, void* stream) {
  if (!W || !spacked || !g || !h) return BL_ERR_NULL;
  if (!dims_ok(1, N, K) || N % 64 || K % 128) return BL_ERR_SHAPE;
  if (iters < 1 || iters > 1000) return BL_ERR_ARG;
  if (!aligned16(W) || !aligned16(spacked)) return BL_ERR_ALIGN;
  const WsLayout L = ws_layout(1, N, K);
  if (!ws || ws_bytes < L.total) return BL_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return BL_ERR_ALIGN;
  const size_t wb = static_cast<size_t>(N) * K * 4;
  const void* outs[4] = {spacked, g, h, sigma};
  const size_t outb[4] = {static_cast<size_t>(N) * K / 8, static_cast<size_t>(K) * 2,
                          static_cast<size_t>(N) * 2, 4};
  for (int i = 0; i < 4; ++i) {
    if (overlap(outs[i], outb[i], W, wb) || overlap(outs[i], outb[i], ws, ws_bytes)) return BL_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outb[i], outs[j], outb[j])) return BL_ERR_ALIAS;
  }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = launch_pack_sign(W, N, K, spacked, s);
  if (e != hipSuccess) return hip_fail(e, "bl_svid_rank1 (signs)");
  auto* scratch = reinterpret_cast<float*>(static_cast<char*>(ws) + L.svid_off);
  return check_launch(launch_svid(W, N, K, iters, g, h, sigma, scratch, s), "bl_svid_rank1");
}

int bl_onebit_linear(const uint16_t* x, const uint16_t* g, const void* spacked, const uint16_t* h,
                     int64_t M, int64_t N, int64_t K, float* y, void* ws, size_t ws_bytes,
                     void* stream) {
  if (!x || !g || !spacked || !h || !y) return BL_ERR_NULL;
  if (!dims_ok(M, N, K) || N % 64 || K % 128 || M > kMaxMtiles * 16 || K > kMaxSignK)
    return BL_ERR_SHAPE;
  if (!aligned16(spacked) || !aligned16(x)) return BL_ERR_ALIGN;
  const WsLayout L = ws_layout(M, N, K);
  if (!ws || ws_bytes < L.total) return BL_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return BL_ERR_ALIGN;
  const size_t yb = static_cast<size_t>(M) * N * 4;
  if (overlap(y, yb, x, M * K * 2) || overlap(y, yb, g, K * 2) || overlap(y, yb, h, N * 2) ||
      overlap(y, yb, spacked, N * K / 8) || overlap(y, yb, ws, ws_bytes))
    return BL_ERR_ALIAS;
  char* w = static_cast<char*>(ws);
  return check_launch(launch_onebit(x, g, spacked, h, M, N, K, y,
                                    reinterpret_cast<float*>(w + L.part_off),
                                    reinterpret_cast<uint32_t*>(w + L.cnt_off),
                                    static_cast<hipStream_t>(stream)),
                      "bl_onebit_linear");
}

int bl_residual_binarize(const float* W, int64_t N, int64_t K, void* planes_o, float* alpha_o,
                         void* planes_r, float* alpha_r, void* stream) {
  if (!W || !planes_o || !alpha_o || !planes_r || !alpha_r) return BL_ERR_NULL;
  if (!dims_ok(1, N, K) || N % 64 || K % 128 || N * (K / 128) > (int64_t(1) << 32))
    return BL_ERR_SHAPE;
  if (!aligned16(W) || !aligned16(planes_o) || !aligned16(planes_r)) return BL_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(alpha_o) & 3u) || (reinterpret_cast<uintptr_t>(alpha_r) & 3u))
    return BL_ERR_ALIGN;
  const size_t pb = static_cast<size_t>(N) * K / 8, ab = static_cast<size_t>(N) * (K / 128) * 4;
  const void* outs[4] = {planes_o, alpha_o, planes_r, alpha_r};
  const size_t outb[4] = {pb, ab, pb, ab};
  for (int i = 0; i < 4; ++i) {
    if (overlap(outs[i], outb[i], W, static_cast<size_t>(N) * K * 4)) return BL_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outb[i], outs[j], outb[j])) return BL_ERR_ALIAS;
  }
  return check_launch(launch_residual_binarize(W, N, K, planes_o, alpha_o, planes_r, alpha_r,
                                               static_cast<hipStream_t>(stream)),
                      "bl_residual_binarize");
}

int bl_residual_linear(const uint16_t* x, const void* planes_o, const float* alpha_o,
                       const void* planes_r, const float* alpha_r, int64_t M, int64_t N, int64_t K,
                       float* y, void* ws, size_t ws_bytes, void* stream) {
  if (!x || !planes_o || !alpha_o || !planes_r || !alpha_r || !y) return BL_ERR_NULL;
  if (!dims_ok(M, N, K) || N % 64 || K % 128 || M > kMaxMtiles * 16 || K > kMaxSignK)
    return BL_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(planes_o) || !aligned16(planes_r)) return BL_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(alpha_o) & 3u) || (reinterpret_cast<uintptr_t>(alpha_r) & 3u))
    return BL_ERR_ALIGN;
  const WsLayout L = ws_layout(M, N, K);
  if (!ws || ws_bytes < L.total) return BL_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return BL_ERR_ALIGN;
  const size_t yb = static_cast<size_t>(M) * N * 4, pb = static_cast<size_t>(N) * K / 8;
  const size_t ab = static_cast<size_t>(N) * (K / 128) * 4;
  if (overlap(y, yb, x, M * K * 2) || overlap(y, yb, planes_o, pb) || overlap(y, yb, planes_r, pb) ||
      overlap(y, yb, alpha_o, ab) || overlap(y, yb, alpha_r, ab) || overlap(y, yb, ws, ws_bytes))
    return BL_ERR_ALIAS;
  char* w = static_cast<char*>(ws);
  return check_launch(launch_residual_linear(x, planes_o, alpha_o, planes_r, alpha_r, M, N, K, y,
                                             reinterpret_cast<float*>(w + L.part_off),
                                             reinterpret_cast<uint32_t*>(w + L.cnt_off),
                                             static_cast<hipStream_t>(stream)),
                      "bl_residual_linear");
}

}  // extern "C"
