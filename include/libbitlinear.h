/*
 * libbitlinear — ternary (BitNet b1.58) and sign-only (OneBit) linear layers for
 * AMD Instinct MI355X (gfx950), as a C ABI over hand-written HIP kernels.
 *
 * Sources (cited by page title and section):
 *  [b158]   "微软、国科大开启1Bit时代：大模型转三进制，速度快4倍能耗降至1/41" — BitNet b1.58
 *           write-up. "BitNet b1.58 介绍": weights in {-1, 0, +1}, BitLinear replaces
 *           nn.Linear, per-token activations scaled into [-Q_b, Q_b] without a zero point,
 *           no biases. "实验及结果": the matrix product reduces to int8 additions (Fig. 3)
 *           and latency was measured with a 2-bit kernel (Fig. 2).
 *  [onebit] "清华、哈工大把大模型压缩到了1bit，把大模型放在手机里跑的愿望就快要实现了！" —
 *           OneBit write-up. "OneBit 框架 / 1. 新的1bit结构" (Fig. 3): +-1 weight matrix plus
 *           two FP16 value vectors g, h; y = ((x ⊙ g) · sign(W)^T) ⊙ h; the 4096x4096 storage
 *           count. "3. 通过知识蒸馏迁移原模型能力": only Sign(W) is kept for inference.
 *           "讨论与分析 / 1. 效率": the element products become bit assignments plus additions.
 *  [billm]  "BiLLM: Pushing the Limit of Post-Training Quantization for LLMs" blog summary.
 *           "方法细节", step 2: a weight binarised once plus its residual binarised again;
 *           "存储位开销分析": two sign bits per weight where the residual is kept.
 *
 * Conventions for every entry point:
 *  - Shapes follow nn.Linear: x is [M, K] row-major (M tokens, K inputs), the weight is
 *    [N, K] (N outputs), y is [M, N] row-major fp32. No bias.
 *  - Every pointer argument is a DEVICE pointer on the current HIP device unless stated.
 *    fp16 values are passed as uint16_t IEEE binary16 bit patterns.
 *  - The caller owns every buffer. The library allocates nothing, frees nothing and keeps
 *    no pointer after returning. All work is queued on `stream` (a hipStream_t; NULL = the
 *    default stream) and is asynchronous: a return of BL_OK means the work was queued.
 *  - Arguments are checked on the host before anything is queued; a failed check returns
 *    its status and queues nothing. A failed launch returns BL_ERR_HIP and
 *    bl_last_error() (thread-local) holds the HIP error text. Nothing aborts or throws.
 *  - Conditions that depend on data values cannot be reported synchronously; they yield
 *    the defined outputs stated per function.
 *  - Workspace: ops that split K across workgroups use `ws`, a device buffer of at least
 *    bl_workspace_bytes(M, N, K) bytes that must be zero-filled before its first use
 *    (bl_workspace_clear or any fill). Every call leaves the bytes it used zero again.
 *    Calls that share one workspace must not overlap in time (same stream, or synchronised).
 *  - Results are deterministic: the integer paths give identical bits on every run and the
 *    fp32 paths use a fixed summation order for a given shape.
 *
 * Packed layouts (the pages fix only 2 bits per ternary weight, 1 bit per sign weight):
 *  T2-PN-64 (ternary). N % 64 == 0, K % 64 == 0. Tile (tn, tk) = rows 64tn..+63, inputs
 *    64tk..+63, 1024 bytes at byte (tn*(K/64) + tk)*1024. Row r of a tile = bytes
 *    16r..16r+15 = little-endian uint32 [P0, P1, N0, N1]. Word X_h covers inputs
 *    k = 64tk + 32h + c (c = 0..31); c = 4j + i is bit 8i + j. P bit set iff w = +1, N bit
 *    set iff w = -1, both clear iff w = 0 (both set: invalid). N*K/4 bytes.
 *  X8-64 (int8 activation bit planes). Row m, 64-input tile t: 16 uint32 words at word
 *    (m*(K/64) + t)*16; word 2b + h holds bit b (two's complement, b = 0..7) of
 *    q[m, 64t + 32h + c] at the same bit positions as T2-PN-64. M*K bytes.
 *  T2-MF64 (ternary, for the int8 matrix cores). N % 64 == 0, K % 64 == 0. Tiles as
 *    T2-PN-64 (same order and size), read as 256 uint32 words. Tile row r = 16f + u
 *    (f = 0..3, u = 0..15) and tile input c = 16g + 4j + i (g, j, i = 0..3) sit in word
 *    4*(16g + u) + j at bits 8i + 2f .. 8i + 2f + 1. For f = 0, 1, 2 the field holds
 *    w + 1 (0, 1, 2; 3 is invalid), for f = 3 w in two's complement (00, 01, 11 for
 *    0, +1, -1; 10 is invalid). N*K/4 bytes. (Lane 16g + u of a wave loads the 16 bytes
 *    at 16*(16g + u): exactly the weights of its four matrix-core fragments, and
 *    word j & (0x03030303 << 2f) is one int8 operand dword of fragment f: bytes
 *    4^f (w + 1) for f < 3, signed bytes 64 w for f = 3.)
 *  S1-128 (sign). N % 64 == 0, K % 128 == 0. Tile (tn, tk) = rows 64tn..+63, inputs
 *    128tk..+127, 1024 bytes at byte (tn*(K/128) + tk)*1024, read as 256 uint32 words.
 *    Tile row r = 16f + u (f = 0..3, u = 0..15) and tile input c = 32s + 8g + 2q + e
 *    (s, g, q = 0..3; e = 0..1) sit in word 4*(16g + u) + f at bit 16e + 4s + q. Bit set
 *    iff the weight is -1. N*K/8 bytes. (Lane 16g + u of a wave loads the 16 bytes at
 *    16*(16g + u): exactly the signs its fp16 matrix-core operands need, and one shift
 *    puts each pair of them at bits 15 and 31.)
 */
#ifndef LIBBITLINEAR_H
#define LIBBITLINEAR_H

#include <stddef.h>
#include <stdint.h>

/* The library is built with hidden default visibility: the declarations below are its only
 * exported symbols. */
#if defined(__GNUC__) || defined(__clang__)
#pragma GCC visibility push(default)
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---------------------------------------------------------------------- */
enum bl_status {
  BL_OK = 0,
  BL_ERR_NULL = 1,       /* a required pointer is NULL */
  BL_ERR_SHAPE = 2,      /* a size is < 1, too large, or not the multiple its layout needs */
  BL_ERR_ALIGN = 3,      /* a pointer lacks the 16-byte alignment its loads need */
  BL_ERR_ALIAS = 4,      /* an output buffer overlaps an input or another output */
  BL_ERR_WORKSPACE = 5,  /* ws is NULL or smaller than bl_workspace_bytes() */
  BL_ERR_HIP = 6,        /* a HIP runtime call or launch failed; see bl_last_error() */
  BL_ERR_ARG = 7,        /* any other invalid argument (e.g. an unknown path, beta_len) */
  BL_ERR_CAPACITY = 8    /* the shape exceeds the library-owned scratch of a no-alloc call */
};

enum bl_path { BL_PATH_AUTO = 0, BL_PATH_GEMV = 1, BL_PATH_GEMM = 2 };

/* Static English text for a status code (never NULL). */
const char* bl_status_string(int status);
/* Thread-local text of the last HIP failure seen by this thread ("" if none). */
const char* bl_last_error(void);
/* Library version, major*10000 + minor*100 + patch. */
int bl_version(void);

/* ---- size queries (pure host functions; 0 for invalid shapes) ---------------------------- */
size_t bl_ternary_packed_bytes(int64_t N, int64_t K);   /* N*K/4, T2-PN-64 */
size_t bl_sign_packed_bytes(int64_t N, int64_t K);      /* N*K/8, S1-128 */
size_t bl_act_planes_bytes(int64_t M, int64_t K);       /* M*K, X8-64 */
/* Bytes of zero-filled workspace that any op below needs for an [M,K] x [N,K]^T product
 * (and bl_ternarize_absmean for an [N,K] matrix). */
size_t bl_workspace_bytes(int64_t M, int64_t N, int64_t K);
/* Queue a zero fill of ws[0:bytes) (a kernel, not a memset, so it may be graph-captured). */
int bl_workspace_clear(void* ws, size_t bytes, void* stream);

/* ---- offline weight preparation ----------------------------------------------------------- */

/* Absmean ternarisation of a float weight [N, K] ([b158] "BitNet b1.58 介绍": ternary
 * weights; the page gives no formula, the reading is absmean):
 *   beta = the fp32 value nearest mean_{n,k} |W[n,k]| (exact sum, single rounding);
 *   code = clip(rne(fl32(W / beta)), -1, 1), decided in fp32.
 * W fp32 [N, K] row-major (16-byte aligned). Outputs (each may be NULL, not both):
 * codes int8 [N, K]; packed T2-PN-64 [N*K/4]. beta: one fp32 (device) written always.
 * Requires N % 64 == 0, K % 64 == 0, N*K < 2^32. If W holds NaN/inf, beta = NaN and every
 * code is 0; if beta == 0 every code is 0. Uses ws (bl_workspace_bytes(1, N, K)). */
int bl_ternarize_absmean(const float* W, int64_t N, int64_t K, int8_t* codes, void* packed,
                         float* beta, void* ws, size_t ws_bytes, void* stream);

/* Pack int8 ternary codes [N, K] into T2-PN-64 ([b158] ternary weights at 2 bits each,
 * "实验及结果"). A code other than -1/0/+1 packs as 0 and adds 1 to *n_invalid (device
 * int32, may be NULL). N % 64 == 0, K % 64 == 0; codes and packed 16-byte aligned. */
int bl_pack_ternary(const int8_t* codes, int64_t N, int64_t K, void* packed,
                    int32_t* n_invalid, void* stream);
/* Inverse of bl_pack_ternary ([b158] "BitNet b1.58 介绍": every weight is -1, 0 or +1):
 * int8 codes [N, K] in {-1, 0, +1}. A (P, N) = (1, 1) pair decodes to 0 and adds 1 to
 * *n_invalid (may be NULL). Shapes and alignment as bl_pack_ternary; codes must not
 * overlap packed. */
int bl_unpack_ternary(const void* packed, int64_t N, int64_t K, int8_t* codes,
                      int32_t* n_invalid, void* stream);

/* Pack int8 ternary codes [N, K] into T2-MF64 ([b158] ternary weights at 2 bits each; the
 * layout serves the int8 matrix-core products below). A code other than -1/0/+1 packs as
 * 0 and adds 1 to *n_invalid (may be NULL). N % 64 == 0, K % 64 == 0; 16-byte aligned. */
int bl_pack_ternary_mf(const int8_t* codes, int64_t N, int64_t K, void* packed,
                       int32_t* n_invalid, void* stream);
/* Convert T2-PN-64 bytes into T2-MF64 (same weights). A (P, N) = (1, 1) pair becomes 0 and
 * adds 1 to *n_invalid (may be NULL). The buffers must not overlap. */
int bl_repack_ternary_mf(const void* t2pn, int64_t N, int64_t K, void* mf, int32_t* n_invalid,
                         void* stream);

/* Pack the signs of a float weight [N, K] into S1-128 ([onebit] "3. 通过知识蒸馏迁移原模型
 * 能力": Sign(W) is what inference keeps). Bit set iff W < 0, so +0, -0 and NaN give +1.
 * N % 64 == 0, K % 128 == 0; W and packed 16-byte aligned. */
int bl_pack_sign(const float* W, int64_t N, int64_t K, void* packed, void* stream);
/* Inverse of bl_pack_sign ([onebit] "1. 新的1bit结构": the weight matrix holds only +-1):
 * int8 signs [N, K] in {-1, +1}. N % 64 == 0, K % 128 == 0; signs must not overlap packed. */
int bl_unpack_sign(const void* packed, int64_t N, int64_t K, int8_t* signs, void* stream);

/* ---- b1.58 forward ------------------------------------------------------------------------- */

/* Per-token absmax int8 quantiser ([b158] "BitNet b1.58 介绍": per-token range
 * [-Q_b, Q_b], no zero point; Q_b = 127):
 *   gamma[m] = max_k |x[m,k]|;  q[m,k] = clip(rne(fl32(fl32(127*x) / gamma[m])), -127, 127);
 *   rowsum[m] = sum_k q[m,k];  planes = X8-64 bit planes of q.
 * x fp16 [M, K] (16-byte aligned). Outputs: gamma fp32 [M] (required); q int8 [M, K],
 * rowsum int32 [M], planes uint32 [M*K/4] (each may be NULL; q or planes must be given).
 * K % 64 == 0. A row holding NaN/inf gets gamma = NaN and q = 0; an all-zero row gets
 * gamma = 0 and q = 0. */
int bl_quant_act_int8(const uint16_t* x, int64_t M, int64_t K, int8_t* q, float* gamma,
                      int32_t* rowsum, uint32_t* planes, void* stream);

/* Add-only decode GEMV ([b158] "实验及结果", Fig. 3: int8 additions only; [onebit]
 * "讨论与分析 / 1. 效率": bit operations plus additions). For M <= 4:
 *   acc[m,n] = sum_k w[n,k] q[m,k] (int32, by popcount additions over the X8-64 planes);
 *   y[m,n] = acc[m,n] * (gamma[m] / 127) * beta[beta_len == 1 ? 0 : n].
 * planes from bl_quant_act_int8, gamma [M], wpacked T2-PN-64 [N, K], beta fp32 [beta_len]
 * with beta_len 1 (per tensor) or N (e.g. stacked q/k/v), y fp32 [M, N]. 1 <= M <= 4,
 * N % 64 == 0, K % 64 == 0. Uses ws. */
int bl_bitlinear_gemv(const uint32_t* planes, const float* gamma, int64_t M, int64_t K,
                      const void* wpacked, const float* beta, int64_t beta_len, int64_t N,
                      float* y, void* ws, size_t ws_bytes, void* stream);

/* Batched / prefill GEMM with int8 matrix cores ([b158] "实验及结果": batched throughput at
 * sequence length 512). Same result as bl_bitlinear_gemv for any M >= 1: the packed
 * weights are expanded to int8 operands and multiplied by q with int32 accumulation
 * (M <= 64: expanded in registers as they stream in; M > 64: expanded once per output
 * tile into LDS and shared by the workgroup's waves).
 * q int8 [M, K] (16-byte aligned rows), other arguments as bl_bitlinear_gemv. Uses ws. */
int bl_bitlinear_gemm(const int8_t* q, const float* gamma, int64_t M, int64_t K,
                      const void* wpacked, const float* beta, int64_t beta_len, int64_t N,
                      float* y, void* ws, size_t ws_bytes, void* stream);

/* Batched product from T2-MF64 weights on int8 matrix cores ([b158] "实验及结果": batched
 * serving; Fig. 3: int8 accumulation), built for batched decode (M <= 64, any M accepted).
 * The matrix cores multiply q by the scaled fields of the layout; for outputs in the first
 * 48 rows of each 64-row band the final sum subtracts rowsum[m], which must be
 * sum_k q[m,k] (bl_quant_act_int8 computes it), so
 *   acc[m,n] = sum_k w[n,k] q[m,k]   exactly (int32), and
 *   y[m,n] = acc[m,n] * (gamma[m] / 127) * beta[beta_len == 1 ? 0 : n].
 * q int8 [M, K] (16-byte aligned rows), rowsum int32 [M], wmf T2-MF64 [N, K]. Outputs: y fp32
 * [M, N] (needs gamma and beta) and/or acc int32 [M, N] (either may be NULL, not both).
 * N % 64 == 0, K % 64 == 0, K <= 65536, M * K < 2^31. Uses ws. */
int bl_bitlinear_gemm_mf(const int8_t* q, const float* gamma, const int32_t* rowsum, int64_t M,
                         int64_t K, const void* wmf, const float* beta, int64_t beta_len,
                         int64_t N, float* y, int32_t* acc, void* ws, size_t ws_bytes,
                         void* stream);

/* The whole b1.58 linear from fp16 activations and T2-MF64 weights. Decode sizes (M <= 4,
 * and M <= 16 for K <= 8192 over fewer than 512 64-row bands): one launch computes gamma,
 * quantises into LDS and multiplies on the int8 matrix cores; otherwise quantise (q, gamma
 * and rowsum into ws), then bl_bitlinear_gemm_mf. Same result as
 * bl_bitlinear_forward on the same weights in T2-PN-64. x fp16 [M, K]; K <= 28672. Uses ws
 * (bl_workspace_bytes(M, N, K)). */
int bl_bitlinear_forward_mf(const uint16_t* x, int64_t M, int64_t K, const void* wmf,
                            const float* beta, int64_t beta_len, int64_t N, float* y, void* ws,
                            size_t ws_bytes, void* stream);

/* Debug: the int32 accumulators acc[m,n] = sum_k w[n,k] q[m,k] of the chosen kernel path,
 * before the epilogue ([b158] "实验及结果", Fig. 3: the product of ternary weights and int8
 * activations is a sum of int8 terms, so it has exactly one correct int32 value). path BL_PATH_GEMV needs planes (M <= 4), BL_PATH_GEMM needs q,
 * BL_PATH_AUTO takes the path bl_bitlinear_forward would take (and needs its operand).
 * acc int32 [M, N]. Uses ws. */
int bl_bitlinear_acc_i32(const int8_t* q, const uint32_t* planes, int64_t M, int64_t K,
                         const void* wpacked, int64_t N, int32_t* acc, int path, void* ws,
                         size_t ws_bytes, void* stream);

/* The whole b1.58 linear from fp16 activations ([b158] "BitNet b1.58 介绍": BitLinear takes
 * the place of nn.Linear, with per-token absmax activations and no bias): quantise, then
 * GEMV (M <= 2) or GEMM, then rescale. x fp16 [M, K]; other arguments as bl_bitlinear_gemm. path selects the kernel
 * (BL_PATH_AUTO picks by M). Uses ws (bl_workspace_bytes(M, N, K)), which also holds the
 * quantised activations. */
int bl_bitlinear_forward(const uint16_t* x, int64_t M, int64_t K, const void* wpacked,
                         const float* beta, int64_t beta_len, int64_t N, float* y, int path,
                         void* ws, size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): bl_bitlinear_forward on the GEMV path
 * (fused quantise + add-only GEMV, same kernels, same bits) with no workspace argument. Its
 * split-K words live in a scratch array owned by the library, one per GPU, 2 MiB, held
 * until the process ends; the first call on a device looks up its address and queues one
 * zero fill, and every call leaves the words zero again. The call itself allocates and
 * frees nothing. Every call on one GPU shares that GPU's scratch: calls that overlap in
 * time on one GPU (other streams, other threads) race and give undefined outputs; order
 * them. Arguments as bl_bitlinear_forward: x fp16 [M, K], wpacked T2-PN-64 [N, K], beta
 * [beta_len], y fp32 [M, N]; 1 <= M <= 4, N % 64 == 0, K % 64 == 0, K <= 28672. Returns
 * BL_ERR_CAPACITY (nothing queued) when M * N > 262144. */
int bl_bitlinear_forward_gemv_noalloc(const uint16_t* x, int64_t M, int64_t K, const void* wpacked,
                                      const float* beta, int64_t beta_len, int64_t N, float* y,
                                      void* stream);

/* ---- whole-stack decode in one launch ------------------------------------------------------- */

/* One linear of a stack: y = BitLinear(x) exactly as bl_bitlinear_forward on the GEMV path
 * computes it. x fp16 [M, K] (16-byte aligned), wpacked T2-PN-64 [N, K] (16-byte aligned),
 * beta fp32 [beta_len] (1 or N), y fp32 [M, N]. N % 64 == 0, K % 64 == 0, K <= 65536. */
typedef struct bl_linear_desc {
  const uint16_t* x;
  const void* wpacked;
  const float* beta;
  float* y;
  int64_t beta_len;
  int64_t N;
  int64_t K;
  int64_t reserved;  /* must be 0 */
} bl_linear_desc;    /* 64 bytes */

/* Bytes of the device plan for `count` linears: 64 + 64 * count. */
size_t bl_stack_plan_bytes(int64_t count);

/* Checks a list of linears and writes its device plan ("prepare once, call many", as the
 * weights are). `linears` is a HOST array of `count` descriptors (1 <= count <= 4096);
 * `plan` a device buffer of bl_stack_plan_bytes(count) bytes, 16-byte aligned, owned by the
 * caller and read by every bl_bitlinear_forward_stack call that uses it. 1 <= M <= 4.
 * Rejected (nothing queued): a y that overlaps any x of its own linear, any weight, beta,
 * another linear's y or the plan (BL_ERR_ALIAS); shapes as above and M * N <= 4194304
 * (BL_ERR_SHAPE). A y that overlaps the x of a LATER linear is allowed: that linear then
 * reads what the earlier one wrote. The plan records which linears read an earlier output.
 * Blocks until the plan is on the device (a synchronous copy on `stream`). */
int bl_stack_prepare(const bl_linear_desc* linears, int64_t count, int64_t M, void* plan,
                     size_t plan_bytes, void* stream);

/* Decode a whole stack of BitLinear layers in ONE persistent launch ([b158] "实验及结果",
 * Table 3: the 70B model's decode throughput is a sweep over all its linears; Fig. 3: each
 * product is int8 additions). The result is bit-identical to calling bl_bitlinear_forward
 * (GEMV path) for linears 0 .. count-1 in order on one stream: linear l reads its x only
 * after linears 0 .. l-1 have written their y (a grid-wide wait between consecutive
 * linears), while the weights of the next linear are already being read during that wait.
 * count and M must be the values the plan was prepared with. Uses ws: any workspace of
 * bl_workspace_bytes(M, N, K) bytes for some N, K is large enough; zero-filled before its
 * first use and left zero. The launch needs every one of its workgroups resident at once
 * (a cooperative launch; it fails with BL_ERR_HIP if the device cannot hold them); the
 * environment variable BL_STACK_GRID = n > 0 caps the grid at n workgroups. Device
 * status, read with bl_stack_status: 0 ok; 1 the plan header does not match count / M
 * (nothing computed); 2 a grid-wide wait exceeded about two seconds (outputs undefined;
 * clear the workspace before reusing it). */
int bl_bitlinear_forward_stack(const void* plan, int64_t count, int64_t M, void* ws,
                               size_t ws_bytes, void* stream);

/* Synchronises `stream` and returns the device status word of `plan` (see above; it stays
 * set until the plan is prepared again), or a negative value if it cannot be read. */
int bl_stack_status(const void* plan, void* stream);

/* ---- OneBit forward ------------------------------------------------------------------------ */

/* OneBit linear ([onebit] "1. 新的1bit结构", Fig. 3): y = ((x ⊙ g) · S^T) ⊙ h with
 * S = sign(W) in S1-128, g fp16 [K] (one per input), h fp16 [N] (one per output),
 * x fp16 [M, K] unquantised (16-byte aligned), y fp32 [M, N]. t = x*g is exact in fp32;
 * each +-t is t with its sign bit set from the packed bit ("bit assignment"), summed in fp32
 * in a fixed order. N % 64 == 0, K % 128 == 0, K <= 2^26, M <= 1048560. Uses ws. */
int bl_onebit_linear(const uint16_t* x, const uint16_t* g, const void* spacked,
                     const uint16_t* h, int64_t M, int64_t N, int64_t K, float* y, void* ws,
                     size_t ws_bytes, void* stream);

/* SVID initialisation of a OneBit layer from a float weight ([onebit] "2. 基于 SVID 初始化
 * 量化模型": sign and magnitude are separated and the magnitude gets a rank-1 approximation,
 * which the reordered layer uses as its value vectors). Writes S = sign(W) as S1-128 (as
 * bl_pack_sign) and the rank-1 fit h g^T of |W| found by `iters` rounds of power iteration
 * (u <- |W| v / ||.||, v <- |W|^T u / ||.||, v_0 = 1/sqrt(K)), with s = || |W|^T u ||:
 * h = fp16(sqrt(s) u) [N], g = fp16(sqrt(s) v) [K], round to nearest even. sigma (fp32 [1],
 * may be NULL) receives s. Reductions run in a fixed order (deterministic). W fp32 [N, K],
 * 16-byte aligned; N % 64 == 0, K % 128 == 0; 1 <= iters <= 1000. Uses ws
 * (bl_workspace_bytes(1, N, K)). */
int bl_svid_rank1(const float* W, int64_t N, int64_t K, int iters, void* spacked, uint16_t* g,
                  uint16_t* h, float* sigma, void* ws, size_t ws_bytes, void* stream);

/* ---- residual binarisation ------------------------------------------------------------------ */

/* Residual binarisation of a float weight ([billm] "方法细节", step 2, binary residual
 * approximation): W ~ alpha_o ⊙ B_o + alpha_r ⊙ B_r. Groups are one output row by 128
 * consecutive inputs (b = k / 128). For each group:
 *   alpha_o = the fp32 value nearest the exact mean of |W| over the group's 128 inputs
 *             (exact sum, one rounding, ties to even),
 *   B_o = sign(W) (+1 for +0, -0 and NaN), R = fl32(W - alpha_o B_o),
 *   alpha_r = the fp32 value nearest the exact mean of |R| over the group, B_r = sign(R).
 * The sign planes use S1-128 (bit set iff -1), N*K/8 bytes each; alpha_o and alpha_r are
 * fp32 [N, K/128] row-major (4-byte aligned). A group holding NaN gets alpha = NaN; one
 * holding inf (and no NaN) gets alpha_o = inf (its residual then holds NaN).
 * W fp32 [N, K] (16-byte aligned); N % 64 == 0, K % 128 == 0. Outputs must not overlap W
 * or each other. */
int bl_residual_binarize(const float* W, int64_t N, int64_t K, void* planes_o, float* alpha_o,
                         void* planes_r, float* alpha_r, void* stream);

/* Residual-binarised linear: y[m, n] = sum_b alpha_o[n,b] (x_b . B_o[n,b]) +
 * alpha_r[n,b] (x_b . B_r[n,b]), x_b the 128 inputs of group b. x fp16 [M, K] unquantised
 * (16-byte aligned), planes and scales from bl_residual_binarize, y fp32 [M, N]. Group dot
 * products are exact products summed in fp32; the sum over groups runs in a fixed order
 * for a given shape. N % 64 == 0, K % 128 == 0, K <= 2^26, M <= 1048560. Uses ws. */
int bl_residual_linear(const uint16_t* x, const void* planes_o, const float* alpha_o,
                       const void* planes_r, const float* alpha_r, int64_t M, int64_t N, int64_t K,
                       float* y, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#if defined(__GNUC__) || defined(__clang__)
#pragma GCC visibility pop
#endif
#endif /* LIBBITLINEAR_H */
