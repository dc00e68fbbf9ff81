// OneBit linear layer: y = ((x ⊙ g) · S^T) ⊙ h with S in {-1, +1} packed as S1-128.
//
// [onebit] "OneBit 框架 / 1. 新的1bit结构" (Fig. 3): the weight is a +-1 matrix and only the
// value vectors g (per input) and h (per output) stay FP16. "讨论与分析 / 1. 效率": with
// binary weights the element products become bit assignments and additions.
//
// Reordered as y = x · (diag(g) S^T) · diag(h): the matrix-core B operand is g itself with
// each element's sign bit assigned from the packed weight bit (the "bit assignment"), so
// every product x * (+-g) is exact in the fp32 accumulator, and h scales each output once.
// The kernel is the shared sign-plane kernel of sign_mfma.h.
#include "sign_mfma.h"

namespace bl {

size_t onebit_part_floats(int64_t M, int64_t N, int64_t K) {
  if (N % 64 || K % 128) return 0;
  return sign_mfma_part_floats(M, N, K, false);
}

hipError_t launch_onebit(const uint16_t* x, const uint16_t* g, const void* spacked,
                         const uint16_t* h, int64_t M, int64_t N, int64_t K, float* y,
                         float* ws_part, uint32_t* ws_cnt, hipStream_t s) {
  SignMfmaArgs a{};
  a.x = x, a.g = g, a.h = h;
  a.p0 = static_cast<const sm_u32x4*>(spacked);
  a.M = M, a.N = N, a.K = K;
  a.y = y, a.part = ws_part, a.cnt = ws_cnt;
  return launch_sign_mfma<false>(a, s);
}

}  // namespace bl
