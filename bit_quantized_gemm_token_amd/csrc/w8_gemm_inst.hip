// Explicit instances of the GEMM family for one format and one Swap-AB
// setting.  The build compiles this file once per (W8_FMT, W8_SWAP) pair so
// the instances compile in parallel.
#include "w8_gemm.hpp"

#ifndef W8_FMT
#error "W8_FMT must be defined"
#endif
#ifndef W8_SWAP
#error "W8_SWAP must be defined"
#endif

#define W8_CAT2(a, b, c) a##b##_##c
#define W8_CAT(a, b, c) W8_CAT2(a, b, c)
#define W8_TABLE_FN W8_CAT(gemm_instances_f, W8_FMT, W8_SWAP)

// One entry per (MB, WN, WK, UNROLL): MB in {1, 2}; (WN, WK) with
// WN*WK <= 16; UNROLL in {1, 2, 4}.
#define W8_I(MB, WN, WK, U) \
  {W8_FMT, MB, WN, WK, U, W8_SWAP, &launch_gemm<W8_FMT, MB, WN, WK, U, W8_SWAP>},
#define W8_U(MB, WN, WK) W8_I(MB, WN, WK, 1) W8_I(MB, WN, WK, 2) W8_I(MB, WN, WK, 4)
#define W8_W(MB)                                                                    \
  W8_U(MB, 1, 1) W8_U(MB, 1, 2) W8_U(MB, 1, 4) W8_U(MB, 1, 8) W8_U(MB, 1, 16)      \
  W8_U(MB, 2, 1) W8_U(MB, 2, 2) W8_U(MB, 2, 4) W8_U(MB, 2, 8) W8_U(MB, 4, 1)       \
  W8_U(MB, 4, 2) W8_U(MB, 4, 4)

namespace w8 {

static const GemmInstance kInstances[] = {W8_W(1) W8_W(2)};

const GemmInstance* W8_TABLE_FN(int* count) {
  *count = (int)(sizeof(kInstances) / sizeof(kInstances[0]));
  return kInstances;
}

}  // namespace w8
