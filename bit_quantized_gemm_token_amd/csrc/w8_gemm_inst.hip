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

// One entry per (MB, NB, WK, UNROLL, PACKED): MB in {1, 2}; (NB, UNROLL) with
// NB * UNROLL <= 4 (the weight registers of one stage); WK in {1, ..., 16};
// PACKED in {0, 1}.
#define W8_I(MB, NB, WK, U, P) \
  {W8_FMT, MB, NB, WK, U, W8_SWAP, P, &launch_gemm<W8_FMT, MB, NB, WK, U, W8_SWAP, P>},
#define W8_P(MB, NB, WK, U) W8_I(MB, NB, WK, U, 0) W8_I(MB, NB, WK, U, 1)
#define W8_U(MB, WK)                                                                   \
  W8_P(MB, 1, WK, 1) W8_P(MB, 1, WK, 2) W8_P(MB, 1, WK, 4) W8_P(MB, 2, WK, 1)         \
  W8_P(MB, 2, WK, 2) W8_P(MB, 4, WK, 1)
#define W8_W(MB) W8_U(MB, 1) W8_U(MB, 2) W8_U(MB, 4) W8_U(MB, 8) W8_U(MB, 16)

namespace w8 {

static const GemmInstance kInstances[] = {W8_W(1) W8_W(2)};

const GemmInstance* W8_TABLE_FN(int* count) {
  *count = (int)(sizeof(kInstances) / sizeof(kInstances[0]));
  return kInstances;
}

}  // namespace w8
