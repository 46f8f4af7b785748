// Explicit instances of the GEMM family for one format, one Swap-AB setting
// and one part: W8_PART 0 and 1 are the GEMM instances with MB = 1 and 2,
// 2 and 3 the MoE grouped instances with MB = 1 and 2, 4 and 5 the Block_FP8
// linear op's instances that quantize in the K loop (XL 3) with MB = 1 and 2,
// 6 and 7 the K-segmented layouts' instances with MB = 1 and 2.  The
// build compiles this file once per (W8_FMT, W8_SWAP, W8_PART) so the
// instances compile in parallel.
#include "w8_gemm.hpp"

#ifndef W8_FMT
#error "W8_FMT must be defined"
#endif
#ifndef W8_SWAP
#error "W8_SWAP must be defined"
#endif
#ifndef W8_PART
#error "W8_PART must be defined"
#endif

#define W8_CAT2(a, b, c, d) a##b##_##c##_##d
#define W8_CAT(a, b, c, d) W8_CAT2(a, b, c, d)
#define W8_MB (W8_PART % 2 + 1)

// One entry per (MB, NB, WK, WN, UNROLL, PACKED, XL, SK): MB in {1, 2}; (NB,
// UNROLL) with NB * UNROLL <= 4 (the weight registers of one stage);
// (WK, WN, XL) in {(1..16, 1, 0), (1..8, 1, 1), (1, 2..8, 1), (1..4, 1, 2),
// (1, 2..8, 2)} (XL 2: fused quantization); PACKED in {0, 1}; SK 0 (one
// workgroup per tile and split) for all of them, SK 1 (stream-K) for NB 1
// with UNROLL 1 or 2 (stream-K never won a tuning, so only the narrowest
// tiles carry it).
#define W8_I(MB, NB, WK, WN, U, P, XL, SK)                                   \
  {W8_FMT, MB, NB, WK, WN, U, W8_SWAP, P, XL, SK,                             \
   &launch_gemm<W8_FMT, MB, NB, WK, WN, U, W8_SWAP, P, XL, SK>},
#define W8_P(MB, NB, WK, WN, U, XL, SK) \
  W8_I(MB, NB, WK, WN, U, 0, XL, SK) W8_I(MB, NB, WK, WN, U, 1, XL, SK)
#define W8_U(MB, WK, WN, XL)                                                                    \
  W8_P(MB, 1, WK, WN, 1, XL, 0) W8_P(MB, 1, WK, WN, 2, XL, 0) W8_P(MB, 1, WK, WN, 4, XL, 0)    \
  W8_P(MB, 2, WK, WN, 1, XL, 0) W8_P(MB, 2, WK, WN, 2, XL, 0) W8_P(MB, 4, WK, WN, 1, XL, 0)    \
  W8_P(MB, 1, WK, WN, 1, XL, 1) W8_P(MB, 1, WK, WN, 2, XL, 1)
#define W8_W(MB)                                                                       \
  W8_U(MB, 1, 1, 0) W8_U(MB, 2, 1, 0) W8_U(MB, 4, 1, 0) W8_U(MB, 8, 1, 0)             \
  W8_U(MB, 16, 1, 0) W8_U(MB, 1, 1, 1) W8_U(MB, 2, 1, 1) W8_U(MB, 4, 1, 1)            \
  W8_U(MB, 8, 1, 1) W8_U(MB, 1, 2, 1) W8_U(MB, 1, 4, 1) W8_U(MB, 1, 8, 1)             \
  W8_U(MB, 1, 1, 2) W8_U(MB, 2, 1, 2) W8_U(MB, 4, 1, 2) W8_U(MB, 1, 2, 2)             \
  W8_U(MB, 1, 4, 2) W8_U(MB, 1, 8, 2)

// The K-segmented layouts (PACKED = T in {2, 4, 8}): WN 1, SK 0, XL 0 and
// (NB, WK, UNROLL) in the set below (single blocks with every K-wave count,
// and two blocks with few K-waves).
#define W8_ST(MB, T)                                                                            \
  W8_I(MB, 1, 1, 1, 1, T, 0, 0) W8_I(MB, 1, 1, 1, 2, T, 0, 0) W8_I(MB, 1, 1, 1, 4, T, 0, 0)    \
  W8_I(MB, 1, 2, 1, 1, T, 0, 0) W8_I(MB, 1, 2, 1, 2, T, 0, 0) W8_I(MB, 1, 4, 1, 1, T, 0, 0)    \
  W8_I(MB, 1, 4, 1, 2, T, 0, 0) W8_I(MB, 1, 8, 1, 1, T, 0, 0) W8_I(MB, 1, 16, 1, 1, T, 0, 0)   \
  W8_I(MB, 2, 1, 1, 1, T, 0, 0) W8_I(MB, 2, 1, 1, 2, T, 0, 0) W8_I(MB, 2, 2, 1, 1, T, 0, 0)    \
  W8_I(MB, 2, 4, 1, 1, T, 0, 0)
// and with the activations quantized into LDS by the kernel (XL 2, the fused
// linear op): waves_k <= 4.
#define W8_SQ(MB, T)                                                                            \
  W8_I(MB, 1, 1, 1, 1, T, 2, 0) W8_I(MB, 1, 1, 1, 2, T, 2, 0) W8_I(MB, 1, 2, 1, 1, T, 2, 0)    \
  W8_I(MB, 1, 2, 1, 2, T, 2, 0) W8_I(MB, 1, 4, 1, 1, T, 2, 0) W8_I(MB, 2, 1, 1, 1, T, 2, 0)    \
  W8_I(MB, 2, 2, 1, 1, T, 2, 0)
#define W8_S(MB) \
  W8_ST(MB, 2) W8_ST(MB, 4) W8_ST(MB, 8) W8_SQ(MB, 2) W8_SQ(MB, 4) W8_SQ(MB, 8)

// Block_FP8's linear op quantizing in the K loop (XL 3): WN 1, WK in {2, 4,
// 8}, tile_n 16 or 32, UNROLL 1 (the shapes it wins on; the bf16
// activations of a stage double its activation registers).  Parts 4 and 5
// hold them (Block_FP8 only).
#define W8_U3(MB, WK) W8_P(MB, 1, WK, 1, 1, 3, 0) W8_P(MB, 2, WK, 1, 1, 3, 0) W8_P(MB, 1, WK, 1, 1, 3, 1)
#define W8_W3(MB) W8_U3(MB, 2) W8_U3(MB, 4) W8_U3(MB, 8)

// The MoE grouped GEMM: the same (MB, NB, UNROLL, PACKED, SK) and (WK, WN, XL)
// in {(1, 1, 0), (2, 1, 0), (4, 1, 0), (8, 1, 0), (1, 2, 1), (1, 4, 1),
// (1, 8, 1)} on quantized activations, and with fused quantization (XL 2) in
// {(1, 4, 2), (1, 8, 2)} (the only fused shapes that ever beat a quantize
// launch + the unfused kernel on the MoE layers measured).
#define W8_MI(MB, NB, WK, WN, U, P, XL, SK)                                  \
  {W8_FMT, MB, NB, WK, WN, U, W8_SWAP, P, XL, SK,                             \
   &launch_moe_gemm<W8_FMT, MB, NB, WK, WN, U, W8_SWAP, P, XL, SK>},
#define W8_MP(MB, NB, WK, WN, U, XL, SK) \
  W8_MI(MB, NB, WK, WN, U, 0, XL, SK) W8_MI(MB, NB, WK, WN, U, 1, XL, SK)
#define W8_MU(MB, WK, WN, XL)                                                                      \
  W8_MP(MB, 1, WK, WN, 1, XL, 0) W8_MP(MB, 1, WK, WN, 2, XL, 0) W8_MP(MB, 1, WK, WN, 4, XL, 0)    \
  W8_MP(MB, 2, WK, WN, 1, XL, 0) W8_MP(MB, 2, WK, WN, 2, XL, 0) W8_MP(MB, 4, WK, WN, 1, XL, 0)    \
  W8_MP(MB, 1, WK, WN, 1, XL, 1) W8_MP(MB, 1, WK, WN, 2, XL, 1)
#define W8_MW(MB)                                                                      \
  W8_MU(MB, 1, 1, 0) W8_MU(MB, 2, 1, 0) W8_MU(MB, 4, 1, 0) W8_MU(MB, 8, 1, 0)         \
  W8_MU(MB, 1, 2, 1) W8_MU(MB, 1, 4, 1) W8_MU(MB, 1, 8, 1)                            \
  W8_MU(MB, 1, 4, 2) W8_MU(MB, 1, 8, 2)

namespace w8 {

#if (W8_PART == 4 || W8_PART == 5) && W8_FMT != 2
#error "parts 4 and 5 exist for Block_FP8 only"
#elif W8_PART < 2 || W8_PART > 3
#if W8_PART < 2
static const GemmInstance kInstances[] = {W8_W(W8_MB)};
#elif W8_PART < 6
static const GemmInstance kInstances[] = {W8_W3(W8_MB)};
#else
static const GemmInstance kInstances[] = {W8_S(W8_MB)};
#endif

const GemmInstance* W8_CAT(gemm_instances_f, W8_FMT, W8_SWAP, W8_PART)(int* count) {
  *count = (int)(sizeof(kInstances) / sizeof(kInstances[0]));
  return kInstances;
}
#else
static const MoeInstance kMoeInstances[] = {W8_MW(W8_MB)};

const MoeInstance* W8_CAT(moe_instances_f, W8_FMT, W8_SWAP, W8_PART)(int* count) {
  *count = (int)(sizeof(kMoeInstances) / sizeof(kMoeInstances[0]));
  return kMoeInstances;
}
#endif

}  // namespace w8
