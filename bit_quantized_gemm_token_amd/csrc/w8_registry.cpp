// Gathers the GEMM instances compiled in the per-(format, swap, part)
// translation units into one table (parts 0, 1, 6, 7 and, for Block_FP8, 4,
// 5: GEMM; 2, 3: MoE).
#include <vector>

#include "w8_launch.hpp"

namespace w8 {

#define W8_DECL_PARTS(F, S)                                \
  const GemmInstance* gemm_instances_f##F##_##S##_0(int*); \
  const GemmInstance* gemm_instances_f##F##_##S##_1(int*); \
  const MoeInstance* moe_instances_f##F##_##S##_2(int*);   \
  const MoeInstance* moe_instances_f##F##_##S##_3(int*);   \
  const GemmInstance* gemm_instances_f##F##_##S##_6(int*); \
  const GemmInstance* gemm_instances_f##F##_##S##_7(int*);
// Block_FP8's K-loop quantization instances
const GemmInstance* gemm_instances_f2_0_4(int*);
const GemmInstance* gemm_instances_f2_0_5(int*);
const GemmInstance* gemm_instances_f2_1_4(int*);
const GemmInstance* gemm_instances_f2_1_5(int*);
W8_DECL_PARTS(0, 0)
W8_DECL_PARTS(0, 1)
W8_DECL_PARTS(1, 0)
W8_DECL_PARTS(1, 1)
W8_DECL_PARTS(2, 0)
W8_DECL_PARTS(2, 1)

namespace {
template <class I>
std::vector<I> gather(const I* (*const* parts)(int*), int n) {
  std::vector<I> v;
  for (int i = 0; i < n; ++i) {
    int c = 0;
    const I* p = parts[i](&c);
    if (c > 0) v.insert(v.end(), p, p + c);
  }
  return v;
}
}  // namespace

#define W8_GEMM_PARTS(F, S)                                                      \
  gemm_instances_f##F##_##S##_0, gemm_instances_f##F##_##S##_1,                 \
      gemm_instances_f##F##_##S##_6, gemm_instances_f##F##_##S##_7
#define W8_MOE_PARTS(F, S) moe_instances_f##F##_##S##_2, moe_instances_f##F##_##S##_3

const MoeInstance* moe_instances(int* count) {
  static const std::vector<MoeInstance> all = [] {
    const MoeInstance* (*const parts[])(int*) = {W8_MOE_PARTS(0, 0), W8_MOE_PARTS(0, 1),
                                                 W8_MOE_PARTS(1, 0), W8_MOE_PARTS(1, 1),
                                                 W8_MOE_PARTS(2, 0), W8_MOE_PARTS(2, 1)};
    return gather<MoeInstance>(parts, 12);
  }();
  *count = (int)all.size();
  return all.data();
}

const GemmInstance* gemm_instances(int* count) {
  static const std::vector<GemmInstance> all = [] {
    const GemmInstance* (*const parts[])(int*) = {
        W8_GEMM_PARTS(0, 0),   W8_GEMM_PARTS(0, 1),   W8_GEMM_PARTS(1, 0),
        W8_GEMM_PARTS(1, 1),   W8_GEMM_PARTS(2, 0),   W8_GEMM_PARTS(2, 1),
        gemm_instances_f2_0_4, gemm_instances_f2_0_5, gemm_instances_f2_1_4,
        gemm_instances_f2_1_5};
    return gather<GemmInstance>(parts, (int)(sizeof(parts) / sizeof(parts[0])));
  }();
  *count = (int)all.size();
  return all.data();
}

}  // namespace w8
