// Gathers the GEMM instances compiled in the per-(format, swap) translation
// units into one table.
#include <vector>

#include "w8_launch.hpp"

namespace w8 {

const GemmInstance* gemm_instances_f0_0(int*);
const GemmInstance* gemm_instances_f0_1(int*);
const GemmInstance* gemm_instances_f1_0(int*);
const GemmInstance* gemm_instances_f1_1(int*);
const GemmInstance* gemm_instances_f2_0(int*);
const GemmInstance* gemm_instances_f2_1(int*);

const MoeInstance* moe_instances_f0_0(int*);
const MoeInstance* moe_instances_f0_1(int*);
const MoeInstance* moe_instances_f1_0(int*);
const MoeInstance* moe_instances_f1_1(int*);
const MoeInstance* moe_instances_f2_0(int*);
const MoeInstance* moe_instances_f2_1(int*);

const MoeInstance* moe_instances(int* count) {
  static const std::vector<MoeInstance> all = [] {
    std::vector<MoeInstance> v;
    const MoeInstance* (*parts[])(int*) = {moe_instances_f0_0, moe_instances_f0_1,
                                           moe_instances_f1_0, moe_instances_f1_1,
                                           moe_instances_f2_0, moe_instances_f2_1};
    for (auto part : parts) {
      int n = 0;
      const MoeInstance* p = part(&n);
      v.insert(v.end(), p, p + n);
    }
    return v;
  }();
  *count = (int)all.size();
  return all.data();
}

const GemmInstance* gemm_instances(int* count) {
  static const std::vector<GemmInstance> all = [] {
    std::vector<GemmInstance> v;
    const GemmInstance* (*parts[])(int*) = {gemm_instances_f0_0, gemm_instances_f0_1,
                                            gemm_instances_f1_0, gemm_instances_f1_1,
                                            gemm_instances_f2_0, gemm_instances_f2_1};
    for (auto part : parts) {
      int n = 0;
      const GemmInstance* p = part(&n);
      v.insert(v.end(), p, p + n);
    }
    return v;
  }();
  *count = (int)all.size();
  return all.data();
}

}  // namespace w8
