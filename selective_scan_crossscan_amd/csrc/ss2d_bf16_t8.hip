// Compiles the SS2D forward kernels for bf16 storage, 8 steps per lane.
#include "ss2d_kernels.h"

namespace ss2d {

hipError_t launch_bf16_t8(const LaunchArgs& a, const Plan& plan, const Scratch& s) {
  if (plan.lanes_per_seq == 32) return launch_gt<uint16_t, 32, 8>(a, plan, s);
  return launch_gt<uint16_t, 64, 8>(a, plan, s);
}

}  // namespace ss2d
