// Compiles the SS2D forward kernels for bf16 storage, 16 steps per lane.
#include "ss2d_kernels.h"

namespace ss2d {

hipError_t launch_bf16_t16(const LaunchArgs& a, const Plan& plan, const Scratch& s) {
  switch (plan.lanes_per_seq) {
    case 16: return launch_gt<uint16_t, 16, 16>(a, plan, s);
    case 32: return launch_gt<uint16_t, 32, 16>(a, plan, s);
    default: return launch_gt<uint16_t, 64, 16>(a, plan, s);
  }
}

}  // namespace ss2d
