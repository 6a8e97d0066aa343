// Instances of the stage-2 backward kernels (aggregate and chunk pass, both tile
// geometries) for fp32 data tensors.
#include "mimo_bwd2.hpp"

namespace mimo {
namespace b2 {
Kern kernels_f32(int md, bool ex) { return kernel_pair<DT_F32>(md, ex); }
}  // namespace b2
}  // namespace mimo
