// Instances of the fp32-intermediate chunk kernels with MT = 64 chunk-tile rows: every
// (NT, PT) tile whose LDS layout fits a compute unit, for bf16 and fp16 inputs, and the
// unit-projection (SISO) instances, and the shape-exact ones (R = 4, C = 16, N = P = 64).
#include "mimo_f32.hpp"

namespace mimo {
namespace f32 {
MIMO_F32_PART_UV_EX(64)
}  // namespace f32
}  // namespace mimo
