// Kernel instantiations of the tile family with ranks padded to 1 and 1 token tile(s) per rank.
#include "mimo_kernels.hpp"

namespace mimo {
MIMO_FAMILY(1, 1)
}  // namespace mimo
