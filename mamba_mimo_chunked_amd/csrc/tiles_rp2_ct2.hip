// Kernel instantiations of the tile family with ranks padded to 2 and 2 token tile(s) per rank.
#include "mimo_kernels.hpp"

namespace mimo {
MIMO_FAMILY(2, 2)
}  // namespace mimo
