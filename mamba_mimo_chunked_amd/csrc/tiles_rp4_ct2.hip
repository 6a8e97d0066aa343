// Kernel instantiations of the tile family with ranks padded to 4 and 2 token tile(s) per rank.
#include "mimo_kernels.hpp"

namespace mimo {
MIMO_FAMILY(4, 2)
}  // namespace mimo
