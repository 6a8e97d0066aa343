// Kernel instantiations of the tile family with ranks padded to 2 and 4 token tile(s) per rank.
#include "mimo_kernels.hpp"

namespace mimo {
MIMO_FAMILY(2, 4)
}  // namespace mimo
