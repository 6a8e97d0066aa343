// Main chunk-kernel instantiations for ranks padded to 1 and 4 token tile(s) per rank.
#include "mimo_kernels.hpp"

namespace mimo {
const kfn* main_table_rp1_ct4() {
#define MIMO_MAIN(NT, PT) main_for<1, 4, NT, PT>()
    static const kfn table[9] = {MIMO_NP_TABLE(MIMO_MAIN)};
#undef MIMO_MAIN
    return table;
}
}  // namespace mimo
