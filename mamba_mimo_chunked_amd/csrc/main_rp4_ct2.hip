// Main chunk-kernel instantiations for ranks padded to 4 and 2 token tile(s) per rank.
#include "mimo_kernels.hpp"

namespace mimo {
const kfn* main_table_rp4_ct2() {
#define MIMO_MAIN(NT, PT) main_for<4, 2, NT, PT>()
    static const kfn table[9] = {MIMO_NP_TABLE(MIMO_MAIN)};
#undef MIMO_MAIN
    return table;
}
}  // namespace mimo
