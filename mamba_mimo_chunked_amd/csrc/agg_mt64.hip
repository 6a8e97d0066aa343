// Segment-aggregate kernel instantiations for chunk tiles of 64 rows.
#include "mimo_kernels.hpp"

namespace mimo {
const kfn* agg_table_mt64() {
#define MIMO_AGG(NT, PT) agg_for<64, NT, PT>()
    static const kfn table[9] = {MIMO_NP_TABLE(MIMO_AGG)};
#undef MIMO_AGG
    return table;
}
}  // namespace mimo
