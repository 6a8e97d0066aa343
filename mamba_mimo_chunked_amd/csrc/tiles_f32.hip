// Instances of the fp32-intermediate chunk kernels: every (MT, NT, PT) tile of
// 32, 64 or 128 whose LDS layout fits a compute unit, for bf16 and fp16 inputs.
#include "mimo_f32.hpp"

namespace mimo {
namespace f32 {

namespace {
template <int MT, int NT, int PT, bool MAIN, bool F16>
constexpr kfn pick() {
    if constexpr (lds32(MT, NT, PT, MAIN).total <= 160 * 1024)
        return k_chunk32<MT, NT, PT, MAIN, F16>;
    else
        return nullptr;
}

#define MIMO_F32_NP(F, MT, MAIN, F16)                                                                            \
    F<MT, 32, 32, MAIN, F16>(), F<MT, 32, 64, MAIN, F16>(), F<MT, 32, 128, MAIN, F16>(), F<MT, 64, 32, MAIN, F16>(), \
        F<MT, 64, 64, MAIN, F16>(), F<MT, 64, 128, MAIN, F16>(), F<MT, 128, 32, MAIN, F16>(),                    \
        F<MT, 128, 64, MAIN, F16>(), F<MT, 128, 128, MAIN, F16>()
#define MIMO_F32_ALL(MAIN, F16) \
    {MIMO_F32_NP(pick, 32, MAIN, F16), MIMO_F32_NP(pick, 64, MAIN, F16), MIMO_F32_NP(pick, 128, MAIN, F16)}
}  // namespace

const F32Set* f32_set() {
    static const F32Set s = {{MIMO_F32_ALL(false, false), MIMO_F32_ALL(false, true)},
                             {MIMO_F32_ALL(true, false), MIMO_F32_ALL(true, true)}};
    return &s;
}

}  // namespace f32
}  // namespace mimo
