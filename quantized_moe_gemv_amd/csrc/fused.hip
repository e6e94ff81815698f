// Single-launch decode of one token through one layer (the units, their
// order and the exchanges between workgroups are in decode_units.h).
#include "plan.h"

namespace mq {
namespace {
constexpr bool kOpaqueTid = false;
constexpr bool kEarlySharedDown = false;
constexpr bool kLateRoutedDown = false;
constexpr bool kLateSharedGateUp = false;
// The row totals' lane sums go through the LDS crossbar: with permlane
// swaps this kernel measured 20.62-20.70 us per call against 20.03-20.06
// (the stack launch the other way round).
constexpr bool kSwapKb = false;
// A gate/up unit loads all its wave slots (the spare ones from a block
// already cached): 18.75 against 19.00 us per call; the stack launch is
// faster without them (513 against 515 us/token).
constexpr bool kSpareGateUpLoads = true;
// The token's loads go out before the unit assignments: 17.82 against
// 18.05 us per call (the stack launch, where the token arrives from the
// previous layer, measured 513.6 against 512.2 us/token).
constexpr bool kTokenFirst = true;
}
}  // namespace mq

#include "decode_units.h"

namespace mq {

// TAIL: the layer tail is applied in the output sums (a separate instance,
// so the layer without a tail carries none of its code).
template <bool TAIL>
__device__ __forceinline__ void decode_one(const Plan& p) {
    __shared__ Shared sh;
    uint16_t* xraw = nullptr;
    if constexpr (TAIL) {
        __shared__ alignas(16) uint16_t xraw_lds[4096];   // the input row as given (the tail's residual)
        xraw = xraw_lds;
    }
    prefetch_args(p);
    const uint32_t tag = first_tag(p);
    decode_layer<TAIL>(p, sh, tag, xraw);
    finish_call(p, tag);
}

__global__ __launch_bounds__(kThreads) void k_decode(Plan p) { decode_one<false>(p); }
__global__ __launch_bounds__(kThreads) void k_decode_tail(Plan p) { decode_one<true>(p); }

}  // namespace mq
