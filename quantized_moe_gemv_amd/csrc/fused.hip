// Single-launch decode of one token through one layer (the units, their
// order and the exchanges between workgroups are in decode_units.h).
#include "plan.h"

namespace mq {
namespace {
constexpr bool kOpaqueTid = false;
}
}  // namespace mq

#include "decode_units.h"

namespace mq {

__global__ __launch_bounds__(kThreads) void k_decode(Plan p) {
    __shared__ Shared sh;
    prefetch_args(p);
    const uint32_t tag = ld_ctr(p.f_epoch) + 1;
    decode_layer(p, sh, tag);
    finish_call(p, sh, tag);
}

}  // namespace mq
