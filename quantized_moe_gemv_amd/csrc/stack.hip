// Single-launch decode of one token through a stack of layers (the units,
// their order and the exchanges between workgroups are in decode_units.h).
#include "plan.h"

namespace mq {
namespace {
constexpr bool kOpaqueTid = true;
constexpr bool kEarlySharedDown = true;
constexpr bool kLateRoutedDown = true;
constexpr bool kLateSharedGateUp = true;
// The row totals' lane sums use permlane swaps: 555.7-556.2 us/token
// against 560.1-560.6 through the LDS crossbar.
constexpr bool kSwapKb = true;
// A gate/up unit's waves skip the spare slots past its end (513 against
// 515 us/token; the lone call is faster with them).
constexpr bool kSpareGateUpLoads = false;
// The unit assignments before the token's loads (see fused.hip).
constexpr bool kTokenFirst = false;
}
}  // namespace mq

#include "decode_units.h"

namespace mq {

// A stack of layers for one token in one launch.  Layer l runs with tag
// epoch + 1 + l; its output sums publish the next layer's input as tagged
// words, so a layer's units start as soon as the words they read are there,
// with no launch between layers.  Every read of a layer's exchange regions
// happens before that layer's output sums complete (each reading workgroup
// feeds them), and the next layer writes those regions only after reading
// its input, so one set of regions serves every layer.  The order of the
// units (layer by layer, in the order above within a layer) keeps every wait
// finite as in the single layer.
__global__ __launch_bounds__(kThreads) void k_decode_stack(const Plan* __restrict__ plans, int n_layers) {
    __shared__ Shared sh;
    const uint32_t base = first_tag(plans[0]) - 1;
    for (int l = 0; l < n_layers; ++l) {
        const Plan& p = plans[l];
        prefetch_args(p);
        decode_layer<false>(p, sh, base + 1 + (uint32_t)l, nullptr);
    }
    finish_call(plans[0], base + (uint32_t)n_layers);
}

// The same with every layer's tail applied in its output sums (a separate
// kernel, so the stack without tails carries none of the tail's code).
__global__ __launch_bounds__(kThreads) void k_decode_stack_tail(const Plan* __restrict__ plans, int n_layers) {
    __shared__ Shared sh;
    __shared__ alignas(16) uint16_t xraw[4096];   // each layer's input row as given (its tail's residual)
    const uint32_t base = first_tag(plans[0]) - 1;
    for (int l = 0; l < n_layers; ++l) {
        const Plan& p = plans[l];
        prefetch_args(p);
        decode_layer<true>(p, sh, base + 1 + (uint32_t)l, xraw);
    }
    finish_call(plans[0], base + (uint32_t)n_layers);
}

// The per-layer arguments of a stack, written into the workspace by one
// small launch per chunk of layers: layer i of the chunk gets the base
// arguments with its own fields.
__global__ void k_stack_plans(Plan base, StackChunk c, Plan* dst) {
    if (threadIdx.x != 0 || (int)blockIdx.x >= c.n) return;
    const StackLayer& s = c.l[blockIdx.x];
    Plan q = base;
    q.x = s.x;
    q.x_w = s.x_w;
    q.out = s.out;
    q.out_w = s.out_w;
    q.router_w = s.router_w;
    q.router_scale = s.router_scale;
    q.pes = s.pes;
    q.logit_bias = s.logit_bias;
    q.eps = s.eps;
    q.in_eps = s.in_eps;
    q.pool_base = s.pool_base;
    q.expert_stride = s.expert_stride;
    q.gate_off = s.gate_off;
    q.up_off = s.up_off;
    q.down_off = s.down_off;
    q.sh_gate = s.sh_gate;
    q.sh_up = s.sh_up;
    q.sh_down = s.sh_down;
    q.ids_out = s.ids_out;
    q.w_out = s.w_out;
    q.logits_out = s.logits_out;
    q.tail = s.tail;
    q.tn_s = s.tn_s;
    q.tn_r = s.tn_r;
    q.tn_o = s.tn_o;
    q.t_eps = s.t_eps;
    q.t_scalar = s.t_scalar;
    q.t_res_in = s.t_res_in;
    q.t_res = s.t_res;
    q.t_res_stride = s.t_res_stride;
    dst[blockIdx.x] = q;
}

}  // namespace mq
