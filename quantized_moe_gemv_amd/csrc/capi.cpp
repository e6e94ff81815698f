// C-ABI entry points: argument checks, workspace carve-up and launches.
#include <hip/hip_runtime.h>
#include <math.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "../../include/moegemv.h"
#include "layout.h"
#include "plan.h"

namespace mq {
__global__ void k_prep(Plan p);
__global__ void k_router(Plan p);
__global__ void k_topk(Plan p);
__global__ void k_gateup(Plan p);
__global__ void k_gateup8(Plan p);
__global__ void k_down(Plan p);
__global__ void k_down8(Plan p);
__global__ void k_combine(Plan p);
__global__ void k_rmsnorm(const uint16_t* x, int64_t xs, uint16_t* y, int64_t ys, int H, float eps);
__global__ void k_debug_read(const uint8_t* data, int rows, int cols, int bits, uint8_t* codes_out, float* w_out);
__global__ void k_decode(Plan p);
__global__ void k_decode_tail(Plan p);
__global__ void k_decode_stack(const Plan* plans, int n_layers);
__global__ void k_decode_stack_tail(const Plan* plans, int n_layers);
__global__ void k_stack_plans(Plan base, StackChunk c, Plan* dst);
__global__ void k_stream_read(const uint4* buf, int64_t n16, uint32_t* sink);
__global__ void k_tail_gemv(Plan p);
int head_groups(int rows);
mq_status launch_head(const HeadArgs& a, int32_t* argmax, hipStream_t s);
mq_status launch_grouped(const Plan& p, hipStream_t s);
bool grouped_ok(int H, int I, int64_t T, int rows_per_token);
int grouped_shared_rows(int ntile, int n_vs);
}  // namespace mq

using namespace mq;

namespace {

constexpr size_t kAlign = 256;

inline size_t up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

struct Sizes {
    int H, E, E_pad, k, I, Is, G_H, G_I, G_s, rsplit, rgroups, ntile, max_tiles, n_vs;
    int n_router, n_sd, n_sc, n_rh, n_src;
    int ebits;
};

// State of the single-launch decode that persists across calls.  It sits at
// the start of the workspace, at offsets that do not depend on the token
// count, and no other kernel writes it.
struct FusedCarve {
    size_t rpart, act, piece, xw, tail, ctr, epoch, total;
    int64_t h_stride, rpart_stride, xw_stride;   // in 8-byte words
};

FusedCarve fused_carve(const Sizes& z) {
    FusedCarve f;
    size_t o = 0;
    auto take = [&](size_t bytes) { size_t at = o; o += up(bytes); return at; };
    f.ctr = take((size_t)3 * kCtrStride * 4);   // (unused), (unused), error flag: first, at fixed offsets
    f.epoch = take((size_t)kFusedMaxWG * 4);    // one word per workgroup
    f.rpart_stride = (int64_t)up((size_t)(z.E + 15) / 16 * 8 * 16 * 8) / 8;
    f.rpart = take((size_t)8 * f.rpart_stride * 8);
    // one copy per XCD of the activations (shared then routed)
    f.h_stride = (int64_t)up(((size_t)z.Is + (size_t)z.k * z.I) * 8 + 8) / 8;
    f.act = take((size_t)8 * f.h_stride * 8);
    f.piece = take((size_t)z.G_H * z.n_src * 64 * 8);
    // one copy per XCD of a stack layer's output row (bf16 pairs)
    f.xw_stride = (int64_t)up((size_t)z.H / 2 * 8) / 8;
    f.xw = take((size_t)8 * f.xw_stride * 8);
    f.tail = take((size_t)z.G_H * 8 * 8);   // per output tile: tagged partial sums of the tail norms
    f.total = o;
    return f;
}

// The largest layer the single-launch decode takes (fused_ok): H <= 3072
// (48 groups), E <= 256, k * I <= 16 * 768, Is <= 8192, n_src <= 32.  Its
// persistent region is reserved at this size in every workspace, and every
// other buffer starts after it, so a workspace shared by layers of
// different sizes and by the other paths never overwrites the tagged words
// the single-launch decode reads across calls (a stale word whose high half
// happened to equal a later tag would pass for a current one).
constexpr int kFusedMaxH = 3072, kFusedMaxE = 256, kFusedMaxKI = 16 * 768, kFusedMaxIs = 8192, kFusedMaxSrc = 32;

size_t fused_region_max() {
    Sizes m;
    memset(&m, 0, sizeof(m));
    m.H = kFusedMaxH;
    m.E = kFusedMaxE;
    m.k = 16;
    m.I = kFusedMaxKI / 16;
    m.Is = kFusedMaxIs;
    m.G_H = kFusedMaxH / kGroup;
    m.n_src = kFusedMaxSrc;
    return fused_carve(m).total;
}

// The single-launch decode holds every unit's loads in registers, one
// workgroup per compute unit.  Workgroups 0 .. n_rh-1 each run a full-row
// routed gate/up unit (2 G_H <= 16 waves x 6 loads); the m = cus - n_rh
// others run one full-row shared gate/up unit each (the first 2 G_s of them)
// and at most kFusedSlotsSD shared down pieces each; routed down work runs
// one tile per routed workgroup for the first S = n_rh / G_H slots and in
// n_rng ranges of at most kFusedTilesD tiles on the shared workgroups for
// the others; router piece i on workgroup G_H + i; output tile a's sum on
// workgroup a.
constexpr int kFusedSlotsSD = 2, kFusedTilesD = 3;

int fused_ranges(const Sizes& z, int cus) {
    const int S = std::min(z.n_rh / z.G_H, z.k), m = cus - z.n_rh;
    return S >= z.k ? 1 : std::min(m / (z.k - S), z.G_H);
}

bool fused_ok(const Sizes& z, int cus) {
    const int m = cus - z.n_rh, r = fused_ranges(z, cus);
    // routed down slots run in tile ranges on the shared workgroups only when
    // the routed workgroups cannot take every slot (S < k)
    const bool ranges = std::min(z.n_rh / z.G_H, z.k) < z.k;
    if (z.G_H > 48 || z.G_I > 12 || z.n_src > kFusedMaxSrc || m < 1 || r < 1 || cus > kFusedMaxWG) return false;
    if (z.H > kFusedMaxH || z.E > kFusedMaxE || z.k * z.I > kFusedMaxKI || z.Is > kFusedMaxIs) return false;
    if (z.ebits != 4) return false;
    return (!ranges || (z.G_H + r - 1) / r <= kFusedTilesD) && 2 * z.G_s <= m && (std::max(z.n_sd - z.n_rh, 0) + m - 1) / m <= kFusedSlotsSD &&
           z.G_H + z.n_router <= cus;
}

int device_cus() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    return cus;
}

// Offsets of every workspace region for up to T tokens; returns the total.
struct Carve {
    size_t r, rsum8, xsum4, xsum8, plog, ids, wts, hhi, hlo, hsum, shi, slo, ssum, dpart;
    size_t xn, x16, xso, counts, offsets, perm, inv, sched, nsched, gdone, gqueue, hg, hso, ysort;
    size_t total;
};

Carve carve(const Sizes& z, int64_t T) {
    Carve c;
    size_t o = fused_region_max();
    auto take = [&](size_t bytes) { size_t at = o; o += up(bytes); return at; };
    c.r = take(T * z.H * 4);
    c.rsum8 = take(T * z.G_H * 16);
    c.xsum4 = take(T * z.G_H * 16);
    c.xsum8 = take(T * z.G_H * 16);
    c.plog = take((size_t)z.rsplit * T * z.E_pad * 4);
    c.ids = take(T * z.k * 4);
    c.wts = take(T * z.k * 4);
    c.hhi = take(T * z.k * z.I * 2);
    c.hlo = take(T * z.k * z.I * 2);
    c.hsum = take(T * z.k * z.G_I * 16);
    c.shi = take(T * z.Is * 2 + 16);
    c.slo = take(T * z.Is * 2 + 16);
    c.ssum = take(T * z.G_s * 16 + 16);
    c.dpart = take(T * kDownSplits * z.H * 4);
    c.xn = take(T * z.H * 2);
    c.x16 = take(T * z.H * 2);
    c.xso = take(T * z.G_H * 8);
    c.counts = take((size_t)z.E * 4);
    c.offsets = take((size_t)(z.E + 1) * 4);
    c.perm = take(T * z.k * 4);
    c.inv = take(T * z.k * 4);
    // sized for the smallest chunk so that the carve grows with T whatever
    // chunk size set_tiles picks
    const size_t nentries = (size_t)(T * z.k + 31) / 32 + z.E + (size_t)z.n_vs * ((T + 31) / 32) + 1;
    c.sched = take(nentries * 8);
    c.nsched = take(8);
    c.gdone = take(nentries * 4);
    c.gqueue = take(nentries * 4);
    const size_t rows = T * (z.k + z.n_vs);
    c.hg = take(rows * z.I * 2);
    c.hso = take(rows * z.G_I * 8);
    c.ysort = take(rows * z.H * 4);
    c.total = o;
    return c;
}

// Group sizes: any multiple of 64 dividing the columns.  DEV_V1 keeps a
// (scale, bias) pair per 64-column block, so larger groups were expanded to
// it when packed and every kernel reads them as group 64.
bool group_ok(int cols, int group) { return group > 0 && group % kGroup == 0 && cols > 0 && cols % group == 0; }

bool qt_dev_ok(const mq_qtensor& t, int bits) {
    return t.codes && t.bits == bits && group_ok(t.cols, t.group) && t.layout == MQ_LAYOUT_DEV_V1 && t.rows > 0;
}

// Checks everything that does not depend on the call's tokens.
mq_status check_layer(const mq_router* rt, const mq_expert_pool* pool, const mq_shared* sh, Sizes* z) {
    if (!rt || !pool) return MQ_ERR_NULL;
    if (!rt->w.codes || !pool->base) return MQ_ERR_NULL;
    if (rt->w.bits != 8 || rt->w.group % kGroup || rt->w.group <= 0 || rt->w.layout != MQ_LAYOUT_DEV_V1)
        return MQ_ERR_UNSUPPORTED;
    if ((pool->bits != 4 && pool->bits != 8) || pool->group % kGroup || pool->group <= 0 ||
        pool->layout != MQ_LAYOUT_DEV_V1)
        return MQ_ERR_UNSUPPORTED;
    const int H = pool->hidden, E = pool->num_experts, I = pool->inter, eb = pool->bits;
    if (H <= 0 || H % kGroup || I <= 0 || I % kGroup || E <= 0 || E > kMaxExperts) return MQ_ERR_SHAPE;
    if (!group_ok(H, rt->w.group) || !group_ok(H, pool->group) || !group_ok(I, pool->group)) return MQ_ERR_SHAPE;
    if (rt->w.rows != E || rt->w.cols != H) return MQ_ERR_SHAPE;
    if (rt->top_k < 1 || rt->top_k > E || rt->top_k > kMaxTopK) return MQ_ERR_SHAPE;
    if (!(rt->eps >= 0.f)) return MQ_ERR_SHAPE;
    if (!aligned(rt->w.codes, kAlign) || !aligned(pool->base, kAlign)) return MQ_ERR_ALIGN;
    if (rt->router_scale && !aligned(rt->router_scale, 16)) return MQ_ERR_ALIGN;
    if (pool->expert_stride % 256 || pool->gate_offset % 256 || pool->up_offset % 256 || pool->down_offset % 256)
        return MQ_ERR_ALIGN;
    const int64_t gu = (int64_t)mq_packed_bytes(I, H, eb, kGroup, MQ_LAYOUT_DEV_V1);
    const int64_t dn = (int64_t)mq_packed_bytes(H, I, eb, kGroup, MQ_LAYOUT_DEV_V1);
    if (pool->gate_offset < 0 || pool->up_offset < 0 || pool->down_offset < 0 ||
        pool->gate_offset + gu > pool->expert_stride || pool->up_offset + gu > pool->expert_stride ||
        pool->down_offset + dn > pool->expert_stride)
        return MQ_ERR_SHAPE;
    int Is = 0;
    if (sh) {
        if (!qt_dev_ok(sh->gate, eb) || !qt_dev_ok(sh->up, eb) || !qt_dev_ok(sh->down, eb)) {
            if (!sh->gate.codes || !sh->up.codes || !sh->down.codes) return MQ_ERR_NULL;
            return MQ_ERR_UNSUPPORTED;
        }
        Is = sh->gate.rows;
        if (Is % kGroup || sh->up.rows != Is || sh->gate.cols != H || sh->up.cols != H || sh->down.rows != H ||
            sh->down.cols != Is)
            return MQ_ERR_SHAPE;
        if (!aligned(sh->gate.codes, kAlign) || !aligned(sh->up.codes, kAlign) || !aligned(sh->down.codes, kAlign))
            return MQ_ERR_ALIGN;
    }
    z->H = H;
    z->ebits = eb;
    z->E = E;
    z->E_pad = (int)pad_rows(E);
    z->k = rt->top_k;
    z->I = I;
    z->Is = Is;
    z->G_H = H / kGroup;
    z->G_I = I / kGroup;
    z->G_s = Is / kGroup;
    z->rgroups = 4;
    z->rsplit = (z->G_H + z->rgroups - 1) / z->rgroups;
    // single-launch decode: router slices of 16 experts in kRouterPieces column pieces
    z->n_router = (E + 15) / 16 * kRouterPieces;
    z->n_sc = (z->G_s + z->G_I - 1) / z->G_I;
    z->n_sd = z->G_H * z->n_sc;
    z->n_rh = 2 * z->k * z->G_I;
    z->n_src = z->k + z->n_sc;
    return MQ_OK;
}

void set_tiles(Sizes* z, int64_t T, bool has_shared) {
    // tokens per grouped work item: 64 up to 1024 tokens, so that no work
    // item outlasts the call's weight streaming, 128 above (fewer re-reads
    // of the weights where the matrix cores bound the call)
    z->ntile = T <= 1024 ? 64 : 128;
    z->n_vs = has_shared ? z->n_sc : 0;
    // every expert may add one partial chunk to the full ones
    const int64_t nch = (T + z->ntile - 1) / z->ntile;
    z->max_tiles = (int)((T * z->k + z->ntile - 1) / z->ntile + z->E + z->n_vs * nch);
}

// Sizes, weights and per-layer router settings of one layer.
void fill_layer(Plan& p, const Sizes& z, const mq_router* router, const mq_expert_pool* pool,
                const mq_shared* shared) {
    p.H = z.H;
    p.E = z.E;
    p.E_pad = z.E_pad;
    p.k = z.k;
    p.I = z.I;
    p.Is = z.Is;
    p.G_H = z.G_H;
    p.G_I = z.G_I;
    p.G_s = z.G_s;
    p.rsplit = z.rsplit;
    p.rgroups = z.rgroups;
    p.has_shared = shared != nullptr;
    p.ebits = z.ebits;
    p.router_w = (const uint8_t*)router->w.codes;
    p.router_scale = router->router_scale;
    p.pes = router->per_expert_scale;
    p.logit_bias = router->logit_bias;
    p.eps = router->eps;
    p.pool_base = (const uint8_t*)pool->base;
    p.expert_stride = pool->expert_stride;
    p.gate_off = pool->gate_offset;
    p.up_off = pool->up_offset;
    p.down_off = pool->down_offset;
    if (shared) {
        p.sh_gate = (const uint8_t*)shared->gate.codes;
        p.sh_up = (const uint8_t*)shared->up.codes;
        p.sh_down = (const uint8_t*)shared->down.codes;
    }
}

// The single-launch decode's regions and unit counts.
void fill_fused(Plan& p, const Sizes& z, uint8_t* ws) {
    const FusedCarve f = fused_carve(z);
    p.f_rpart = (uint64_t*)(ws + f.rpart);
    p.f_hs = (uint64_t*)(ws + f.act);
    p.f_h = p.f_hs + z.Is;
    p.h_stride = f.h_stride;
    p.rpart_stride = f.rpart_stride;
    p.f_piece = (uint64_t*)(ws + f.piece);
    p.f_tail = (uint64_t*)(ws + f.tail);
    p.xw_stride = f.xw_stride;
    uint32_t* ctr = (uint32_t*)(ws + f.ctr);
    p.f_epoch = (uint32_t*)(ws + f.epoch);
    p.f_err = ctr + 2 * kCtrStride;
    p.n_router = z.n_router;
    p.n_sd = z.n_sd;
    p.n_sc = z.n_sc;
    p.n_rh = z.n_rh;
    p.n_src = z.n_src;
}

bool same_sizes(const Sizes& a, const Sizes& b) {
    return a.H == b.H && a.E == b.E && a.k == b.k && a.I == b.I && a.Is == b.Is;
}

// Checks every layer of a stack; all must have the sizes of the first.
mq_status check_stack(int32_t n, const mq_router* routers, const mq_expert_pool* pools, const mq_shared* shared,
                      Sizes* z) {
    if (!routers || !pools) return MQ_ERR_NULL;
    if (n < 1) return MQ_ERR_SHAPE;
    for (int l = 0; l < n; ++l) {
        Sizes zl;
        const mq_status st = check_layer(routers + l, pools + l, shared ? shared + l : nullptr, &zl);
        if (st != MQ_OK) return st;
        if (l == 0)
            *z = zl;
        else if (!same_sizes(*z, zl))
            return MQ_ERR_SHAPE;
    }
    return MQ_OK;
}

size_t stack_plans_offset(const Sizes&) { return fused_region_max(); }

static_assert(sizeof(Plan) + sizeof(StackChunk) + sizeof(Plan*) <= 4096, "k_stack_plans arguments exceed 4 KiB");

// The per-layer arguments follow the decode state; the total also covers a
// one-token moe_layer_forward on the same workspace.
size_t stack_bytes(Sizes z, int32_t n, bool has_shared) {
    set_tiles(&z, 1, has_shared);
    return std::max(stack_plans_offset(z) + up((size_t)n * sizeof(Plan)), carve(z, 1).total);
}

}  // namespace

extern "C" size_t mq_workspace_bytes(const mq_router* router, const mq_expert_pool* pool, const mq_shared* shared,
                                     int32_t max_tokens) {
    Sizes z;
    if (max_tokens < 0 || check_layer(router, pool, shared, &z) != MQ_OK) return 0;
    int64_t T = max_tokens > 0 ? max_tokens : 1;
    set_tiles(&z, T, shared != nullptr);
    return carve(z, T).total;
}

constexpr int kTailMaxH = 16384;   // the tail kernels' row length

// Checks a layer tail against the layer's hidden size.
mq_status check_tail(const mq_tail* t, int H) {
    if (!t) return MQ_OK;
    if (H > kTailMaxH) return MQ_ERR_UNSUPPORTED;
    if (!(t->eps >= 0.f) || !(t->eps < INFINITY) || !(fabsf(t->layer_scalar) < INFINITY)) return MQ_ERR_UNSUPPORTED;
    const float* w[3] = {t->norm_shared, t->norm_routed, t->norm_out};
    for (const float* q : w)
        if (q && !aligned(q, 16)) return MQ_ERR_ALIGN;
    if (!t->residual_is_input && t->residual) {
        if (!aligned(t->residual, 8) || t->residual_stride % 4) return MQ_ERR_ALIGN;
        if (t->residual_stride < H) return MQ_ERR_SHAPE;
    }
    return MQ_OK;
}

// The tail's fields of a plan; x_rows/x_stride are the layer's input rows as
// given (the residual when residual_is_input).
void fill_tail(Plan& p, const mq_tail* t, const uint16_t* x_rows, int64_t x_stride) {
    p.tail = t != nullptr;
    if (!t) return;
    p.tn_s = t->norm_shared;
    p.tn_r = t->norm_routed;
    p.tn_o = t->norm_out;
    p.t_eps = t->eps;
    p.t_scalar = t->layer_scalar;
    p.t_res_in = t->residual_is_input != 0;
    if (p.t_res_in) {
        p.t_res = x_rows;
        p.t_res_stride = x_stride;
    } else {
        p.t_res = (const uint16_t*)t->residual;
        p.t_res_stride = t->residual_stride;
    }
}

// One layer call on the scratch region ws of ws_bytes bytes (the caller's
// workspace, or the static scratch of the allocation-free entry point).
static mq_status layer_forward(const mq_act* x, const mq_router* router, const mq_expert_pool* pool,
                               const mq_shared* shared, mq_act* out, const mq_opts* opts, void* ws_ptr,
                               size_t ws_bytes, void* stream) {
    if (!x || !out || !opts) return MQ_ERR_NULL;
    Sizes z;
    mq_status st = check_layer(router, pool, shared, &z);
    if (st != MQ_OK) return st;
    const int T = x->tokens;
    if (T < 0 || out->tokens != T || x->hidden != z.H || out->hidden != z.H) return MQ_ERR_SHAPE;
    if (x->dtype != MQ_DTYPE_BF16 || (out->dtype != MQ_DTYPE_BF16 && out->dtype != MQ_DTYPE_F32))
        return MQ_ERR_UNSUPPORTED;
    if (x->row_stride < x->hidden || out->row_stride < out->hidden) return MQ_ERR_SHAPE;
    if (opts->path < MQ_PATH_AUTO || opts->path > MQ_PATH_FUSED) return MQ_ERR_UNSUPPORTED;
    if (opts->path == MQ_PATH_FUSED && T > 1) return MQ_ERR_UNSUPPORTED;
    // the single-launch and grouped kernels take 4-bit experts only
    if ((opts->path == MQ_PATH_FUSED || opts->path == MQ_PATH_GROUPED) && z.ebits != 4) return MQ_ERR_UNSUPPORTED;
    // given routing and the experts-ready event: GEMV kernels only
    const bool given = opts->route_ids != nullptr;
    if (given != (opts->route_w != nullptr) || (opts->route_slots && !given)) return MQ_ERR_NULL;
    if ((given || opts->experts_ready) && opts->path != MQ_PATH_AUTO && opts->path != MQ_PATH_GEMV)
        return MQ_ERR_UNSUPPORTED;
    const float in_eps = opts->input_rmsnorm_eps;
    if (!(in_eps >= 0.f) || !(in_eps < INFINITY)) return MQ_ERR_UNSUPPORTED;
    st = check_tail(opts->tail, z.H);
    if (st != MQ_OK) return st;
    if (T == 0) return MQ_OK;
    if (!x->data || !out->data || !ws_ptr) return x->data && out->data ? MQ_ERR_WORKSPACE : MQ_ERR_NULL;
    if (!aligned(x->data, 16) || x->row_stride % 8) return MQ_ERR_ALIGN;
    if (!aligned(out->data, 4) || !aligned(ws_ptr, kAlign)) return MQ_ERR_ALIGN;
    set_tiles(&z, T, shared != nullptr);
    Carve c = carve(z, T);
    if (ws_bytes < c.total) return MQ_ERR_WORKSPACE;

    uint8_t* ws = (uint8_t*)ws_ptr;
    Plan p;
    memset(&p, 0, sizeof(p));
    p.T = T;
    fill_layer(p, z, router, pool, shared);
    p.x = (const uint16_t*)x->data;
    p.x_stride = x->row_stride;
    fill_tail(p, opts->tail, p.x, p.x_stride);
    p.out = out->data;
    p.out_stride = out->row_stride;
    p.out_f32 = out->dtype == MQ_DTYPE_F32;
    p.ids_out = opts->topk_ids;
    p.w_out = opts->topk_w;
    p.logits_out = opts->logits;
    p.r = (float*)(ws + c.r);
    p.rsum8 = (float*)(ws + c.rsum8);
    p.xsum4 = (float*)(ws + c.xsum4);
    p.xsum8 = (float*)(ws + c.xsum8);
    p.plog = (float*)(ws + c.plog);
    p.ids = (int32_t*)(ws + c.ids);
    p.wts = (float*)(ws + c.wts);
    p.hhi = (uint16_t*)(ws + c.hhi);
    p.hlo = (uint16_t*)(ws + c.hlo);
    p.hsum = (float*)(ws + c.hsum);
    p.shi = (uint16_t*)(ws + c.shi);
    p.slo = (uint16_t*)(ws + c.slo);
    p.ssum = (float*)(ws + c.ssum);
    p.dpart = (float*)(ws + c.dpart);
    p.counts = (int32_t*)(ws + c.counts);
    p.offsets = (int32_t*)(ws + c.offsets);
    p.perm = (int32_t*)(ws + c.perm);
    p.inv = (int32_t*)(ws + c.inv);
    p.sched = (int2*)(ws + c.sched);
    p.nsched = (int32_t*)(ws + c.nsched);
    p.gdone = (int32_t*)(ws + c.gdone);
    p.gqueue = (int32_t*)(ws + c.gqueue);
    p.hg = (_Float16*)(ws + c.hg);
    p.hso = (float*)(ws + c.hso);
    p.ysort = (float*)(ws + c.ysort);
    p.max_tiles = z.max_tiles;
    p.ntile = z.ntile;
    p.n_vs = z.n_vs;
    p.n_vs_dn = grouped_shared_rows(z.ntile, z.n_vs);

    fill_fused(p, z, ws);

    hipStream_t s = (hipStream_t)stream;
    (void)hipGetLastError();
    int cus = 0;
    const bool gemv_only = given || opts->experts_ready;
    if (opts->path == MQ_PATH_FUSED || (opts->path == MQ_PATH_AUTO && T == 1 && !gemv_only)) {
        cus = device_cus();
        if (cus <= 0) return MQ_ERR_HIP;
        if (opts->path == MQ_PATH_FUSED && !fused_ok(z, cus)) return MQ_ERR_UNSUPPORTED;
    }
    const bool fused =
        opts->path == MQ_PATH_FUSED || (opts->path == MQ_PATH_AUTO && T == 1 && !gemv_only && fused_ok(z, cus));
    p.n_rng = fused ? fused_ranges(z, cus) : 0;
    p.nwg = fused ? cus : 0;
    p.in_eps = fused ? in_eps : 0.f;
    if (!fused && in_eps > 0.f) {   // normalise into the workspace, then run on that
        uint16_t* xn = (uint16_t*)(ws + c.xn);
        hipLaunchKernelGGL(k_rmsnorm, dim3(T), dim3(256), 0, s, p.x, p.x_stride, xn, (int64_t)z.H, z.H, in_eps);
        p.x = xn;
        p.x_stride = z.H;
    }
    if (fused) {
        hipLaunchKernelGGL(p.tail ? k_decode_tail : k_decode, dim3(cus), dim3(1024), 0, s, p);
        return hipGetLastError() == hipSuccess ? MQ_OK : MQ_ERR_HIP;
    }
    // the grouped kernels take 4-bit experts; AUTO runs 8-bit experts on the GEMV kernels at any T
    const bool grouped =
        opts->path == MQ_PATH_GROUPED || (opts->path == MQ_PATH_AUTO && T > 4 && z.ebits == 4 && !gemv_only);
    if (grouped && (z.ebits != 4 || !grouped_ok(z.H, z.I, T, z.k + z.n_vs))) return MQ_ERR_UNSUPPORTED;
    if (grouped) {
        p.x16 = (_Float16*)(ws + c.x16);
        p.xso = (float*)(ws + c.xso);
        // column splits of the router scores: about 512 workgroups over
        // (16-token tiles) x (64-expert row tiles), at most rsplit and 16,
        // none empty
        const int64_t tiles = ((T + 15) / 16) * (z.E_pad / 64);
        int ks = (int)std::min<int64_t>(std::min(z.rsplit, 16), std::max<int64_t>(1, (512 + tiles - 1) / tiles));
        const int gpw = (z.G_H + ks - 1) / ks;
        p.rsplit_used = (z.G_H + gpw - 1) / gpw;
    }

    if (grouped) {
        st = launch_grouped(p, s);
        if (st != MQ_OK) return st;
    } else {
        hipLaunchKernelGGL(k_prep, dim3(T), dim3(256), 0, s, p);
        if (given) {
            p.ids = const_cast<int32_t*>(opts->route_ids);
            p.wts = const_cast<float*>(opts->route_w);
            p.slots = opts->route_slots;
        } else {
            hipLaunchKernelGGL(k_router, dim3(z.E_pad / 64, z.rsplit, (T + kRouterTokens - 1) / kRouterTokens),
                               dim3(256), 0, s, p);
            hipLaunchKernelGGL(k_topk, dim3(T), dim3(256), 0, s, p);
        }
        auto gateup = z.ebits == 8 ? k_gateup8 : k_gateup;
        auto down = z.ebits == 8 ? k_down8 : k_down;
        const int routed_items = z.k * (z.I / 64), shared_items = z.Is / 64;
        if (opts->experts_ready) {
            // the shared expert (its gate/up items and the last down split)
            // first, then the routed experts once the event has completed
            if (shared_items > 0) {
                p.gu_item0 = routed_items;
                hipLaunchKernelGGL(gateup, dim3(T, shared_items), dim3(256), 0, s, p);
                p.dn_split0 = kDownSplits - 1;
                hipLaunchKernelGGL(down, dim3(T, z.H / 64, 1), dim3(256), 0, s, p);
            }
            if (hipStreamWaitEvent(s, (hipEvent_t)opts->experts_ready, 0) != hipSuccess) return MQ_ERR_HIP;
            p.gu_item0 = 0;
            hipLaunchKernelGGL(gateup, dim3(T, routed_items), dim3(256), 0, s, p);
            p.dn_split0 = 0;
            hipLaunchKernelGGL(down, dim3(T, z.H / 64, shared_items > 0 ? kDownSplits - 1 : kDownSplits), dim3(256),
                               0, s, p);
        } else {
            hipLaunchKernelGGL(gateup, dim3(T, routed_items + shared_items), dim3(256), 0, s, p);
            hipLaunchKernelGGL(down, dim3(T, z.H / 64, kDownSplits), dim3(256), 0, s, p);
        }
        if (p.tail)
            hipLaunchKernelGGL(k_tail_gemv, dim3(T), dim3(1024), 0, s, p);
        else
            hipLaunchKernelGGL(k_combine, dim3(T, (z.H + 255) / 256), dim3(256), 0, s, p);
    }
    return hipGetLastError() == hipSuccess ? MQ_OK : MQ_ERR_HIP;
}

extern "C" mq_status moe_layer_forward(const mq_act* x, const mq_router* router, const mq_expert_pool* pool,
                                       const mq_shared* shared, mq_act* out, const mq_opts* opts, void* stream) {
    if (!opts) return MQ_ERR_NULL;
    return layer_forward(x, router, pool, shared, out, opts, opts->workspace, opts->workspace_bytes, stream);
}

// ---------------------------------------------------------------- allocation-free entry point
//
// moe_layer_forward_noalloc runs the same kernels on a fixed scratch array
// in device memory instead of a caller workspace, for callers that cannot
// allocate.  Each device that the library runs on holds its own copy of
// `scratch` until the process ends.  In host code the array's name only
// stands for the symbol: its device address comes from hipGetSymbolAddress,
// taken once per device with that device current, and only that address is
// ever passed to kernels.

constexpr size_t kScratchBytes = (size_t)40 << 20;   // every call of up to 128 tokens of the Gemma-shaped layer

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];     // device address of `scratch`, per device
bool g_scratch_clear[kMaxDevices];    // cleared once before its first use
}  // namespace

__global__ void k_zero_fill(uint4* p, int64_t n16) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = make_uint4(0, 0, 0, 0);
}

// The current device's scratch address; on the first call on a device the
// array is zero-filled on `s` (a fill kernel, never a memset node).  That
// first call must not be under stream capture: a captured clear would run
// again at every replay and reset the state that later calls depend on.
static mq_status device_scratch(hipStream_t s, void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MQ_ERR_HIP;
    if (dev >= kMaxDevices) return MQ_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return MQ_ERR_HIP;
        g_scratch_ptr[dev] = ptr;
    }
    if (!g_scratch_clear[dev]) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(s, &cs) != hipSuccess) return MQ_ERR_HIP;
        if (cs != hipStreamCaptureStatusNone) return MQ_ERR_UNSUPPORTED;
        hipLaunchKernelGGL(k_zero_fill, dim3(1024), dim3(256), 0, s, (uint4*)g_scratch_ptr[dev],
                           (int64_t)(kScratchBytes / 16));
        if (hipGetLastError() != hipSuccess) return MQ_ERR_HIP;
        g_scratch_clear[dev] = true;
    }
    *out = g_scratch_ptr[dev];
    return MQ_OK;
}

extern "C" size_t mq_noalloc_scratch_bytes(void) { return kScratchBytes; }

extern "C" mq_status moe_layer_forward_noalloc(const mq_act* x, const mq_router* router,
                                               const mq_expert_pool* pool, const mq_shared* shared, mq_act* out,
                                               const mq_opts* opts, void* stream) {
    if (!x || !out || !opts) return MQ_ERR_NULL;
    if (x->tokens == 0) return layer_forward(x, router, pool, shared, out, opts, nullptr, 0, stream);
    const size_t need = mq_workspace_bytes(router, pool, shared, x->tokens > 0 ? x->tokens : 1);
    if (need == 0) return layer_forward(x, router, pool, shared, out, opts, nullptr, 0, stream);
    if (need > kScratchBytes) return MQ_ERR_TOO_LARGE;
    (void)hipGetLastError();
    void* ws = nullptr;
    const mq_status st = device_scratch((hipStream_t)stream, &ws);
    if (st != MQ_OK) return st;
    return layer_forward(x, router, pool, shared, out, opts, ws, kScratchBytes, stream);
}

extern "C" size_t mq_stack_workspace_bytes(const mq_router* routers, const mq_expert_pool* pools,
                                           const mq_shared* shared, int32_t n_layers) {
    Sizes z;
    if (check_stack(n_layers, routers, pools, shared, &z) != MQ_OK) return 0;
    return stack_bytes(z, n_layers, shared != nullptr);
}

extern "C" mq_status moe_stack_forward(const mq_act* x, int32_t n_layers, const mq_router* routers,
                                       const mq_expert_pool* pools, const mq_shared* shared, float between_eps,
                                       mq_act* out, const mq_opts* opts, void* stream) {
    if (!x || !out || !opts) return MQ_ERR_NULL;
    Sizes z;
    mq_status st = check_stack(n_layers, routers, pools, shared, &z);
    if (st != MQ_OK) return st;
    if (x->tokens != 1 || out->tokens != 1 || x->hidden != z.H || out->hidden != z.H) return MQ_ERR_SHAPE;
    if (x->dtype != MQ_DTYPE_BF16 || (out->dtype != MQ_DTYPE_BF16 && out->dtype != MQ_DTYPE_F32))
        return MQ_ERR_UNSUPPORTED;
    if (opts->path != MQ_PATH_AUTO && opts->path != MQ_PATH_FUSED) return MQ_ERR_UNSUPPORTED;
    const float in_eps = opts->input_rmsnorm_eps;
    if (!(in_eps >= 0.f) || !(in_eps < INFINITY) || !(between_eps >= 0.f) || !(between_eps < INFINITY))
        return MQ_ERR_UNSUPPORTED;
    if (opts->tail)
        for (int l = 0; l < n_layers; ++l) {
            st = check_tail(opts->tail + l, z.H);
            if (st != MQ_OK) return st;
            if (l > 0 && !opts->tail[l].residual_is_input && opts->tail[l].residual) return MQ_ERR_UNSUPPORTED;
        }
    if (!x->data || !out->data || !opts->workspace) return x->data && out->data ? MQ_ERR_WORKSPACE : MQ_ERR_NULL;
    if (!aligned(x->data, 16) || !aligned(out->data, 4) || !aligned(opts->workspace, kAlign)) return MQ_ERR_ALIGN;
    if (opts->workspace_bytes < stack_bytes(z, n_layers, shared != nullptr)) return MQ_ERR_WORKSPACE;
    (void)hipGetLastError();
    const int cus = device_cus();
    if (cus <= 0) return MQ_ERR_HIP;
    if (!fused_ok(z, cus)) return MQ_ERR_UNSUPPORTED;

    uint8_t* ws = (uint8_t*)opts->workspace;
    Plan base;
    memset(&base, 0, sizeof(base));
    base.T = 1;
    fill_layer(base, z, routers, pools, shared);
    fill_fused(base, z, ws);
    base.n_rng = fused_ranges(z, cus);
    base.nwg = cus;
    base.x_stride = x->row_stride;
    base.out_stride = out->row_stride;
    base.out_f32 = out->dtype == MQ_DTYPE_F32;
    uint64_t* xw = (uint64_t*)(ws + fused_carve(z).xw);
    Plan* plans = (Plan*)(ws + stack_plans_offset(z));
    hipStream_t s = (hipStream_t)stream;
    for (int l0 = 0; l0 < n_layers; l0 += kStackChunk) {
        StackChunk c;
        memset(&c, 0, sizeof(c));
        c.n = std::min(kStackChunk, n_layers - l0);
        for (int i = 0; i < c.n; ++i) {
            const int l = l0 + i;
            StackLayer& L = c.l[i];
            const mq_router& r = routers[l];
            const mq_expert_pool& pl = pools[l];
            L.x = l == 0 ? (const uint16_t*)x->data : nullptr;
            L.x_w = l == 0 ? nullptr : xw;
            L.out = l == n_layers - 1 ? out->data : nullptr;
            L.out_w = l == n_layers - 1 ? nullptr : xw;
            L.router_w = (const uint8_t*)r.w.codes;
            L.router_scale = r.router_scale;
            L.pes = r.per_expert_scale;
            L.logit_bias = r.logit_bias;
            L.eps = r.eps;
            L.in_eps = l == 0 ? in_eps : between_eps;
            L.pool_base = (const uint8_t*)pl.base;
            L.expert_stride = pl.expert_stride;
            L.gate_off = pl.gate_offset;
            L.up_off = pl.up_offset;
            L.down_off = pl.down_offset;
            if (shared) {
                L.sh_gate = (const uint8_t*)shared[l].gate.codes;
                L.sh_up = (const uint8_t*)shared[l].up.codes;
                L.sh_down = (const uint8_t*)shared[l].down.codes;
            }
            if (opts->tail) {
                const mq_tail& t = opts->tail[l];
                L.tail = 1;
                L.tn_s = t.norm_shared;
                L.tn_r = t.norm_routed;
                L.tn_o = t.norm_out;
                L.t_eps = t.eps;
                L.t_scalar = t.layer_scalar;
                L.t_res_in = t.residual_is_input != 0;
                L.t_res = l == 0 && !L.t_res_in ? (const uint16_t*)t.residual : nullptr;
                L.t_res_stride = t.residual_stride;
            }
            L.ids_out = opts->topk_ids ? opts->topk_ids + (int64_t)l * z.k : nullptr;
            L.w_out = opts->topk_w ? opts->topk_w + (int64_t)l * z.k : nullptr;
            L.logits_out = opts->logits ? opts->logits + (int64_t)l * z.E : nullptr;
        }
        hipLaunchKernelGGL(k_stack_plans, dim3(c.n), dim3(64), 0, s, base, c, plans + l0);
    }
    hipLaunchKernelGGL(opts->tail ? k_decode_stack_tail : k_decode_stack, dim3(cus), dim3(1024), 0, s,
                       (const Plan*)plans, (int)n_layers);
    return hipGetLastError() == hipSuccess ? MQ_OK : MQ_ERR_HIP;
}

// ---------------------------------------------------------------- routing only

// Workspace carve of mq_route for T tokens (router input, its lane sums, the
// column splits' partial scores).
struct RouteCarve {
    size_t r, rsum8, xsum4, plog, total;
};

static RouteCarve route_carve(int H, int E, int64_t T) {
    RouteCarve c;
    size_t o = 0;
    auto take = [&](size_t bytes) { size_t at = o; o += up(bytes); return at; };
    const int G_H = H / kGroup, rsplit = (G_H + 3) / 4;
    c.r = take(T * H * 4);
    c.rsum8 = take(T * G_H * 16);
    c.xsum4 = take(T * G_H * 16);
    c.plog = take((size_t)rsplit * T * pad_rows(E) * 4);
    c.total = o;
    return c;
}

static mq_status check_router(const mq_router* rt, int H) {
    if (!rt) return MQ_ERR_NULL;
    if (!rt->w.codes) return MQ_ERR_NULL;
    if (rt->w.bits != 8 || rt->w.group <= 0 || rt->w.group % kGroup || rt->w.layout != MQ_LAYOUT_DEV_V1)
        return MQ_ERR_UNSUPPORTED;
    const int E = rt->w.rows;
    if (H <= 0 || H % kGroup || rt->w.cols != H || !group_ok(H, rt->w.group) || E <= 0 || E > kMaxExperts)
        return MQ_ERR_SHAPE;
    if (rt->top_k < 1 || rt->top_k > E || rt->top_k > kMaxTopK || !(rt->eps >= 0.f)) return MQ_ERR_SHAPE;
    if (!aligned(rt->w.codes, kAlign)) return MQ_ERR_ALIGN;
    if (rt->router_scale && !aligned(rt->router_scale, 16)) return MQ_ERR_ALIGN;
    return MQ_OK;
}

extern "C" size_t mq_route_workspace_bytes(const mq_router* router, int32_t max_tokens) {
    if (!router || max_tokens < 0 || check_router(router, router->w.cols) != MQ_OK) return 0;
    return route_carve(router->w.cols, router->w.rows, max_tokens > 0 ? max_tokens : 1).total;
}

extern "C" mq_status mq_route(const mq_act* x, const mq_router* router, int32_t* ids, float* w, float* logits,
                              void* workspace, size_t workspace_bytes, void* stream) {
    if (!x || !router) return MQ_ERR_NULL;
    const int H = x->hidden, T = x->tokens;
    mq_status st = check_router(router, H);
    if (st != MQ_OK) return st;
    if (T < 0 || x->row_stride < H) return MQ_ERR_SHAPE;
    if (x->dtype != MQ_DTYPE_BF16) return MQ_ERR_UNSUPPORTED;
    if (T == 0) return MQ_OK;
    if (!x->data || !ids || !w) return MQ_ERR_NULL;
    if (!workspace) return MQ_ERR_WORKSPACE;
    if (!aligned(x->data, 16) || x->row_stride % 8 || !aligned(workspace, kAlign)) return MQ_ERR_ALIGN;
    const RouteCarve c = route_carve(H, router->w.rows, T);
    if (workspace_bytes < c.total) return MQ_ERR_WORKSPACE;
    uint8_t* ws = (uint8_t*)workspace;
    Plan p;
    memset(&p, 0, sizeof(p));
    p.T = T;
    p.H = H;
    p.E = router->w.rows;
    p.E_pad = (int)pad_rows(p.E);
    p.k = router->top_k;
    p.G_H = H / kGroup;
    p.rgroups = 4;
    p.rsplit = (p.G_H + p.rgroups - 1) / p.rgroups;
    p.ebits = 4;
    p.router_w = (const uint8_t*)router->w.codes;
    p.router_scale = router->router_scale;
    p.pes = router->per_expert_scale;
    p.logit_bias = router->logit_bias;
    p.eps = router->eps;
    p.x = (const uint16_t*)x->data;
    p.x_stride = x->row_stride;
    p.r = (float*)(ws + c.r);
    p.rsum8 = (float*)(ws + c.rsum8);
    p.xsum4 = (float*)(ws + c.xsum4);
    p.plog = (float*)(ws + c.plog);
    p.ids = ids;
    p.wts = w;
    p.logits_out = logits;
    hipStream_t s = (hipStream_t)stream;
    (void)hipGetLastError();
    hipLaunchKernelGGL(k_prep, dim3(T), dim3(256), 0, s, p);
    hipLaunchKernelGGL(k_router, dim3(p.E_pad / 64, p.rsplit, (T + kRouterTokens - 1) / kRouterTokens), dim3(256), 0,
                       s, p);
    hipLaunchKernelGGL(k_topk, dim3(T), dim3(256), 0, s, p);
    return hipGetLastError() == hipSuccess ? MQ_OK : MQ_ERR_HIP;
}

extern "C" mq_status mq_workspace_errors(const void* workspace, size_t workspace_bytes, uint32_t* errors,
                                         void* stream) {
    if (!workspace || !errors) return MQ_ERR_NULL;
    if (!aligned(workspace, kAlign)) return MQ_ERR_ALIGN;
    // the error flag sits at a fixed offset at the start of every workspace
    const size_t at = 2 * kCtrStride * sizeof(uint32_t);
    if (workspace_bytes < at + sizeof(uint32_t)) return MQ_ERR_WORKSPACE;
    (void)hipGetLastError();
    hipStream_t s = (hipStream_t)stream;
    if (hipMemcpyAsync(errors, (const uint8_t*)workspace + at, sizeof(uint32_t), hipMemcpyDeviceToHost, s) !=
            hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return MQ_ERR_HIP;
    return MQ_OK;
}

extern "C" mq_status mq_rmsnorm(const mq_act* x, mq_act* out, float eps, void* stream) {
    if (!x || !out) return MQ_ERR_NULL;
    if (x->dtype != MQ_DTYPE_BF16 || out->dtype != MQ_DTYPE_BF16) return MQ_ERR_UNSUPPORTED;
    if (x->tokens != out->tokens || x->hidden != out->hidden || x->tokens < 0 || x->hidden <= 0 ||
        x->row_stride < x->hidden || out->row_stride < out->hidden || !(eps >= 0.f))
        return MQ_ERR_SHAPE;
    if (x->tokens == 0) return MQ_OK;
    if (!x->data || !out->data) return MQ_ERR_NULL;
    if (!aligned(x->data, 2) || !aligned(out->data, 2)) return MQ_ERR_ALIGN;
    (void)hipGetLastError();
    hipLaunchKernelGGL(k_rmsnorm, dim3(x->tokens), dim3(256), 0, (hipStream_t)stream, (const uint16_t*)x->data,
                       x->row_stride, (uint16_t*)out->data, out->row_stride, x->hidden, eps);
    return hipGetLastError() == hipSuccess ? MQ_OK : MQ_ERR_HIP;
}

static mq_status debug_read(const mq_qtensor* t, uint8_t* codes_out, float* w_out, void* stream) {
    if (!t || !t->codes || (!codes_out && !w_out)) return MQ_ERR_NULL;
    if (!(t->bits == 4 || t->bits == 8) || t->group <= 0 || t->group % kGroup || t->layout != MQ_LAYOUT_DEV_V1)
        return MQ_ERR_UNSUPPORTED;
    if (t->rows <= 0 || t->cols <= 0 || t->cols % t->group) return MQ_ERR_SHAPE;
    if (!aligned(t->codes, 16)) return MQ_ERR_ALIGN;
    const int blocks = (int)(pad_rows(t->rows) / kTileRows) * (t->cols / kGroup);
    (void)hipGetLastError();
    hipLaunchKernelGGL(k_debug_read, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const uint8_t*)t->codes,
                       t->rows, t->cols, t->bits, codes_out, w_out);
    return hipGetLastError() == hipSuccess ? MQ_OK : MQ_ERR_HIP;
}

extern "C" mq_status mq_debug_unpack_codes(const mq_qtensor* t, uint8_t* codes_out, void* stream) {
    if (!codes_out) return MQ_ERR_NULL;
    return debug_read(t, codes_out, nullptr, stream);
}

extern "C" mq_status mq_debug_dequant(const mq_qtensor* t, float* w_out, void* stream) {
    if (!w_out) return MQ_ERR_NULL;
    return debug_read(t, nullptr, w_out, stream);
}

extern "C" mq_status mq_stream_read(const void* buf, size_t bytes, uint32_t* sink, int32_t workgroups,
                                    void* stream) {
    if (!buf || !sink) return MQ_ERR_NULL;
    if (!aligned(buf, 16) || bytes % 16) return MQ_ERR_ALIGN;
    if (workgroups < 1 || bytes == 0) return MQ_ERR_SHAPE;
    (void)hipGetLastError();
    hipLaunchKernelGGL(k_stream_read, dim3(workgroups), dim3(256), 0, (hipStream_t)stream, (const uint4*)buf,
                       (int64_t)(bytes / 16), sink);
    return hipGetLastError() == hipSuccess ? MQ_OK : MQ_ERR_HIP;
}

extern "C" size_t mq_qgemv_workspace_bytes(int32_t rows, int32_t tokens) {
    if (rows <= 0 || tokens < 0 || tokens > kHeadTokens) return 0;
    return up((size_t)std::max(tokens, 1) * head_groups(rows) * sizeof(float2));
}

extern "C" mq_status mq_qgemv(const mq_qtensor* w, const mq_act* x, mq_act* y, float softcap, int32_t* argmax,
                              void* workspace, size_t workspace_bytes, void* stream) {
    if (!w || !x) return MQ_ERR_NULL;
    if (!w->codes) return MQ_ERR_NULL;
    if (!(w->bits == 4 || w->bits == 8) || w->group <= 0 || w->group % kGroup || w->layout != MQ_LAYOUT_DEV_V1)
        return MQ_ERR_UNSUPPORTED;
    if (w->rows <= 0 || w->cols <= 0 || w->cols % w->group) return MQ_ERR_SHAPE;
    const int T = x->tokens;
    if (T < 0 || x->hidden != w->cols || x->row_stride < x->hidden) return MQ_ERR_SHAPE;
    if (x->dtype != MQ_DTYPE_BF16) return MQ_ERR_UNSUPPORTED;
    if (T > kHeadTokens || head_lds_bytes(T, w->cols) > (size_t)kHeadLdsBytes) return MQ_ERR_UNSUPPORTED;
    if (y && (y->tokens != T || y->hidden != w->rows || y->row_stride < y->hidden)) return MQ_ERR_SHAPE;
    if (y && y->dtype != MQ_DTYPE_BF16 && y->dtype != MQ_DTYPE_F32) return MQ_ERR_UNSUPPORTED;
    if (!(softcap >= 0.f) || !(softcap < INFINITY)) return MQ_ERR_UNSUPPORTED;
    if (!y && !argmax) return MQ_ERR_NULL;
    if (T == 0) return MQ_OK;
    if (!x->data || (y && !y->data)) return MQ_ERR_NULL;
    if (!aligned(w->codes, 16) || !aligned(x->data, 16) || x->row_stride % 8) return MQ_ERR_ALIGN;
    if (y && !aligned(y->data, 4)) return MQ_ERR_ALIGN;
    if (argmax) {
        if (!workspace) return MQ_ERR_WORKSPACE;
        if (!aligned(workspace, 16)) return MQ_ERR_ALIGN;
        if (workspace_bytes < mq_qgemv_workspace_bytes(w->rows, T)) return MQ_ERR_WORKSPACE;
    }
    HeadArgs a;
    memset(&a, 0, sizeof(a));
    a.w = (const uint8_t*)w->codes;
    a.rows = w->rows;
    a.cols = w->cols;
    a.bits = w->bits;
    a.T = T;
    a.x = (const uint16_t*)x->data;
    a.x_stride = x->row_stride;
    a.y = y ? y->data : nullptr;
    a.y_stride = y ? y->row_stride : 0;
    a.y_f32 = y && y->dtype == MQ_DTYPE_F32;
    a.cap = softcap;
    a.part = argmax ? (float2*)workspace : nullptr;
    (void)hipGetLastError();
    return launch_head(a, argmax, (hipStream_t)stream);
}

extern "C" const char* mq_status_str(mq_status s) {
    switch (s) {
        case MQ_OK: return "ok";
        case MQ_ERR_NULL: return "required pointer is NULL";
        case MQ_ERR_SHAPE: return "inconsistent or unsupported sizes";
        case MQ_ERR_ALIGN: return "misaligned pointer, offset or stride";
        case MQ_ERR_UNSUPPORTED: return "unsupported bits, group, layout, dtype or path";
        case MQ_ERR_WORKSPACE: return "workspace missing or too small";
        case MQ_ERR_HIP: return "HIP runtime error";
        case MQ_ERR_BUFFER: return "host buffer too small";
        case MQ_ERR_TOO_LARGE: return "the call needs more scratch than the fixed static buffer holds";
    }
    return "unknown status";
}
