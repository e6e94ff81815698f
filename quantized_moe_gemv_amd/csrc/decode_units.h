// Single-launch decode of one token through the whole layer.
//
// The layer is cut into units of weight streaming, given to one workgroup
// per compute unit:
//   without expert ids: router pieces    16 experts x a column range  -> partial scores
//                       shared gate/up   32 rows x all columns         -> h (shared)
//                       shared down      64 output rows x a chunk of Is -> partial outputs
//   with expert ids:    routed gate/up   (slot j, 32 rows, all columns) -> h
//                       routed down      (slot j, a range of output tiles) -> partial outputs
//                       output sums      (64 output rows, every source) -> out
// Full-row gate/up units hold complete sums, so only the router scores, the
// activations and the partial outputs cross between workgroups.  A
// workgroup puts out the loads of all its units that need no expert ids at
// once, and those of the rest as soon as it knows the ids, so the memory
// system has its whole remaining stream in flight; the units are computed as
// their data lands.  Each wait is bounded.  Partial results are
// 64-bit words carrying the call's epoch in their high half: a reader
// issues all of its loads, then re-reads only the words whose tag is not yet
// current.  Each sum has a fixed reducer which sums in a fixed order, so
// results repeat bit for bit.
//
// Results that many workgroups read (partial router scores, GeGLU
// activations) are written once per XCD (eight copies) and each reader takes
// the copy of its own XCD, so the readers do not all queue on the same
// memory channels.  Every workgroup that runs routed units sums the router
// scores and selects the experts itself, which costs less than waiting for
// one workgroup to publish them.
//
// The shared expert and the router do not depend on each other, so the
// shared gate/up streams while the routing decision is made ("Decode",
// phase table: the shared expert overlaps the wait for the expert ids).
#pragma once
#include <math.h>

#include "device.h"
#include "plan.h"

namespace mq {
// Internal linkage: each kernel file compiles its own copy, with its own
// kOpaqueTid, kEarlySharedDown, kLateRoutedDown, kLateSharedGateUp, kSwapKb,
// kSpareGateUpLoads and kTokenFirst (defined before this file is included;
// they change speed only, never the arithmetic).
namespace {

// Sum over the four lanes of a row's column blocks (lane%16 + 16 kb): by
// permlane swaps or through the LDS crossbar, which give the same bits.
__device__ __forceinline__ float row_sum_kb(float v) {
    if constexpr (kSwapKb) return sum_kb(v);
    else return sum_kb_bpermute(v);
}

// 1024 threads: four waves per SIMD, so the dependent chains of one wave
// (dequantisation, dot steps, reductions) are hidden behind the others.
constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kItems = 2;           // 16-byte code loads per lane per unit (<= 32 items)
constexpr int kSpinLimit = 1 << 20;
constexpr int kCopies = 8;         // replicas of broadcast results, one per XCD
constexpr int kItemsRH = 6;        // 16-byte code loads per lane of a full-row gate/up unit (2 G_H <= 96)
constexpr int kSlotsSD = 2;        // shared down pieces of a shared workgroup
constexpr int kTilesD = 3;         // output tiles of a routed down unit
constexpr int kGroupsD = 2;        // column groups per wave pair and tile of a routed down unit (G_I <= 16)
constexpr int kItemsD = kGroupsD * kTilesD;   // 16-byte code loads per lane of a routed down unit
constexpr int kRq = kRouterPieces;

// The copy of a broadcast result that this workgroup reads: the one of the
// XCD it runs on (XCC_ID).  Every copy holds the same words, so the choice
// only decides which memory channels serve the read.
__device__ __forceinline__ int xcc_copy() {
    uint32_t v;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
    return (int)(v & (kCopies - 1));
}

// The thread's index.  With kOpaqueTid it is opaque to the optimiser at each
// use: in the stack kernel's layer loop, index arithmetic is then recomputed
// where it is used instead of being hoisted and held in registers across the
// whole layer (which spills).  The single-layer kernel keeps plain indices.
__device__ __forceinline__ unsigned tix() {
    unsigned t = threadIdx.x;
    if constexpr (kOpaqueTid) asm volatile("" : "+v"(t));
    return t;
}

// ----------------------------------------------------------------- words and counters

__device__ __forceinline__ uint64_t ld_word(const uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_word(uint64_t* p, uint32_t tag, uint32_t payload) {
    __hip_atomic_store(p, ((uint64_t)tag << 32) | payload, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_ctr(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Re-reads the words of v (at p[m * pstride], m < 4) whose tag is not yet
// current, all of them in each round, until every one is.  Bounded: gives
// up after kSpinLimit rounds, or at once when any wait of the call has
// already given up, and records that in *err (bit kErrWait).  Bit m of `want` selects the
// words that take part.
__device__ __forceinline__ void await_words(const uint64_t* p, int pstride, uint64_t v[4], uint32_t want,
                                            uint32_t tag, uint32_t* err) {
    uint32_t stale = 0;
#pragma unroll
    for (int m = 0; m < 4; ++m)
        if (((want >> m) & 1) && (uint32_t)(v[m] >> 32) != tag) stale |= 1u << m;
    int spins = 0;
    while (stale) {
        if (++spins > kSpinLimit || ((spins & 63) == 0 && (ld_ctr(err) & kErrWait))) {
            atomicOr(err, kErrWait);
            break;
        }
        __builtin_amdgcn_s_sleep(2);
#pragma unroll
        for (int m = 0; m < 4; ++m)
            if ((stale >> m) & 1) v[m] = ld_word(p + m * pstride);
#pragma unroll
        for (int m = 0; m < 4; ++m)
            if ((uint32_t)(v[m] >> 32) == tag) stale &= ~(1u << m);
    }
}

// Payload of a word once its tag is current.  Bounded, and gives up at once
// once any wait of the call has failed (recorded in *err).
__device__ __forceinline__ uint32_t wait_word(const uint64_t* p, uint32_t tag, uint32_t* err) {
    uint64_t v = ld_word(p);
    int spins = 0;
    while ((uint32_t)(v >> 32) != tag) {
        if (++spins > kSpinLimit || ((spins & 63) == 0 && (ld_ctr(err) & kErrWait))) {
            atomicOr(err, kErrWait);
            break;
        }
        __builtin_amdgcn_s_sleep(2);
        v = ld_word(p);
    }
    return (uint32_t)v;
}

// Payloads of words base[0 .. n) into dst: every load is issued before any
// is checked, so the gather costs one round trip when the words are there (a
// stale word is then waited for on its own).  Threads t0.. load, for
// n <= 4 (kThreads - t0): t0 > 0 keeps waves that have just published a
// unit's results out of it, since a wave's loads wait for its earlier stores,
// which are written through to memory.
__device__ __forceinline__ void gather_words(const uint64_t* base, int n, uint32_t tag, uint32_t* err,
                                             uint32_t* dst, int t0) {
    if (n <= 0) {
        __syncthreads();
        return;
    }
    const int me = (int)tix() - t0, nthr = kThreads - t0;
    if (me >= 0) {
        uint64_t v[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int i = me + nthr * m;
            v[m] = ld_word(base + (i < n ? i : n - 1));   // unconditional: see issue_loads
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int i = me + nthr * m;
            if (i < n) {
                if ((uint32_t)(v[m] >> 32) != tag) v[m] = ((uint64_t)tag << 32) | wait_word(base + i, tag, err);
                dst[i] = (uint32_t)v[m];
            }
        }
    }
    __syncthreads();
}


// ----------------------------------------------------------------- units

enum { U_ROUTER = 0, U_SH = 1, U_SD = 2, U_RH = 3, U_NONE = 4 };

struct Unit {
    int kind;
    int a, b;         // router: slice; SH: half tile; SD: out tile, chunk; RH: slot, half tile
    int q;            // piece index of the column range (router, gate/up)
    int g0, ng;       // column-group range
};

struct Shared {
    // arrays read with 16-byte LDS accesses come first and stay 16-byte aligned
    alignas(16) uint16_t x[4096];
    alignas(16) uint16_t h16[16 * 64];   // one source's GeGLU activations, fp16
    alignas(16) float lg[256];           // expert scores (padding: -inf)
    alignas(16) uint64_t key[256];       // selection keys (padding: 0)
    alignas(16) float xr[4096];          // router input numerator x * router_scale
    alignas(16) float selv[kMaxTopK];    // selected scores (padding: -inf)
    float pes[256];           // per_expert_scale (1 when absent)
    float lbias[256];         // logit_bias (0 when absent)
    alignas(16) uint32_t gbuf[2048];     // gathered payloads (partial results of other units)
    alignas(16) float xsum[64 * 4];   // x summed over each lane's 16 columns of a group (4-bit blocks)
    float rsum[64 * 4];       // router input summed over each lane's 16 columns (8-bit blocks)
    float c8[512];            // per 8-column chunk: sum of x
    float c4[1024];           // per 4-column quarter: sum of x * router_scale
    float red[kWaves][64];
    float red2[kWaves][kTilesD][32];   // per-wave row sums of a routed down unit
    float hsx[16], hsa[16];   // per staged group: sum of the activations, of the stored operand
    alignas(16) uint16_t hzero[8];       // zeros: the operand lanes that hold no token
    int32_t ids[kMaxTopK];
    float wts[kMaxTopK];
    float rc;                 // router input scale 1/sqrt(mean(x^2)+eps)/sqrt(H)
};
// First loading thread of the activation and output-sum gathers: waves 0
// and 1 publish the units' results (the ids gather, after the router pieces
// publish, measured no faster without them and keeps every thread).
constexpr int kGatherT0 = 128;
static_assert(sizeof(Shared::gbuf) / 4 <= 4 * (kThreads - kGatherT0), "a gather fills gbuf in one round");

// First wave of the down units (shared pieces, routed down units).  Waves 0
// and 1 publish the units' results, and a wave's later loads, and the waits
// the compiler places before it reuses registers, wait for its stores, which
// are written through to memory.  So when the units fit the other waves
// (G_I <= 14: two items per wave of a piece, kGroupsD groups per wave pair),
// those two waves take no part in them, and the output sums run on wave 2.
// (Measured: the lone call 0.25 us faster, the stack launch 4 us per token
// slower; both kernels keep one layout, so that a stack equals chained calls
// bit for bit.)
__device__ __forceinline__ int down_w0(const Plan& p) { return p.G_I <= kGroupsD * (kWaves / 2 - 1) ? 2 : 0; }
constexpr int kSumWave = 2;   // the wave that sums an output tile

// Column range q of nq over G groups.
__device__ __forceinline__ void krange(int G, int nq, int q, int* g0, int* ng) {
    const int a = q * G / nq, b = (q + 1) * G / nq;
    *g0 = a;
    *ng = b - a;
}

__device__ __forceinline__ Unit no_unit() {
    Unit x;
    x.kind = U_NONE;
    x.a = x.b = x.q = x.g0 = x.ng = 0;
    return x;
}

// Router piece i: 16 experts (slice i / 8) x column range i % 8.
__device__ __forceinline__ Unit unit_router(const Plan& p, int i) {
    Unit x = no_unit();
    if (i >= 0 && i < p.n_router) {
        x.kind = U_ROUTER;
        x.a = i / kRq;
        x.q = i % kRq;
        krange(p.G_H, kRq, x.q, &x.g0, &x.ng);
    }
    return x;
}

// Full-row shared gate/up unit i: half tile i of the shared expert, every
// column group.
__device__ __forceinline__ Unit unit_sh(const Plan& p, int i) {
    Unit x = no_unit();
    if (i >= 0 && i < 2 * p.G_s) {
        x.kind = U_SH;
        x.a = i;
        x.ng = p.G_H;
    }
    return x;
}

// Full-row routed gate/up unit w: slot w / (2 G_I), half tile w % (2 G_I),
// every column group.
__device__ __forceinline__ Unit unit_rh(const Plan& p, int w) {
    Unit x = no_unit();
    if (w < p.n_rh) {
        x.kind = U_RH;
        x.a = w / (2 * p.G_I);
        x.b = w % (2 * p.G_I);
        x.ng = p.G_H;
    }
    return x;
}

// Shared down piece i: output tile i / n_sc, chunk i % n_sc of Is.
__device__ __forceinline__ Unit unit_sd(const Plan& p, int i) {
    Unit x = no_unit();
    if (i >= 0 && i < p.n_sd) {
        x.kind = U_SD;
        x.a = i / p.n_sc;
        x.b = i % p.n_sc;
        x.g0 = x.b * p.G_I;
        x.ng = min(p.G_I, p.G_s - x.g0);
    }
    return x;
}

// A routed down unit: one selected expert (slot b) over output tiles
// t0 .. t0+nt-1, so its activations are staged once for all those tiles.
struct DownUnit {
    int b, t0, nt;
};

// Workgroup roles.  Workgroups 0 .. n_rh-1 ("routed") run one full-row
// routed gate/up unit and shared down piece w each; the m = grid - n_rh
// others ("shared") run the full-row shared gate/up units (one each, the
// first 2 G_s of them) and any further shared down pieces.  Routed down
// work: the first S = min(n_rh / G_H, k) slots one tile per routed
// workgroup, the other slots in n_rng tile ranges each on the shared
// workgroups.  The sum of output tile a runs on workgroup a, after all its
// other work, and router piece i on workgroup G_H + i: in a stack of layers
// the workgroups that sum are the last to finish a layer, and the router
// pieces of the next layer then load their weights during that tail.
__device__ __forceinline__ DownUnit unit_rdu(const Plan& p, int w, int nwg) {
    DownUnit d;
    d.b = d.t0 = d.nt = 0;
    const int S = min(p.n_rh / p.G_H, p.k);
    if (w < p.n_rh) {
        if (w < S * p.G_H) {
            d.b = w / p.G_H;
            d.t0 = w % p.G_H;
            d.nt = 1;
        }
        return d;
    }
    const int v = w - p.n_rh;
    if (S < p.k && v < (p.k - S) * p.n_rng) {
        const int r = v % p.n_rng;
        d.b = S + v / p.n_rng;
        d.t0 = r * p.G_H / p.n_rng;
        d.nt = (r + 1) * p.G_H / p.n_rng - d.t0;
    }
    return d;
}

// Shared down piece s of workgroup w: piece w on the routed workgroups, the
// rest (j = n_rh + v + m s for shared workgroup v) on the shared ones.
__device__ __forceinline__ Unit sd_piece(const Plan& p, int w, int nwg, int s) {
    if (w < p.n_rh) return s == 0 ? unit_sd(p, w) : no_unit();
    const int m = nwg - p.n_rh, j = p.n_rh + (w - p.n_rh) + m * s;
    return unit_sd(p, j);
}

// A unit's weight loads, issued before the unit waits or computes.
template <int N>
struct LoadsN {
    uint4 c[N];
    uint2 s[N];
};
typedef LoadsN<kItems> Loads;

__device__ __forceinline__ const uint8_t* tile4(const uint8_t* m, int tile, int G) {
    return m + (int64_t)tile * G * kBlk4;
}

// The loads of one unit.  Within a unit, item it of wave w (it = w + 8m)
// reads the block base[it & 1] + (it >> 1) * step, so each wave needs two
// uniform base pointers, fixed for the unit, and one scalar add per item:
//   router:  it -> 8-bit block (slice rows, group g0 + it)
//   gate/up: even it -> gate, odd it -> up, group g0 + it/2, one half tile
//   down:    group g0 + it/2, rows of half (it & 1) of the output tile
// A wave issues no load for an item past the unit's end (a branch that is
// uniform over the wave, so no register is half written by a load; the
// compute skips those items), and a workgroup without the unit issues
// nothing: every load costs address-unit time and a place in the compute
// unit's queue, which the wanted loads behind it wait through (a router
// piece of 5-6 groups used to load all 32 of its wave slots: stack 529 ->
// 513 us/token, decode 19.27 -> 19.00 us without them).
template <int N>
__device__ __forceinline__ void issue_loads(const Plan& p, const Shared& sh, const Unit& x, LoadsN<N>& L) {
    if (x.kind == U_NONE) return;
    // items of wave w: it = w - w0 + nw m (a shared down piece leaves the
    // waves below down_w0 out)
    const int w0 = x.kind == U_SD ? down_w0(p) : 0, nw = kWaves - w0;
    const int wave = wave_id() - w0, lane = tix() & 63, par = wave & 1;
    if (wave < 0) return;
    const uint8_t* b0 = p.router_w;
    const uint8_t* b1 = p.router_w;
    int64_t step = 0;
    int n = 0, oc = 0, os = kCodes4;
    if (x.kind == U_ROUTER) {
        const int tile = x.a >> 2, j = x.a & 3;
        b0 = p.router_w + ((int64_t)tile * p.G_H + x.g0) * kBlk8;
        b1 = b0 + kBlk8;
        step = 2 * kBlk8;
        n = x.ng;
        oc = j * 1024;
        os = kCodes8 + 8 * (j >> 1);   // pair j is .x (j even) or .y
    } else if (x.kind == U_SH || x.kind == U_RH) {
        const int ht = x.kind == U_SH ? x.a : x.b;
        const uint8_t* g;
        const uint8_t* u;
        if (x.kind == U_SH) {
            g = p.sh_gate;
            u = p.sh_up;
        } else {
            const uint8_t* blob = p.pool_base + (int64_t)sh.ids[x.a] * p.expert_stride;
            g = blob + p.gate_off;
            u = blob + p.up_off;
        }
        const int64_t o = ((int64_t)(ht >> 1) * p.G_H + x.g0) * kBlk4;
        b0 = g + o;
        b1 = u + o;
        step = kBlk4;
        n = 2 * x.ng;
        oc = (ht & 1) * 1024;
        os = kCodes4 + 8 * (ht & 1);
    } else if (x.kind == U_SD) {
        b0 = b1 = p.sh_down + ((int64_t)x.a * p.G_s + x.g0) * kBlk4;
        step = kBlk4;
        n = 2 * x.ng;
        oc = par * 1024;
        os = kCodes4 + 8 * par;
    }
    const uint8_t* wb = (par ? b1 : b0) + (int64_t)(wave >> 1) * step;
    const int lc = oc + lane * 16, ls = os + (lane & 15) * 16;
#pragma unroll
    for (int m = 0; m < N; ++m) {
        // kSpareGateUpLoads: a gate/up unit's waves load every slot (the
        // spare ones from the router's first block), so that every path
        // issues the same number of loads and the compiler can wait for one
        // item at a time
        if ((kSpareGateUpLoads && (x.kind == U_SH || x.kind == U_RH)) || wave + nw * m < n) {
            const uint8_t* blk = wave + nw * m < n ? wb + (int64_t)(nw / 2) * m * step : p.router_w;
            L.c[m] = ld_stream16(blk + lc);
            L.s[m] = *(const uint2*)(blk + ls);
        }
    }
}

// ----------------------------------------------------------------- setup

__device__ __forceinline__ float sum8_bf16(const uint4& v) {
    return ((bf16_lo(v.x) + bf16_hi(v.x)) + (bf16_lo(v.y) + bf16_hi(v.y))) +
           ((bf16_lo(v.z) + bf16_hi(v.z)) + (bf16_lo(v.w) + bf16_hi(v.w)));
}

// The token and the small per-expert vectors, loaded into registers before
// any weight so that they head the memory queues.
struct TokenLoads {
    uint4 x;
    uint64_t xw[4];  // the same columns as tagged bf16 pairs (input published by the previous layer)
    float4 r0, r1;   // router_scale of the thread's 8 columns
    float pes, lb;   // per_expert_scale and logit_bias of expert tix()
    bool need;       // the workgroup runs a unit that reads the token
};

__device__ __forceinline__ void load_token(const Plan& p, TokenLoads& t, bool need) {
    const int c = tix();
    t.x = make_uint4(0, 0, 0, 0);
    t.r0 = t.r1 = make_float4(1.f, 1.f, 1.f, 1.f);
    t.pes = 1.f;
    t.lb = 0.f;
    t.need = need;
    if (c < p.H / 8) {
        if (!need) {
        } else if (p.x_w) {
            const uint64_t* xw = p.x_w + xcc_copy() * p.xw_stride + 4 * c;
#pragma unroll
            for (int i = 0; i < 4; ++i) t.xw[i] = ld_word(xw + i);
        } else {
            t.x = *(const uint4*)(p.x + 8 * c);
        }
        if (p.router_scale) {
            t.r0 = *(const float4*)(p.router_scale + 8 * c);
            t.r1 = *(const float4*)(p.router_scale + 8 * c + 4);
        }
    }
    if (c < p.E) {
        if (p.pes) t.pes = p.pes[c];
        if (p.logit_bias) t.lb = p.logit_bias[c];
    }
}

// The token into LDS, the router input scale, and the column sums the block
// dots need: thread c holds columns 8c .. 8c+7 and contributes its partial
// sums; each lane set is then a sum of two (4-bit) or four (8-bit) of them.
// xraw (TAIL only): LDS for the input row as given, the layer tail's residual.
template <bool TAIL>
__device__ __forceinline__ void stage_token(const Plan& p, Shared& sh, const TokenLoads& tl, uint32_t tag,
                                            uint16_t* xraw) {
    const int t = tix();
    const int nch = p.H / 8;
    uint4 v = tl.x;
    if (p.x_w && tl.need && t < nch) {
        // the previous layer's output row, published with that layer's tag
        // (one below this layer's): wait for any word not yet current
        const uint64_t* xw = p.x_w + xcc_copy() * p.xw_stride + 4 * t;
        uint64_t w4[4] = {tl.xw[0], tl.xw[1], tl.xw[2], tl.xw[3]};
        await_words(xw, 1, w4, 0xFu, tag - 1, p.f_err);
        v = make_uint4((uint32_t)w4[0], (uint32_t)w4[1], (uint32_t)w4[2], (uint32_t)w4[3]);
    }
    if constexpr (TAIL)
        if (p.t_res_in && t < nch) *(uint4*)(xraw + 8 * t) = v;
    if (p.in_eps > 0.f) {
        // the input row first goes through a unit-weight RMSNorm, rounded to
        // bf16 (the norm between the layers of a stack)
        float s0 = 0.f;
        if (t < nch) {
            const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) s0 += bf16_lo(wv[i]) * bf16_lo(wv[i]) + bf16_hi(wv[i]) * bf16_hi(wv[i]);
        }
        s0 = wave_sum(s0);
        if ((t & 63) == 0) sh.red[t >> 6][1] = s0;
        __syncthreads();
        float tot = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) tot += sh.red[w][1];
        const float inv = 1.0f / sqrtf(tot / (float)p.H + p.in_eps);
        auto nrm = [&](uint32_t wd) {
            return (uint32_t)f32_to_bf16(bf16_lo(wd) * inv) | ((uint32_t)f32_to_bf16(bf16_hi(wd) * inv) << 16);
        };
        v = make_uint4(nrm(v.x), nrm(v.y), nrm(v.z), nrm(v.w));
    }
    if (t < p.E) {
        sh.pes[t] = tl.pes;
        sh.lbias[t] = tl.lb;
    }
    if (t < 8) sh.hzero[t] = 0;
    float ss = 0.f;
    if (t < nch) {
        *(uint4*)(sh.x + 8 * t) = v;
        const float a[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                            bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
        const float rs[8] = {tl.r0.x, tl.r0.y, tl.r0.z, tl.r0.w, tl.r1.x, tl.r1.y, tl.r1.z, tl.r1.w};
        float q0 = 0.f, q1 = 0.f;   // sums of columns 8t..8t+3 and 8t+4..8t+7 (times router_scale)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ss += a[2 * i] * a[2 * i] + a[2 * i + 1] * a[2 * i + 1];
            const float r = a[2 * i] * rs[2 * i] + a[2 * i + 1] * rs[2 * i + 1];
            if (i < 2) q0 += r; else q1 += r;
        }
        float4* xr = (float4*)(sh.xr + 8 * t);
        xr[0] = make_float4(a[0] * rs[0], a[1] * rs[1], a[2] * rs[2], a[3] * rs[3]);
        xr[1] = make_float4(a[4] * rs[4], a[5] * rs[5], a[6] * rs[6], a[7] * rs[7]);
        sh.c8[t] = sum8_bf16(v);
        sh.c4[2 * t] = q0;
        sh.c4[2 * t + 1] = q1;
    }
    ss = wave_sum(ss);
    if ((t & 63) == 0) sh.red[t >> 6][0] = ss;
    __syncthreads();
    if (t < p.G_H * 4) {
        float tot = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) tot += sh.red[w][0];
        const float rc = (1.0f / sqrtf(tot / (float)p.H + p.eps)) * (1.0f / sqrtf((float)p.H));
        if (t == 0) sh.rc = rc;
        const int g = t >> 2, kb = t & 3;
        // 4-bit lane set: chunks 8g + kb (columns 32*0 + 8kb) and 8g + 4 + kb
        sh.xsum[t] = sh.c8[8 * g + kb] + sh.c8[8 * g + 4 + kb];
        // 8-bit lane set: quarters (16 ks + 4 kb) for ks = 0..3, quarter index = 16g + 4ks + kb
        const float r = (sh.c4[16 * g + kb] + sh.c4[16 * g + 4 + kb]) + (sh.c4[16 * g + 8 + kb] + sh.c4[16 * g + 12 + kb]);
        sh.rsum[t] = r * rc;
    }
    __syncthreads();
}

// Expert ids and weights, computed by every workgroup that needs them from
// its XCD's copy of the partial scores: sum the pieces of each score in
// order, rank every expert (the number of scores that beat it: higher, or
// equal with a lower index), keep ranks < k in rank order, then the softmax
// over the selected scores times per_expert_scale.  One workgroup reports
// the scores, ids and weights to the caller's optional outputs.
__device__ __forceinline__ void fetch_ids(const Plan& p, Shared& sh, uint32_t tag) {
    const int nslice = (p.E + 15) / 16, epad = (p.E + 31) & ~31;
    gather_words(p.f_rpart + xcc_copy() * p.rpart_stride, nslice * kRq * 16, tag, p.f_err, sh.gbuf, 0);
    // workgroup 0 runs the first routed unit, so it always fetches the ids
    const bool reporter = blockIdx.x == 0;
    // Selection key of expert e: the score's bits made order-preserving as an
    // unsigned integer (NaN as -inf, -0 as +0) above 0xFFFF - e, so that keys
    // compare as (score, then lower index); padding keys are 0, below all.
    for (int e = tix(); e < epad; e += kThreads) {
        float s = -INFINITY;
        uint64_t key = 0;
        if (e < p.E) {
            const int slice = e >> 4, r = e & 15;
            float a[kRq];
#pragma unroll
            for (int q = 0; q < kRq; ++q) a[q] = __uint_as_float(sh.gbuf[(slice * kRq + q) * 16 + r]);
            s = ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
            s += sh.lbias[e];
            if (reporter && p.logits_out) p.logits_out[e] = s;
            if (!(s == s)) s = -INFINITY;   // a NaN score ranks last; ids stay distinct
            if (s == 0.f) s = 0.f;
            uint32_t u = __float_as_uint(s);
            u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
            key = ((uint64_t)u << 32) | (uint32_t)(0xFFFF - e);
        }
        sh.lg[e] = s;
        sh.key[e] = key;
    }
    if (tix() < kMaxTopK) sh.selv[tix()] = -INFINITY;
    __syncthreads();
    // Rank of expert e = the number of keys above its key.  Each expert's
    // comparisons are split over nparts adjacent lanes, summed by shuffles.
    // Part q reads the key pairs q, q + nparts, ...: the parts of a wave read
    // adjacent 16-byte pieces, on distinct LDS banks.
    {
        const int lg2 = epad <= 128 ? 3 : 2, nparts = 1 << lg2;   // nparts * epad <= kThreads
        const int e = tix() >> lg2, part = tix() & (nparts - 1), len = epad >> lg2;
        int rank = 0;
        if (e < p.E) {
            const uint64_t me = sh.key[e];
            const uint64_t* kp = sh.key + 2 * part;
#pragma unroll 8
            for (int o = 0; o < len; o += 2) {
                const ulonglong2 k0 = *(const ulonglong2*)(kp + o * nparts);
                rank += (int)(k0.x > me) + (int)(k0.y > me);
            }
        }
        rank = lg2 == 3 ? group_sum_i<true>(rank) : group_sum_i<false>(rank);
        if (e < p.E && part == 0 && rank < p.k) {
            sh.ids[rank] = e;
            sh.selv[rank] = sh.lg[e];
        }
    }
    __syncthreads();
    // softmax over the selected scores (padding entries are -inf, so 0), on
    // the last wave: it has one gate/up item fewer than wave 0 and publishes
    // nothing (stack 585 -> 576 us/token, the lone call unchanged)
    if (wave_id() == kWaves - 1) {
        const int j = tix() & (kMaxTopK - 1);
        const float ej = expf(sh.selv[j] - sh.selv[0]);
        static_assert(kMaxTopK == 16, "the softmax sums one 16-lane row");
        const float den = sum16(ej);
        if ((tix() & 63) < p.k) {
            const float w = ej / den * sh.pes[sh.ids[j]];
            sh.wts[j] = w;
            if (reporter) {
                if (p.ids_out) p.ids_out[j] = sh.ids[j];
                if (p.w_out) p.w_out[j] = w;
            }
        }
    }
    // No barrier: the other waves go on to issue their routed loads, which
    // need only the ids.  sh.wts is first read by the routed down units,
    // after the barriers of the gate/up unit or of the activation gather,
    // and what the softmax reads (selv, ids, pes) is not written before
    // those barriers either.
}

// One source's activations (64 tagged words per group, from group g0, fp16
// in the low half of the payload) into LDS as the matrix-core operand of
// the token: the columns with (c & 2) != 0 divided by 16 (see codes8),
// with each group's sums of the activations (hsx) and of the stored
// operand (hsa).  ng <= kWaves: wave w converts group w.
__device__ __forceinline__ void stage_h(const Plan& p, Shared& sh, const uint64_t* h, int g0, int ng, uint32_t tag) {
    gather_words(h + 64 * g0, ng * 64, tag, p.f_err, sh.gbuf, kGatherT0);
    const int q = tix(), lane = q & 63, g = wave_id();
    if (g < ng) {
        const _Float16 x = __builtin_bit_cast(_Float16, (uint16_t)sh.gbuf[q]);
        const _Float16 a = (lane & 2) ? x * (_Float16)0.0625f : x;
        sh.h16[q] = __builtin_bit_cast(uint16_t, a);
        const float sx = wave_sum((float)x), sa = wave_sum((float)a);
        if (lane == 0) {
            sh.hsx[g] = sx;
            sh.hsa[g] = sa;
        }
    }
    __syncthreads();
}

// ----------------------------------------------------------------- compute

// The token's staged activations as the A operand of
// v_mfma_f32_16x16x32_f16 (16 tokens x 32 columns): the lanes of token 0
// (lane % 16 == 0) read columns 32 kh + 8 (lane / 16) .. +7 of a group,
// the others read zeros.
struct TokOp {
    const uint16_t* base;
    int gstride, kh;
};
__device__ __forceinline__ TokOp tok_op(const Shared& sh) {
    const int lane = tix() & 63;
    const bool on = (lane & 15) == 0;
    return {on ? sh.h16 + 8 * (lane >> 4) : sh.hzero, on ? 64 : 0, on ? 32 : 0};
}

// The same operand over the staged token x (bf16), for the gate/up units.
__device__ __forceinline__ TokOp tok_op_x(const Shared& sh) {
    const int lane = tix() & 63;
    const bool on = (lane & 15) == 0;
    return {on ? sh.x + 8 * (lane >> 4) : sh.hzero, on ? 64 : 0, on ? 32 : 0};
}

// Rows 16 r + lane % 16 (r = 0, 1) of one 4-bit half block against group g
// of the staged bf16 token, on the matrix cores with the codes as bf16
// 128 + q (exact) in the B operand: lanes 0..15 of d[r] get
// sum_c (128 + q_c) x_c + neg over the group's 64 columns.
__device__ __forceinline__ void half_block_mma_bf16(const uint4& c, const TokOp& t, int g, float neg, float d[2]) {
    const bf16x8_t a0 = *(const bf16x8_t*)(t.base + g * t.gstride);
    const bf16x8_t a1 = *(const bf16x8_t*)(t.base + g * t.gstride + t.kh);
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        float4_t acc = {neg, 0.f, 0.f, 0.f};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, codes8_bf16(w[2 * r]), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, codes8_bf16(w[2 * r + 1]), acc, 0, 0, 0);
        d[r] = acc[0];
    }
}

// Rows 16 r + lane % 16 (r = 0, 1) of one 4-bit half block (the lane's
// 16-byte code c: word 2 r + kh holds rows 16 r.., columns 32 kh + 8 (lane /
// 16)..) against group g of the staged token, on the matrix cores with the
// codes as the B operand (D[token][row]): lanes 0..15 of d[r] get
// sum_c code_c a_c + neg over the group's 64 columns (neg = -1024 sum_c a_c
// makes it sum_c q_c x_c).
__device__ __forceinline__ void half_block_mma(const uint4& c, const TokOp& t, int g, float neg, float d[2]) {
    const half8_t a0 = *(const half8_t*)(t.base + g * t.gstride);
    const half8_t a1 = *(const half8_t*)(t.base + g * t.gstride + t.kh);
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        float4_t acc = {neg, 0.f, 0.f, 0.f};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, codes8(w[2 * r]), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, codes8(w[2 * r + 1]), acc, 0, 0, 0);
        d[r] = acc[0];
    }
}

// Row totals over the lanes and waves: v[r] holds rows 16*r + lane%16; after
// the call sh.red[w][row] holds wave w's part of each row.
__device__ __forceinline__ void reduce_rows(Shared& sh, const float* v, int nr) {
    const int wave = wave_id(), lane = tix() & 63;
    for (int r = 0; r < nr; ++r) {
        const float s = row_sum_kb(v[r]);
        if (lane < 16) sh.red[wave][16 * r + lane] = s;
    }
    __syncthreads();
}

// Row totals of a unit on the matrix cores: lanes 0..15 of v[r] already
// hold the wave's part of rows 16*r + lane; after the call sh.red[w][row]
// holds wave w's part of each row.
__device__ __forceinline__ void store_rows(Shared& sh, const float* v, int nr) {
    const int wave = wave_id(), lane = tix() & 63;
    for (int r = 0; r < nr; ++r)
        if (lane < 16) sh.red[wave][16 * r + lane] = v[r];
    __syncthreads();
}

// Sums in wave order.  The reads all go out before the first add (a loop
// whose reads each waited for the previous one took about 0.4 us, on the
// path of every publish step).
__device__ __forceinline__ float row_total(const Shared& sh, int row) {
    float t[kWaves];
#pragma unroll
    for (int w = 0; w < kWaves; ++w) t[w] = sh.red[w][row];
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) v += t[w];
    return v;
}

// Row (0..63) of a unit whose even waves hold rows 0..31 and odd waves
// rows 32..63 (gate/up: gate and up rows; down: the two halves of a tile).
__device__ __forceinline__ float row_total_par(const Shared& sh, int row) {
    const int par = row >> 5, r = row & 31;
    float t[kWaves / 2];
#pragma unroll
    for (int i = 0; i < kWaves / 2; ++i) t[i] = sh.red[2 * i + par][r];
    float v = 0.f;
#pragma unroll
    for (int i = 0; i < kWaves / 2; ++i) v += t[i];
    return v;
}

__device__ __forceinline__ void run_router(const Plan& p, Shared& sh, const Unit& x, const Loads& L, uint32_t tag) {
    const int wave = wave_id(), lane = tix() & 63, kb = lane >> 4;
    float acc = 0.f;
#pragma unroll
    for (int m = 0; m < kItems; ++m) {
        const int it = wave + kWaves * m;
        if (it < x.ng) {
            const int g = x.g0 + it;
            const uint32_t cw[4] = {L.c[m].x, L.c[m].y, L.c[m].z, L.c[m].w};
            float d = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float4 r = *(const float4*)(sh.xr + 64 * g + 16 * i + 4 * kb);
                d = fmaf((float)(cw[i] & 0xFFu), r.x, d);
                d = fmaf((float)((cw[i] >> 8) & 0xFFu), r.y, d);
                d = fmaf((float)((cw[i] >> 16) & 0xFFu), r.z, d);
                d = fmaf((float)(cw[i] >> 24), r.w, d);
            }
            const uint32_t sw = (x.a & 1) ? L.s[m].y : L.s[m].x;
            acc = fmaf(bf16_lo(sw), d * sh.rc, fmaf(bf16_hi(sw), sh.rsum[g * 4 + kb], acc));
        }
    }
    reduce_rows(sh, &acc, 1);
    if (wave_id() < 16 * kCopies / 64) {
        const int r = tix() & 15, c = tix() >> 4;
        st_word(p.f_rpart + c * p.rpart_stride + (int64_t)(x.a * kRq + x.q) * 16 + r, tag,
                __float_as_uint(row_total(sh, r)));
    }
    __syncthreads();
}

// Full-row gate/up unit (routed: one selected expert; shared: the shared
// expert): 32 rows of gate and up over every column group, so the workgroup
// holds complete sums and publishes h = gelu(g) * u for its 32 rows without
// any partial exchange.
__device__ __forceinline__ void run_rh(const Plan& p, Shared& sh, const Unit& x, const LoadsN<kItemsRH>& L,
                                       uint32_t tag) {
    const int wave = wave_id();
    const TokOp to = tok_op_x(sh);
    float acc[2] = {0.f, 0.f};    // lanes 0..15: rows 16*r + lane of the wave's matrix (gate: even waves, up: odd)
#pragma unroll
    for (int m = 0; m < kItemsRH; ++m) {
        const int it = wave + kWaves * m;
        if (it < 2 * x.ng) {
            const int g = it >> 1;
            const float4 x4 = *(const float4*)(sh.xsum + 4 * g);
            const float xs = (x4.x + x4.y) + (x4.z + x4.w);   // x over the group's 64 columns
            float d[2];
            half_block_mma_bf16(L.c[m], to, g, -128.f * xs, d);
            const uint32_t sw[2] = {L.s[m].x, L.s[m].y};
#pragma unroll
            for (int r = 0; r < 2; ++r) acc[r] += fmaf(bf16_lo(sw[r]), d[r], bf16_hi(sw[r]) * xs);
        }
    }
    store_rows(sh, acc, 2);
    if (wave_id() == 0 && tix() < 32) {
        const int r = tix();
        const float h = gelu_tanh(row_total_par(sh, r)) * row_total_par(sh, 32 + r);
        const _Float16 hh = (_Float16)h;
        flag_error(p.f_err, f16_bad(hh), kErrRange);
        const uint32_t h16 = __builtin_bit_cast(uint16_t, hh);
        uint64_t* hout = x.kind == U_SH ? p.f_hs + 32 * x.a + r : p.f_h + (int64_t)x.a * p.I + 32 * x.b + r;
#pragma unroll
        for (int c = 0; c < kCopies; ++c) st_word(hout + c * p.h_stride, tag, h16);
    }
    // no barrier: the next writer of sh.red (a later unit's row totals)
    // comes after the barriers of that unit's activation gather or of the
    // ids, and nothing else that wave 0 reads here is written before them
}

// Shared down piece: one 64-row output tile from one chunk of the shared
// activations -> partial outputs (source k + chunk).
__device__ __forceinline__ void stage_sd(const Plan& p, Shared& sh, const Unit& x, uint32_t tag) {
    stage_h(p, sh, p.f_hs + xcc_copy() * p.h_stride, x.g0, x.ng, tag);
}

// The piece from its activations staged in LDS.
__device__ __forceinline__ void sd_compute(const Plan& p, Shared& sh, const Unit& x, const Loads& L, uint32_t tag) {
    const int w0 = down_w0(p), nw = kWaves - w0;
    const int wave = wave_id() - w0;
    const TokOp to = tok_op(sh);
    float acc[2] = {0.f, 0.f};    // lanes 0..15: rows 32*(wave & 1) + 16*r + lane of the output tile
#pragma unroll
    for (int m = 0; m < kItems; ++m) {
        const int it = wave + nw * m;
        if (wave >= 0 && it < 2 * x.ng) {
            const int gl = it >> 1;
            const float hx = sh.hsx[gl];
            float d[2];
            half_block_mma(L.c[m], to, gl, -1024.f * sh.hsa[gl], d);
            const uint32_t sw[2] = {L.s[m].x, L.s[m].y};
#pragma unroll
            for (int r = 0; r < 2; ++r) acc[r] += fmaf(bf16_lo(sw[r]), d[r], bf16_hi(sw[r]) * hx);
        }
    }
    store_rows(sh, acc, 2);
    uint64_t* dst = p.f_piece + ((int64_t)x.a * p.n_src + p.k + x.b) * 64;
    if (wave_id() == 0) st_word(dst + tix(), tag, __float_as_uint(row_total_par(sh, tix())));
    // no barrier: as at the end of run_rh
}

__device__ __forceinline__ void run_sd_piece(const Plan& p, Shared& sh, const Unit& x, const Loads& L, uint32_t tag) {
    stage_sd(p, sh, x, tag);
    sd_compute(p, sh, x, L, tag);
}

// Loads of a routed down unit: for each of its tiles, wave w >= w0 takes
// groups v/2 + np j (v = w - w0, np = (kWaves - w0) / 2, j < kGroupsD) of
// the expert's intermediate, half w % 2 of the tile (w0 = down_w0).
__device__ __forceinline__ void issue_rdu(const Plan& p, const Shared& sh, const DownUnit& d, LoadsN<kItemsD>& L) {
    const int w0 = down_w0(p), np = (kWaves - w0) / 2;
    const int wave = wave_id() - w0, lane = tix() & 63, par = wave & 1;
    if (wave < 0) return;
    const uint8_t* base = p.pool_base + (int64_t)sh.ids[d.b] * p.expert_stride + p.down_off +
                          ((int64_t)d.t0 * p.G_I + (wave >> 1)) * kBlk4;
    const int lc = par * 1024 + lane * 16, ls = kCodes4 + 8 * par + (lane & 15) * 16;
#pragma unroll
    for (int t = 0; t < kTilesD; ++t)
#pragma unroll
        for (int j = 0; j < kGroupsD; ++j)
            if (t < d.nt && (wave >> 1) + np * j < p.G_I) {
                const uint8_t* blk = base + ((int64_t)t * p.G_I + np * j) * kBlk4;
                L.c[kGroupsD * t + j] = ld_stream16(blk + lc);
                L.s[kGroupsD * t + j] = *(const uint2*)(blk + ls);
            }
}

// Routed down unit: the weighted partial outputs of one selected expert for
// each of its tiles (source = slot).
__device__ __forceinline__ void run_rdu(const Plan& p, Shared& sh, const DownUnit& d, const LoadsN<kItemsD>& L,
                                        uint32_t tag) {
    stage_h(p, sh, p.f_h + xcc_copy() * p.h_stride + (int64_t)d.b * p.I, 0, p.G_I, tag);
    const int w0 = down_w0(p), np = (kWaves - w0) / 2;
    const int wave = wave_id(), lane = tix() & 63;
    const TokOp to = tok_op(sh);
    const float wf = sh.wts[d.b];
    float acc[kTilesD][2];   // lanes 0..15: rows 32*(wave & 1) + 16*r + lane of tile t
#pragma unroll
    for (int t = 0; t < kTilesD; ++t) acc[t][0] = acc[t][1] = 0.f;
#pragma unroll
    for (int j = 0; j < kGroupsD; ++j) {
        const int g = ((wave - w0) >> 1) + np * j;
        if (wave >= w0 && g < p.G_I) {
            const float hx = sh.hsx[g], neg = -1024.f * sh.hsa[g];
#pragma unroll
            for (int t = 0; t < kTilesD; ++t)
                if (t < d.nt) {
                    const int m = kGroupsD * t + j;
                    float dd[2];
                    half_block_mma(L.c[m], to, g, neg, dd);
                    const uint32_t sw[2] = {L.s[m].x, L.s[m].y};
#pragma unroll
                    for (int r = 0; r < 2; ++r) acc[t][r] += wf * fmaf(bf16_lo(sw[r]), dd[r], bf16_hi(sw[r]) * hx);
                }
        }
    }
#pragma unroll
    for (int t = 0; t < kTilesD; ++t)
        if (t < d.nt)
#pragma unroll
            for (int r = 0; r < 2; ++r)
                if (lane < 16) sh.red2[wave][t][16 * r + lane] = acc[t][r];
    __syncthreads();
    if (wave_id() == 0) {
        const int row = tix(), par = row >> 5;
#pragma unroll
        for (int t = 0; t < kTilesD; ++t)
            if (t < d.nt) {
                float u[kWaves / 2];
#pragma unroll
                for (int i = 0; i < kWaves / 2; ++i) u[i] = sh.red2[2 * i + par][t][row & 31];
                float v = 0.f;
#pragma unroll
                for (int i = 0; i < kWaves / 2; ++i) v += u[i];
                st_word(p.f_piece + ((int64_t)(d.t0 + t) * p.n_src + d.b) * 64 + row, tag, __float_as_uint(v));
            }
    }
    // no barrier: sh.red2 is written again only by the next layer's routed
    // down unit, after the barrier that ends this layer
}

// Writes output row `row` (v: its fp32 value) to out and, in a stack, to
// the next layer's input words.
__device__ __forceinline__ void put_row(const Plan& p, int row, float v, uint32_t tag) {
    // a wait of this call that gave up may have fed stale partial results
    // into the sums: the output then reads NaN rather than a plausible row
    if (ld_ctr(p.f_err) & kErrWait) v = __builtin_nanf("");
    const uint32_t b = f32_to_bf16(v);
    if (!p.out) {
    } else if (p.out_f32) {
        ((float*)p.out)[row] = v;
    } else {
        ((uint16_t*)p.out)[row] = (uint16_t)b;
    }
    if (p.out_w) {
        // the next layer's input: bf16 pairs (row 2i in the low half), one copy per XCD
        const uint32_t b1 = next_lane_in_row(b);   // read by even lanes only
        if ((tix() & 1) == 0) {
#pragma unroll
            for (int c = 0; c < kCopies; ++c) st_word(p.out_w + c * p.xw_stride + (row >> 1), tag, b | (b1 << 16));
        }
    }
}

// Output tile a: every source's partial outputs summed in source order
// (routed slots, then shared chunks), rounded once.  With the layer tail the
// two branches are summed apart, s (shared) and r (routed); every output
// tile publishes five partial sums over its 64 rows,
//     s^2, r^2, (w_s s)^2, (w_r r)^2, (w_s s)(w_r r),
// and each one sums all tiles' in tile order: that gives the two branch
// norms' factors a, b and, since |a w_s s + b w_r r|^2 expands into those
// sums, the output norm's factor c without a second exchange.
// The output sums of tile a with the layer tail (see run_reduce).
// Sum of the gathered sources s0 .. s1-1 (< 32) of row r, in source order,
// eight reads at a time.
__device__ __forceinline__ float sum_sources(const Shared& sh, int s0, int s1, int r) {
    float v = 0.f;
    for (int b = s0; b < s1; b += 8) {
        float t[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) t[i] = __uint_as_float(sh.gbuf[min(b + i, 31) * 64 + r]);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (b + i < s1) v += t[i];
    }
    return v;
}

__device__ __forceinline__ void run_reduce_tail(const Plan& p, Shared& sh, int a, uint32_t tag, const uint16_t* xraw) {
    const int row = 64 * a + tix();
    float sv = 0.f, rv = 0.f, ws = 1.f, wr = 1.f;
    if (wave_id() == 0) {
        if (p.tn_s) ws = p.tn_s[row];
        if (p.tn_r) wr = p.tn_r[row];
        rv = sum_sources(sh, 0, p.k, tix());
        sv = sum_sources(sh, p.k, p.n_src, tix());
        const float q[5] = {wave_sum(sv * sv), wave_sum(rv * rv), wave_sum((ws * sv) * (ws * sv)),
                            wave_sum((wr * rv) * (wr * rv)), wave_sum((ws * sv) * (wr * rv))};
        if (tix() < 8) {
            float mine = 0.f;
#pragma unroll
            for (int i = 0; i < 5; ++i)
                if ((int)tix() == i) mine = q[i];
            st_word(p.f_tail + (int64_t)a * 8 + tix(), tag, __float_as_uint(mine));
        }
    }
    gather_words(p.f_tail, p.G_H * 8, tag, p.f_err, sh.gbuf, kGatherT0);
    if (wave_id() == 0) {
        float tot[5] = {0.f, 0.f, 0.f, 0.f, 0.f};
        for (int t2 = 0; t2 < p.G_H; ++t2)
#pragma unroll
            for (int i = 0; i < 5; ++i) tot[i] += __uint_as_float(sh.gbuf[t2 * 8 + i]);
        const float H = (float)p.H;
        const float fa = p.tn_s ? 1.0f / sqrtf(tot[0] / H + p.t_eps) : 1.0f;
        const float fb = p.tn_r ? 1.0f / sqrtf(tot[1] / H + p.t_eps) : 1.0f;
        const float ff = fa * fa * tot[2] + fb * fb * tot[3] + 2.0f * fa * fb * tot[4];
        const float fc = p.tn_o ? 1.0f / sqrtf(ff / H + p.t_eps) : 1.0f;
        const float wo = p.tn_o ? p.tn_o[row] : 1.0f;
        float res = 0.f;
        if (p.t_res_in)
            res = bf16_to_f32(xraw[row]);
        else if (p.t_res)
            res = bf16_to_f32(p.t_res[row]);
        put_row(p, row, p.t_scalar * (res + fc * wo * (fa * ws * sv + fb * wr * rv)), tag);
    }
    // the layer's closing barrier follows
}

template <bool TAIL>
__device__ __forceinline__ void run_reduce(const Plan& p, Shared& sh, int a, uint32_t tag, const uint16_t* xraw) {
    const uint64_t* tilep = p.f_piece + (int64_t)a * p.n_src * 64;
    gather_words(tilep, p.n_src * 64, tag, p.f_err, sh.gbuf, kGatherT0);
    if constexpr (!TAIL) {
        if (wave_id() == kSumWave) {
            const int r = (int)tix() - 64 * kSumWave;
            put_row(p, 64 * a + r, sum_sources(sh, 0, p.n_src, r), tag);
        }
        // the layer's closing barrier follows
    } else {
        run_reduce_tail(p, sh, a, tag, xraw);
    }
}

// ----------------------------------------------------------------- the kernel

// Phases of a workgroup (every branch below is taken by all of its waves):
//   1. the token's loads, then the weight loads of its router piece and
//      shared gate/up pieces;
//   2. those units;
//   3. the expert ids (waits for the router pieces), then the weight loads of
//      its remaining units at once: a full-row routed gate/up unit (routed
//      workgroups) or shared down pieces (shared workgroups), and a routed
//      down unit;
//   4. those units, then (workgroup a < G_H) the sum of output tile a.
// Every wait is for a unit earlier in the order router < shared gate/up <
// ids < routed gate/up < shared down < routed down < output sums, and each
// workgroup runs its units in that order, so with all workgroups resident
// every wait ends.

// Touch every field of the argument block the kernel reads, in one batch.
// Left alone, the compiler fetches the block field by field near each first
// use: a chain of dependent scalar-cache misses before the first weight load.
// Once the lines are cached, later reads of the fields hit.
__device__ __forceinline__ void prefetch_args(const Plan& p) {
    asm volatile("" ::"s"(p.x), "s"(p.router_w), "s"(p.router_scale), "s"(p.pes), "s"(p.logit_bias),
                 "s"(p.f_epoch), "s"(p.pool_base), "s"(p.sh_gate), "s"(p.sh_up), "s"(p.sh_down));
    asm volatile("" ::"s"(p.f_rpart), "s"(p.f_hs), "s"(p.f_h), "s"(p.f_piece),
                 "s"(p.f_err), "s"(p.out), "s"(p.ids_out), "s"(p.w_out), "s"(p.logits_out));
    asm volatile("" ::"s"(p.E), "s"(p.k), "s"(p.H), "s"(p.I), "s"(p.G_H), "s"(p.G_I), "s"(p.G_s), "s"(p.n_src),
                 "s"(p.n_router), "s"(p.n_rh), "s"(p.n_sd), "s"(p.n_sc), "s"(p.n_rng), "s"(p.eps));
    asm volatile("" ::"s"(p.x_w), "s"(p.out_w), "s"(p.xw_stride), "s"(p.in_eps));
    asm volatile("" ::"s"(p.h_stride), "s"(p.rpart_stride), "s"(p.expert_stride), "s"(p.gate_off), "s"(p.up_off),
                 "s"(p.down_off), "s"(p.out_f32), "s"(p.nwg));
}

// One layer for one token: the workgroup's part of the unit order above.
// Ends with every wave past its last use of the shared memory.
template <bool TAIL>
__device__ __forceinline__ void decode_layer(const Plan& p, Shared& sh, uint32_t tag, uint16_t* xraw) {
    const int nwg = p.nwg, w = blockIdx.x;
    // kTokenFirst: the token's loads go out before the unit assignments,
    // whose integer divisions otherwise delay them
    const bool need = w < p.n_rh || (w - p.G_H >= 0 && w - p.G_H < p.n_router) || (w - p.n_rh >= 0 && w - p.n_rh < 2 * p.G_s);
    TokenLoads tl;
    if constexpr (kTokenFirst) load_token(p, tl, need);
    const Unit ur = unit_router(p, w - p.G_H);
    const Unit us = unit_sh(p, w - p.n_rh);
    const Unit rh = unit_rh(p, w);
    const DownUnit du = unit_rdu(p, w, nwg);
    if constexpr (!kTokenFirst) load_token(p, tl, need);
    Loads lrt;
    LoadsN<kItemsRH> lsh;
    issue_loads(p, sh, ur, lrt);
    // In a stack the shared gate/up loads (6.7 MB in all) wait for the token:
    // issued at the layer's start they would compete with the previous
    // layer's routed down units and output sums, which are still running.
    if constexpr (!kLateSharedGateUp) issue_loads(p, sh, us, lsh);
    // A routed workgroup's shared down piece needs no ids: its weights load
    // while the router runs, when the memory is far from busy.  In a stack
    // they go out before the token (the previous layer's output sums are
    // still running, so the wait for the token hides them); in a lone call
    // the token comes first, since the staging barrier may then wait for them.
    const Unit usd0 = rh.kind == U_RH ? sd_piece(p, w, nwg, 0) : no_unit();
    Loads lsd0;
    if constexpr (kEarlySharedDown) issue_loads(p, sh, usd0, lsd0);
    stage_token<TAIL>(p, sh, tl, tag, xraw);
    if constexpr (!kEarlySharedDown) issue_loads(p, sh, usd0, lsd0);
    if constexpr (kLateSharedGateUp) issue_loads(p, sh, us, lsh);
    if (ur.kind == U_ROUTER) run_router(p, sh, ur, lrt, tag);
    // Units end without a barrier after wave 0 reads their row totals in
    // sh.red (see run_rh); the next writer of sh.red must follow a barrier.
    // Every later unit starts with a gather or the ids, which have one, and
    // the layer ends with one; only a router piece followed by a shared
    // gate/up unit on one workgroup would not (not so in the present layout,
    // where router and shared workgroups are disjoint), so take one then.
    if (ur.kind == U_ROUTER && us.kind == U_SH) __syncthreads();
    if (us.kind == U_SH) run_rh(p, sh, us, lsh, tag);
    if (rh.kind == U_RH || du.nt > 0) fetch_ids(p, sh, tag);
    LoadsN<kItemsD> ld;
    if (rh.kind == U_RH && kLateRoutedDown) {
        // The down unit's loads go out once the gate/up weights have landed
        // (they would share the memory's rate with them) and after the shared
        // piece's activation gather (loads complete in issue order, so the
        // gather would wait for them).  In a lone call the piece's compute
        // then waits for those loads (the compiler waits for every load in
        // flight before it), which costs more than it saves.
        LoadsN<kItemsRH> lr;
        issue_loads(p, sh, rh, lr);
        run_rh(p, sh, rh, lr, tag);
        if (usd0.kind == U_SD) stage_sd(p, sh, usd0, tag);
        if (du.nt > 0) issue_rdu(p, sh, du, ld);
        if (usd0.kind == U_SD) sd_compute(p, sh, usd0, lsd0, tag);
    } else if (rh.kind == U_RH) {
        LoadsN<kItemsRH> lr;
        issue_loads(p, sh, rh, lr);
        if (du.nt > 0) issue_rdu(p, sh, du, ld);
        run_rh(p, sh, rh, lr, tag);
        if (usd0.kind == U_SD) run_sd_piece(p, sh, usd0, lsd0, tag);
    } else {
        Unit usd[kSlotsSD];
        Loads lsd[kSlotsSD];
#pragma unroll
        for (int s = 0; s < kSlotsSD; ++s) {
            usd[s] = sd_piece(p, w, nwg, s);
            issue_loads(p, sh, usd[s], lsd[s]);
        }
        if (du.nt > 0) issue_rdu(p, sh, du, ld);
#pragma unroll
        for (int s = 0; s < kSlotsSD; ++s)
            if (usd[s].kind == U_SD) run_sd_piece(p, sh, usd[s], lsd[s], tag);
    }
    if (du.nt > 0) run_rdu(p, sh, du, ld, tag);
    if (w < p.G_H) run_reduce<TAIL>(p, sh, w, tag, xraw);
    __syncthreads();
}

// Tags: every workgroup keeps its own epoch word, the last tag it used.  A
// call reads it at the start (tag = epoch + 1) and stores its last tag at
// the end.  Every workgroup runs every call and calls on one workspace
// follow each other in stream order, so all workgroups of a call read the
// same epoch without any exchange, and no workgroup has to learn that the
// others are done (a counter over all workgroups cost a round trip to one
// contended address at the end of every call).
__device__ __forceinline__ uint32_t first_tag(const Plan& p) { return ld_ctr(p.f_epoch + blockIdx.x) + 1; }

__device__ __forceinline__ void finish_call(const Plan& p, uint32_t last_tag) {
    if (tix() == 0) __hip_atomic_store(p.f_epoch + blockIdx.x, last_tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace
}  // namespace mq
