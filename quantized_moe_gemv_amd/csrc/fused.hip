// Single-launch decode of one token through the whole layer.
//
// The layer is cut into ~25 KB units of weight streaming, listed in
// dependency order and dealt round-robin to one workgroup per compute unit
// (unit u runs on workgroup u % grid; each workgroup runs its units in
// increasing order):
//   router pieces   16 experts x a column range      -> partial scores
//   shared gate/up  32 rows x a column range          -> partial g, u
//   shared down     64 output rows x a chunk of Is    -> partial outputs
//   routed gate/up  (slot j, 32 rows, column range)   -> partial g, u
//   routed down     (64 output rows, slot j)          -> partial outputs
// Every dependency points to an earlier unit, so with all workgroups
// resident every wait ends; each wait is also bounded.  Partial results are
// 64-bit words carrying the call's epoch in their high half.  An arrival
// counter per target tells its last contributor to reduce (in a fixed
// order, so results repeat bit for bit), and one thread per consumer
// workgroup polls a single done-counter before the data is read, which
// keeps polling light.  Each workgroup issues the loads of its next unit
// before it computes the current one.
//
// Results that many workgroups read (expert ids, GeGLU activations) are
// written once per XCD (eight copies) and each reader takes the copy of its
// own XCD, so the readers do not all queue on the same memory channels.
//
// The shared expert and the router do not depend on each other, so the
// shared branch streams while the routing decision is made ("Decode",
// phase table: the shared expert overlaps the wait for the expert ids).
#include <math.h>

#include "device.h"
#include "plan.h"

namespace mq {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kItems = 3;           // 16-byte code loads per lane per unit
constexpr int kSpinLimit = 1 << 20;
constexpr int kCopies = 8;         // replicas of broadcast results, one per XCD

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

// Payload of a word once its tag is current.  Bounded, and gives up at once
// once any wait of the call has failed (recorded in *err).
__device__ __forceinline__ uint32_t wait_word(const uint64_t* p, uint32_t tag, uint32_t* err) {
    uint64_t v = ld_word(p);
    int spins = 0;
    while ((uint32_t)(v >> 32) != tag) {
        if (++spins > kSpinLimit || ((spins & 63) == 0 && ld_ctr(err))) {
            atomicOr(err, 1u);
            break;
        }
        __builtin_amdgcn_s_sleep(2);
        v = ld_word(p);
    }
    return (uint32_t)v;
}

// One thread waits until *ctr >= target; then the workgroup proceeds together.
__device__ __forceinline__ void wait_ctr(const uint32_t* ctr, uint32_t target, uint32_t* err) {
    if (threadIdx.x == 0) {
        int spins = 0;
        while (ld_ctr(ctr) < target) {
            if (++spins > kSpinLimit || ((spins & 63) == 0 && ld_ctr(err))) {
                atomicOr(err, 1u);
                break;
            }
            __builtin_amdgcn_s_sleep(4);
        }
    }
    __syncthreads();
}

// Payloads of words base[0 .. n) into dst, for n <= 4 * kThreads: every
// load is issued before any is checked, so the gather costs one round trip.
__device__ __forceinline__ void gather_words(const uint64_t* base, int n, uint32_t tag, uint32_t* err,
                                             uint32_t* dst) {
    uint64_t v[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int i = threadIdx.x + kThreads * m;
        v[m] = i < n ? ld_word(base + i) : 0;
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int i = threadIdx.x + kThreads * m;
        if (i < n) {
            if ((uint32_t)(v[m] >> 32) != tag) v[m] = ((uint64_t)tag << 32) | wait_word(base + i, tag, err);
            dst[i] = (uint32_t)v[m];
        }
    }
    __syncthreads();
}

__device__ __forceinline__ void bump(uint32_t* ctr) {
    __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ----------------------------------------------------------------- units

enum { U_ROUTER = 0, U_SG = 1, U_SD = 2, U_RG = 3, U_RD = 4, U_NONE = 5 };

struct Unit {
    int kind;
    int a, b;         // router: slice; SG: half tile; SD: out tile, chunk; RG: slot, half tile; RD: out tile, slot
    int q;            // piece index of the column range (router, gate/up)
    int g0, ng;       // column-group range
};

struct Shared {
    uint16_t x[4096];
    float xsum[64 * 4];       // x summed over each lane's 16 columns of a group (4-bit blocks)
    float rsum[64 * 4];       // router input summed over each lane's 16 columns (8-bit blocks)
    float rc;                 // router input scale 1/sqrt(mean(x^2)+eps)/sqrt(H)
    float red[kWaves][64];
    uint16_t hhi[16 * 64];    // one source's activations, bf16 high and low parts
    uint16_t hlo[16 * 64];
    float hsum[16 * 4];
    uint32_t gbuf[2048];      // gathered payloads (partial results of other units)
    float lg[256];            // expert scores
    int32_t ids[kMaxTopK];
    float wts[kMaxTopK];
    uint32_t flag;
};

// Column range q of nq over G groups.
__device__ __forceinline__ void krange(int G, int nq, int q, int* g0, int* ng) {
    const int a = q * G / nq, b = (q + 1) * G / nq;
    *g0 = a;
    *ng = b - a;
}

__device__ __forceinline__ Unit decode_unit(const Plan& p, int u) {
    Unit x;
    x.a = x.b = x.q = x.g0 = x.ng = 0;
    if (u < p.n_router) {
        x.kind = U_ROUTER;
        x.a = u / p.rq;
        x.q = u % p.rq;
        krange(p.G_H, p.rq, x.q, &x.g0, &x.ng);
        return x;
    }
    u -= p.n_router;
    if (u < p.n_sg) {
        x.kind = U_SG;
        x.a = u / p.gq;
        x.q = u % p.gq;
        krange(p.G_H, p.gq, x.q, &x.g0, &x.ng);
        return x;
    }
    u -= p.n_sg;
    if (u < p.n_sd) {
        x.kind = U_SD;
        x.a = u / p.n_sc;
        x.b = u % p.n_sc;
        x.g0 = x.b * p.G_I;
        x.ng = min(p.G_I, p.G_s - x.g0);
        return x;
    }
    u -= p.n_sd;
    if (u < p.n_rg) {
        x.kind = U_RG;
        const int per = 2 * p.G_I * p.gq;
        x.a = u / per;
        x.b = (u % per) / p.gq;
        x.q = u % p.gq;
        krange(p.G_H, p.gq, x.q, &x.g0, &x.ng);
        return x;
    }
    u -= p.n_rg;
    if (u < p.n_rd) {
        x.kind = U_RD;
        x.a = u / p.k;
        x.b = u % p.k;
        x.ng = p.G_I;
        return x;
    }
    x.kind = U_NONE;
    return x;
}

__device__ __forceinline__ bool needs_ids(const Unit& x) { return x.kind == U_RG || x.kind == U_RD; }

// A unit's weight loads, issued before the unit waits or computes.
struct Loads {
    uint4 c[kItems];
    uint2 s[kItems];
};

__device__ __forceinline__ const uint8_t* tile4(const uint8_t* m, int tile, int G) {
    return m + (int64_t)tile * G * kBlk4;
}

__device__ __forceinline__ void issue_loads(const Plan& p, const Shared& sh, const Unit& x, Loads& L) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
    for (int m = 0; m < kItems; ++m) {
        const int it = wave + kWaves * m;
        L.c[m] = make_uint4(0, 0, 0, 0);
        L.s[m] = make_uint2(0, 0);
        if (x.kind == U_ROUTER) {
            if (it < x.ng) {
                const int tile = x.a >> 2, j = x.a & 3;
                const uint8_t* blk = p.router_w + ((int64_t)tile * p.G_H + x.g0 + it) * kBlk8;
                L.c[m] = ld_stream16(blk + (j * 64 + lane) * 16);
                L.s[m].x = *(const uint32_t*)(blk + kCodes8 + (lane & 15) * 16 + 4 * j);
            }
        } else if (x.kind == U_SG || x.kind == U_RG) {
            // items: (group, matrix), gate for even items and up for odd ones
            if (it < 2 * x.ng) {
                const int g = x.g0 + (it >> 1);
                const uint8_t* m0;
                int ht;
                if (x.kind == U_SG) {
                    ht = x.a;
                    m0 = (it & 1) ? p.sh_up : p.sh_gate;
                } else {
                    ht = x.b;
                    const uint8_t* blob = p.pool_base + (int64_t)sh.ids[x.a] * p.expert_stride;
                    m0 = blob + ((it & 1) ? p.up_off : p.gate_off);
                }
                const int jh = ht & 1;
                const uint8_t* blk = tile4(m0, ht >> 1, p.G_H) + (int64_t)g * kBlk4;
                L.c[m] = ld_stream16(blk + jh * 1024 + lane * 16);
                L.s[m] = *(const uint2*)(blk + kCodes4 + (lane & 15) * 16 + 8 * jh);
            }
        } else if (x.kind == U_SD || x.kind == U_RD) {
            // items: (group, half of the 64-row output tile)
            if (it < 2 * x.ng) {
                const int gl = it >> 1, half = it & 1;
                const uint8_t* blk;
                if (x.kind == U_SD)
                    blk = tile4(p.sh_down, x.a, p.G_s) + (int64_t)(x.g0 + gl) * kBlk4;
                else
                    blk = tile4(p.pool_base + (int64_t)sh.ids[x.b] * p.expert_stride + p.down_off, x.a, p.G_I) +
                          (int64_t)gl * kBlk4;
                L.c[m] = ld_stream16(blk + half * 1024 + lane * 16);
                L.s[m] = *(const uint2*)(blk + kCodes4 + (lane & 15) * 16 + 8 * half);
            }
        }
    }
}

// ----------------------------------------------------------------- setup

__device__ __forceinline__ void stage_token(const Plan& p, Shared& sh) {
    const int t = threadIdx.x;
    if (t < p.H / 8) *(uint4*)(sh.x + 8 * t) = *(const uint4*)(p.x + 8 * t);
    __syncthreads();
    float ss = 0.f;
    for (int i = t; i < p.H; i += kThreads) {
        const float v = bf16_to_f32(sh.x[i]);
        ss += v * v;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);
    if ((t & 63) == 0) sh.red[t >> 6][0] = ss;
    __syncthreads();
    if (t == 0) {
        float s = 0.f;
        for (int w = 0; w < kWaves; ++w) s += sh.red[w][0];
        sh.rc = (1.0f / sqrtf(s / (float)p.H + p.eps)) * (1.0f / sqrtf((float)p.H));
    }
    __syncthreads();
    const float rc = sh.rc;
    for (int q = t; q < p.G_H * 4; q += kThreads) {
        const int g = q >> 2, kb = q & 3;
        float s4 = 0.f, s8 = 0.f;
        for (int ks = 0; ks < 2; ++ks)
            for (int e = 0; e < 8; ++e) s4 += bf16_to_f32(sh.x[64 * g + 32 * ks + 8 * kb + e]);
        for (int ks = 0; ks < 4; ++ks)
            for (int e = 0; e < 4; ++e) {
                const int i = 64 * g + 16 * ks + 4 * kb + e;
                s8 += bf16_to_f32(sh.x[i]) * rc * (p.router_scale ? p.router_scale[i] : 1.0f);
            }
        sh.xsum[q] = s4;
        sh.rsum[q] = s8;
    }
    __syncthreads();
}

// The last router piece: sum the partial scores of every piece in order,
// select the top k (higher score first, ties to the lower expert index),
// softmax over the selected scores times per_expert_scale, and publish
// ids and weights (every copy) and the caller's optional outputs.
__device__ __forceinline__ void reduce_topk(const Plan& p, Shared& sh, uint32_t tag) {
    wait_ctr(p.c_router, (uint32_t)p.n_router, p.f_err);
    const int nslice = (p.E + 15) / 16;
    gather_words(p.f_rpart, nslice * p.rq * 16, tag, p.f_err, sh.gbuf);
    for (int e = threadIdx.x; e < p.E; e += kThreads) {
        const int slice = e >> 4, r = e & 15;
        float s = 0.f;
        for (int q = 0; q < p.rq; ++q) s += __uint_as_float(sh.gbuf[(slice * p.rq + q) * 16 + r]);
        if (p.logit_bias) s += p.logit_bias[e];
        if (p.logits_out) p.logits_out[e] = s;
        sh.lg[e] = s;
    }
    __syncthreads();
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        float v[4];
        bool live[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int e = lane + 64 * m;
            live[m] = e < p.E;
            float s = live[m] ? sh.lg[e] : -INFINITY;
            if (!(s == s)) s = -INFINITY;
            v[m] = s;
        }
        float selv[kMaxTopK];
        int seli[kMaxTopK];
#pragma unroll
        for (int j = 0; j < kMaxTopK; ++j) {
            if (j < p.k) {
                float bv = -INFINITY;
                int bi = 0x7FFFFFFF;
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int e = lane + 64 * m;
                    if (live[m] && (v[m] > bv || (v[m] == bv && e < bi))) { bv = v[m]; bi = e; }
                }
#pragma unroll
                for (int o = 32; o >= 1; o >>= 1) {
                    const float ov = __shfl_xor(bv, o, 64);
                    const int oi = __shfl_xor(bi, o, 64);
                    if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
                }
                selv[j] = bv;
                seli[j] = bi;
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    if (lane + 64 * m == bi) live[m] = false;
            }
        }
        if (lane == 0) {
            float den = 0.f;
#pragma unroll
            for (int j = 0; j < kMaxTopK; ++j)
                if (j < p.k) den += expf(selv[j] - selv[0]);
#pragma unroll
            for (int j = 0; j < kMaxTopK; ++j)
                if (j < p.k) {
                    const float w = expf(selv[j] - selv[0]) / den * (p.pes ? p.pes[seli[j]] : 1.0f);
                    sh.ids[j] = seli[j];
                    sh.wts[j] = w;
                    if (p.ids_out) p.ids_out[j] = seli[j];
                    if (p.w_out) p.w_out[j] = w;
                }
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < kCopies * 2 * p.k; i += kThreads) {
        const int c = i / (2 * p.k), j = (i % (2 * p.k)) >> 1;
        const uint32_t payload = (i & 1) ? __float_as_uint(sh.wts[j]) : (uint32_t)sh.ids[j];
        st_word(p.f_ids + c * p.ids_stride + (i % (2 * p.k)), tag, payload);
    }
    __syncthreads();
}

// Expert ids and weights from this XCD's copy.
__device__ __forceinline__ void fetch_ids(const Plan& p, Shared& sh, uint32_t tag) {
    const uint64_t* src = p.f_ids + (blockIdx.x % kCopies) * p.ids_stride;
    if (threadIdx.x < 2 * p.k) {
        const uint32_t v = wait_word(src + threadIdx.x, tag, p.f_err);
        if (threadIdx.x & 1)
            sh.wts[threadIdx.x >> 1] = __uint_as_float(v);
        else
            sh.ids[threadIdx.x >> 1] = (int32_t)v;
    }
    __syncthreads();
}

// One source's activations (64 tagged words per group, from group g0) into
// LDS as bf16 high/low parts, with each lane's column sums.
__device__ __forceinline__ void stage_h(const Plan& p, Shared& sh, const uint64_t* h, int g0, int ng, uint32_t tag) {
    gather_words(h + 64 * g0, ng * 64, tag, p.f_err, sh.gbuf);
    for (int q = threadIdx.x; q < ng * 64; q += kThreads) {
        sh.hhi[q] = (uint16_t)(sh.gbuf[q] >> 16);
        sh.hlo[q] = (uint16_t)(sh.gbuf[q] & 0xFFFFu);
    }
    __syncthreads();
    for (int q = threadIdx.x; q < ng * 4; q += kThreads) {
        const int gl = q >> 2, qb = q & 3;
        float s = 0.f;
        for (int ks = 0; ks < 2; ++ks)
            for (int e = 0; e < 8; ++e) {
                const int i = 64 * gl + 32 * ks + 8 * qb + e;
                s += bf16_to_f32(sh.hhi[i]) + bf16_to_f32(sh.hlo[i]);
            }
        sh.hsum[q] = s;
    }
    __syncthreads();
}

// ----------------------------------------------------------------- compute

// Rows 16*r + lane%16 (r = 0, 1) of one 4-bit half block against the lane's
// 16 input values (bf16 pairs xa for columns 8*(lane/16).., xb for +32):
// adds sum((128 + q) * x) to d[r].
__device__ __forceinline__ void half_block_dot(const uint4& c, const uint4& xa, const uint4& xb, float d[2]) {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
    const uint32_t xk[2][4] = {{xa.x, xa.y, xa.z, xa.w}, {xb.x, xb.y, xb.z, xb.w}};
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) d[i >> 1] = dot2_bf16(q4_pair(w[i], q), xk[i & 1][q], d[i >> 1]);
}

// Row totals over the lanes and waves: v[r] holds rows 16*r + lane%16; after
// the call sh.red[w][row] holds wave w's part of each row.
__device__ __forceinline__ void reduce_rows(Shared& sh, const float* v, int nr) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    for (int r = 0; r < nr; ++r) {
        const float s = sum_kb(v[r]);
        if (lane < 16) sh.red[wave][16 * r + lane] = s;
    }
    __syncthreads();
}

__device__ __forceinline__ float row_total(const Shared& sh, int row) {
    float v = 0.f;
    for (int w = 0; w < kWaves; ++w) v += sh.red[w][row];
    return v;
}

__device__ __forceinline__ void run_router(const Plan& p, Shared& sh, const Unit& x, const Loads& L, uint32_t tag) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, kb = lane >> 4;
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
                const int col = 64 * g + 16 * i + 4 * kb;
                const uint2 xv = *(const uint2*)(sh.x + col);
                float r[4] = {bf16_lo(xv.x), bf16_hi(xv.x), bf16_lo(xv.y), bf16_hi(xv.y)};
                if (p.router_scale)
#pragma unroll
                    for (int e = 0; e < 4; ++e) r[e] *= p.router_scale[col + e];
#pragma unroll
                for (int e = 0; e < 4; ++e) d = fmaf((float)((cw[i] >> (8 * e)) & 0xFFu), r[e], d);
            }
            acc = fmaf(bf16_lo(L.s[m].x), d * sh.rc, fmaf(bf16_hi(L.s[m].x), sh.rsum[g * 4 + kb], acc));
        }
    }
    reduce_rows(sh, &acc, 1);
    if (threadIdx.x < 16)
        st_word(p.f_rpart + ((int64_t)(x.a * p.rq + x.q) * 16 + threadIdx.x), tag,
                __float_as_uint(row_total(sh, threadIdx.x)));
    __syncthreads();
    if (threadIdx.x == 0) bump(p.c_router);
    if (x.a * p.rq + x.q == p.n_router - 1) reduce_topk(p, sh, tag);
}

// Gate/up piece: 32 rows x a column range -> partial (g, u).  The last of
// the gq pieces of a half tile reduces them and publishes h = gelu(g) * u.
__device__ __forceinline__ void run_gateup(const Plan& p, Shared& sh, const Unit& x, const Loads& L, uint32_t tag) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, kb = lane >> 4;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};    // rows 16*r + lane%16: r = 0, 1 gate, 2, 3 up
#pragma unroll
    for (int m = 0; m < kItems; ++m) {
        const int it = wave + kWaves * m;
        if (it < 2 * x.ng) {
            const int g = x.g0 + (it >> 1), mat = it & 1;
            const uint4 xa = *(const uint4*)(sh.x + 64 * g + 8 * kb);
            const uint4 xb = *(const uint4*)(sh.x + 64 * g + 32 + 8 * kb);
            const float xs = sh.xsum[g * 4 + kb];
            float d[2] = {0.f, 0.f};
            half_block_dot(L.c[m], xa, xb, d);
            const uint32_t sw[2] = {L.s[m].x, L.s[m].y};
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const float v = fmaf(bf16_lo(sw[r]), fmaf(-128.f, xs, d[r]), bf16_hi(sw[r]) * xs);
                if (mat == 0) acc[r] += v; else acc[2 + r] += v;
            }
        }
    }
    reduce_rows(sh, acc, 4);
    const bool shared = x.kind == U_SG;
    const int ht = shared ? x.a : x.b;
    uint64_t* base = shared ? p.f_sgpart + (int64_t)ht * p.gq * 64
                            : p.f_rgpart + ((int64_t)x.a * 2 * p.G_I + ht) * p.gq * 64;
    if (threadIdx.x < 64) st_word(base + x.q * 64 + threadIdx.x, tag, __float_as_uint(row_total(sh, threadIdx.x)));
    __syncthreads();
    if (x.q != p.gq - 1) return;
    // the last piece of the half tile: sum all pieces in order, then GeGLU
    gather_words(base, p.gq * 64, tag, p.f_err, sh.gbuf);
    if (threadIdx.x < 32) {
        const int r = threadIdx.x;
        float gv = 0.f, uv = 0.f;
        for (int q = 0; q < p.gq; ++q) {
            gv += __uint_as_float(sh.gbuf[q * 64 + r]);
            uv += __uint_as_float(sh.gbuf[q * 64 + 32 + r]);
        }
        const float h = gelu_tanh(gv) * uv;
        const uint16_t h1 = f32_to_bf16(h);
        const uint16_t h2 = f32_to_bf16(h - bf16_to_f32(h1));
        uint64_t* hout = shared ? p.f_hs + 32 * ht : p.f_h + (int64_t)x.a * p.I + 32 * ht;
#pragma unroll
        for (int c = 0; c < kCopies; ++c) st_word(hout + c * p.h_stride + r, tag, ((uint32_t)h1 << 16) | h2);
    }
    __syncthreads();
    if (threadIdx.x == 0) bump(shared ? p.c_hs : p.c_h + x.a * kCtrStride);
}

// Down piece: one 64-row output tile from one source -> partial outputs.  The
// last of the n_src pieces of a tile sums them in source order into out.
__device__ __forceinline__ void run_down(const Plan& p, Shared& sh, const Unit& x, const Loads& L, uint32_t tag) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, kb = lane >> 4;
    const bool shared = x.kind == U_SD;
    const float wf = shared ? 1.0f : sh.wts[x.b];
    float acc[4] = {0.f, 0.f, 0.f, 0.f};    // rows 16*r + lane%16 of the output tile
#pragma unroll
    for (int m = 0; m < kItems; ++m) {
        const int it = wave + kWaves * m;
        if (it < 2 * x.ng) {
            const int gl = it >> 1, half = it & 1;
            const uint4 ha = *(const uint4*)(sh.hhi + 64 * gl + 8 * kb);
            const uint4 hb = *(const uint4*)(sh.hhi + 64 * gl + 32 + 8 * kb);
            const uint4 la = *(const uint4*)(sh.hlo + 64 * gl + 8 * kb);
            const uint4 lb = *(const uint4*)(sh.hlo + 64 * gl + 32 + 8 * kb);
            const float hs = sh.hsum[gl * 4 + kb];
            float d[2] = {0.f, 0.f};
            half_block_dot(L.c[m], ha, hb, d);
            half_block_dot(L.c[m], la, lb, d);
            const uint32_t sw[2] = {L.s[m].x, L.s[m].y};
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const float v = wf * fmaf(bf16_lo(sw[r]), fmaf(-128.f, hs, d[r]), bf16_hi(sw[r]) * hs);
                if (half == 0) acc[r] += v; else acc[2 + r] += v;
            }
        }
    }
    reduce_rows(sh, acc, 4);
    const int src = shared ? p.k + x.b : x.b;
    uint64_t* tilep = p.f_piece + (int64_t)x.a * p.n_src * 64;
    if (threadIdx.x < 64) st_word(tilep + src * 64 + threadIdx.x, tag, __float_as_uint(row_total(sh, threadIdx.x)));
    __syncthreads();
    if (shared || x.b != p.k - 1) return;
    // the last source of this output tile: sum every source in order
    gather_words(tilep, p.n_src * 64, tag, p.f_err, sh.gbuf);
    if (threadIdx.x < 64) {
        float v = 0.f;
        for (int s2 = 0; s2 < p.n_src; ++s2) v += __uint_as_float(sh.gbuf[s2 * 64 + threadIdx.x]);
        const int row = 64 * x.a + threadIdx.x;
        if (p.out_f32)
            ((float*)p.out)[row] = v;
        else
            ((uint16_t*)p.out)[row] = f32_to_bf16(v);
    }
    __syncthreads();
}

__device__ __forceinline__ void run_unit(const Plan& p, Shared& sh, const Unit& x, const Loads& L, uint32_t tag) {
    switch (x.kind) {
        case U_ROUTER:
            run_router(p, sh, x, L, tag);
            break;
        case U_SG:
        case U_RG:
            run_gateup(p, sh, x, L, tag);
            break;
        case U_SD:
            wait_ctr(p.c_hs, (uint32_t)(2 * p.G_s), p.f_err);
            stage_h(p, sh, p.f_hs + (blockIdx.x % kCopies) * p.h_stride, x.g0, x.ng, tag);
            run_down(p, sh, x, L, tag);
            break;
        case U_RD:
            wait_ctr(p.c_h + x.b * kCtrStride, (uint32_t)(2 * p.G_I), p.f_err);
            stage_h(p, sh, p.f_h + (blockIdx.x % kCopies) * p.h_stride + (int64_t)x.b * p.I, 0, x.ng, tag);
            run_down(p, sh, x, L, tag);
            break;
        default:
            break;
    }
}

// ----------------------------------------------------------------- the kernel

__global__ __launch_bounds__(kThreads) void k_decode(Plan p) {
    __shared__ Shared sh;
    const uint32_t tag = ld_ctr(p.f_epoch) + 1;
    const int nwg = gridDim.x;
    // Units u, u + nwg, u + 2 nwg are in flight: their loads are issued as soon
    // as their addresses are known (routed units need the expert ids first).
    // Every branch below is taken by all waves alike: `have` lives in registers
    // and changes only where every wave passes.
    int u = blockIdx.x;
    Unit u0 = decode_unit(p, u), u1 = decode_unit(p, u + nwg), u2 = decode_unit(p, u + 2 * nwg);
    Loads l0, l1, l2;
    bool i0 = false, i1 = false, i2 = false, have = false;
    if (u0.kind != U_NONE && !needs_ids(u0)) { issue_loads(p, sh, u0, l0); i0 = true; }
    if (u1.kind != U_NONE && !needs_ids(u1)) { issue_loads(p, sh, u1, l1); i1 = true; }
    stage_token(p, sh);
    while (u0.kind != U_NONE) {
        if (!i0) {
            if (!have) {
                fetch_ids(p, sh, tag);
                have = true;
            }
            issue_loads(p, sh, u0, l0);
        }
        if (!i1 && u1.kind != U_NONE && (!needs_ids(u1) || have)) { issue_loads(p, sh, u1, l1); i1 = true; }
        if (!i2 && u2.kind != U_NONE && (!needs_ids(u2) || have)) { issue_loads(p, sh, u2, l2); i2 = true; }
        run_unit(p, sh, u0, l0, tag);
        if (u0.kind == U_ROUTER && u0.a * p.rq + u0.q == p.n_router - 1) have = true;   // it ran the top-k
        u += nwg;
        u0 = u1; l0 = l1; i0 = i1;
        u1 = u2; l1 = l2; i1 = i2;
        u2 = decode_unit(p, u + 2 * nwg);
        i2 = false;
    }
    // The last workgroup to finish clears every counter and advances the epoch.
    __syncthreads();
    if (threadIdx.x == 0) sh.flag = atomicAdd(p.c_done, 1u) + 1 == (uint32_t)nwg;
    __syncthreads();
    if (sh.flag) {
        for (int i = threadIdx.x; i < p.n_ctr; i += kThreads)
            __hip_atomic_store(p.c_base + i * kCtrStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (threadIdx.x == 0) __hip_atomic_store(p.f_epoch, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

}  // namespace mq
