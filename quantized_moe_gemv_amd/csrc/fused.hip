// Single-launch decode of one token through the whole layer.
//
// One workgroup per compute unit pulls units of work from a queue ordered
// by dependency:
//   router slices (16 experts each)        -> expert scores
//   shared-expert gate/up half tiles       -> shared GeGLU activations
//   routed gate/up half tiles (k experts)  -> routed GeGLU activations
//   down bundles (4 output half tiles x one source of <= 64*G_I columns)
//                                          -> partial outputs; the last
//                                             bundle of an output range sums
//                                             them in a fixed order into out.
// A workgroup only ever waits for units that come earlier in the queue, and
// those are already held by running workgroups, so the waits always end
// (and are bounded anyway).  Results cross workgroups as 64-bit words that
// carry the call's epoch in their high half: a consumer polls a word until
// its epoch is current, which needs no cache flush.  Every reduction runs in
// a fixed order, so the output is the same bit for bit from run to run.
//
// The shared expert and the router do not depend on each other, so the
// shared gate/up streams while the scores are computed ("Decode", phase
// table: the shared branch overlaps the wait for the routing decision).
#include <math.h>

#include "device.h"
#include "plan.h"

namespace mq {

constexpr int kFusedThreads = 512;
constexpr int kWaves = kFusedThreads / 64;
constexpr int kSpinLimit = 1 << 22;

__device__ __forceinline__ uint64_t ld_word(const uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_word(uint64_t* p, uint32_t tag, uint32_t payload) {
    __hip_atomic_store(p, ((uint64_t)tag << 32) | payload, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Payload of a word once its tag is current (bounded wait).
__device__ __forceinline__ uint32_t wait_word(const uint64_t* p, uint32_t tag, uint32_t* err) {
    uint64_t v = ld_word(p);
    int spins = 0;
    while ((uint32_t)(v >> 32) != tag) {
        if (++spins > kSpinLimit) {
            atomicOr(err, 1u);
            break;
        }
        __builtin_amdgcn_s_sleep(1);
        v = ld_word(p);
    }
    return (uint32_t)v;
}

struct FusedShared {
    uint16_t x[4096];          // the token (bf16), H <= 4096
    float xsum[64 * 4];        // per (group, lane quarter) sums of x over a lane's 16 columns
    float r[4096];             // router input
    float rsum[64 * 4];        // per (group, lane quarter) sums of r over a lane's 16 columns (8-bit)
    float red[kWaves][4][32];  // cross-wave reduction
    float red2[kWaves][4][32];
    uint16_t hhi[16 * 64];     // one source's activations (<= 16 groups), bf16 high part
    uint16_t hlo[16 * 64];
    float hsum[16 * 4];
    int32_t ids[kMaxTopK];
    float wts[kMaxTopK];
    int have_ids;
    int unit;
    uint32_t flag;
};

// Stage the token and its lane sums into LDS; the router input too when asked.
__device__ __forceinline__ void stage_token(const Plan& p, FusedShared& sh, bool router) {
    const uint16_t* x = p.x;
    for (int i = threadIdx.x; i < p.H; i += kFusedThreads) sh.x[i] = x[i];
    __syncthreads();
    for (int q = threadIdx.x; q < p.G_H * 4; q += kFusedThreads) {
        const int g = q >> 2, kb = q & 3;
        float s4 = 0.f;
        for (int ks = 0; ks < 2; ++ks)
            for (int e = 0; e < 8; ++e) s4 += bf16_to_f32(sh.x[64 * g + 32 * ks + 8 * kb + e]);
        sh.xsum[q] = s4;
    }
    if (!router) {
        __syncthreads();
        return;
    }
    float ss = 0.f;
    for (int i = threadIdx.x; i < p.H; i += kFusedThreads) {
        const float v = bf16_to_f32(sh.x[i]);
        ss += v * v;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);
    if ((threadIdx.x & 63) == 0) sh.red[threadIdx.x >> 6][0][0] = ss;
    __syncthreads();
    ss = 0.f;
    for (int w = 0; w < kWaves; ++w) ss += sh.red[w][0][0];
    const float c = (1.0f / sqrtf(ss / (float)p.H + p.eps)) * (1.0f / sqrtf((float)p.H));
    for (int i = threadIdx.x; i < p.H; i += kFusedThreads)
        sh.r[i] = bf16_to_f32(sh.x[i]) * c * (p.router_scale ? p.router_scale[i] : 1.0f);
    __syncthreads();
    for (int q = threadIdx.x; q < p.G_H * 4; q += kFusedThreads) {
        const int g = q >> 2, kb = q & 3;
        float s8 = 0.f;
        for (int ks = 0; ks < 4; ++ks)
            for (int e = 0; e < 4; ++e) s8 += sh.r[64 * g + 16 * ks + 4 * kb + e];
        sh.rsum[q] = s8;
    }
    __syncthreads();
}

// Router slice s: experts 16s .. 16s+15 over all groups -> tagged score words.
__device__ __forceinline__ void unit_router(const Plan& p, FusedShared& sh, int s, uint32_t tag) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, kb = lane >> 4;
    const int tile = s >> 2, j = s & 3;
    const uint8_t* base = p.router_w + (int64_t)tile * p.G_H * kBlk8;
    float acc = 0.f;
    for (int g = wave; g < p.G_H; g += kWaves) {
        const uint8_t* blk = base + (int64_t)g * kBlk8;
        const uint4 c = *(const uint4*)(blk + (j * 64 + lane) * 16);
        const uint32_t sb = *(const uint32_t*)(blk + kCodes8 + (lane & 15) * 16 + 4 * j);
        const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
        const float* r = sh.r + 64 * g + 4 * kb;
        float d = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 rv = *(const float4*)(r + 16 * i);
            d = fmaf((float)(cw[i] & 0xFFu), rv.x, d);
            d = fmaf((float)((cw[i] >> 8) & 0xFFu), rv.y, d);
            d = fmaf((float)((cw[i] >> 16) & 0xFFu), rv.z, d);
            d = fmaf((float)(cw[i] >> 24), rv.w, d);
        }
        acc = fmaf(bf16_lo(sb), d, fmaf(bf16_hi(sb), sh.rsum[g * 4 + kb], acc));
    }
    acc = sum_kb(acc);
    if (kb == 0) sh.red[wave][0][lane] = acc;
    __syncthreads();
    if (threadIdx.x < 16) {
        float v = 0.f;
        for (int w = 0; w < kWaves; ++w) v += sh.red[w][0][threadIdx.x];
        const int e = 16 * s + threadIdx.x;
        if (e < p.E) {
            if (p.logit_bias) v += p.logit_bias[e];
            if (p.logits_out) p.logits_out[e] = v;
            st_word(p.f_logit + e, tag, __float_as_uint(v));
        }
    }
    __syncthreads();
}

// Scores -> top-k and weights in LDS (every workgroup that needs them computes them).
__device__ __forceinline__ void fetch_topk(const Plan& p, FusedShared& sh, uint32_t tag) {
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        float v[4];
        bool live[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int e = lane + 64 * m;
            live[m] = e < p.E;
            float s = -INFINITY;
            if (live[m]) {
                s = __uint_as_float(wait_word(p.f_logit + e, tag, p.f_err));
                if (!(s == s)) s = -INFINITY;
            }
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
                    sh.ids[j] = seli[j];
                    sh.wts[j] = expf(selv[j] - selv[0]) / den * (p.pes ? p.pes[seli[j]] : 1.0f);
                }
            sh.have_ids = 1;
        }
    }
    __syncthreads();
}

// Gate/up half tile: rows 32*jh .. 32*jh+31 of 64-row tile t, all G_H groups,
// -> 32 tagged words (bf16 high | bf16 low) of h = gelu_tanh(g) * u.
__device__ __forceinline__ void unit_gateup(const Plan& p, FusedShared& sh, const uint8_t* gw, const uint8_t* uw, int t, int jh,
                            uint64_t* hout, uint32_t tag) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, kb = lane >> 4;
    const uint8_t* gt = gw + (int64_t)t * p.G_H * kBlk4 + jh * 1024 + lane * 16;
    const uint8_t* ut = uw + (int64_t)t * p.G_H * kBlk4 + jh * 1024 + lane * 16;
    const int sbo = kCodes4 - jh * 1024 - lane * 16 + (lane & 15) * 16 + 8 * jh;
    constexpr int kMaxG = 8;   // groups per wave held in flight (G_H <= 64)
    uint4 cg[kMaxG], cu[kMaxG];
    uint2 sg[kMaxG], su[kMaxG];
#pragma unroll
    for (int m = 0; m < kMaxG; ++m) {
        const int g = wave + kWaves * m;
        if (g < p.G_H) {
            const int64_t o = (int64_t)g * kBlk4;
            cg[m] = ld_stream16(gt + o);
            cu[m] = ld_stream16(ut + o);
            sg[m] = *(const uint2*)(gt + o + sbo);
            su[m] = *(const uint2*)(ut + o + sbo);
        }
    }
    float ag[2] = {0.f, 0.f}, au[2] = {0.f, 0.f};
#pragma unroll
    for (int m = 0; m < kMaxG; ++m) {
        const int g = wave + kWaves * m;
        if (g < p.G_H) {
            const uint4 xa = *(const uint4*)(sh.x + 64 * g + 8 * kb);
            const uint4 xb = *(const uint4*)(sh.x + 64 * g + 32 + 8 * kb);
            const float xs = sh.xsum[g * 4 + kb];
            const uint32_t wg[4] = {cg[m].x, cg[m].y, cg[m].z, cg[m].w};
            const uint32_t wu[4] = {cu[m].x, cu[m].y, cu[m].z, cu[m].w};
            const uint32_t xk[2][4] = {{xa.x, xa.y, xa.z, xa.w}, {xb.x, xb.y, xb.z, xb.w}};
            float dg[2] = {0.f, 0.f}, du[2] = {0.f, 0.f};
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    dg[i >> 1] = dot2_bf16(q4_pair(wg[i], q), xk[i & 1][q], dg[i >> 1]);
                    du[i >> 1] = dot2_bf16(q4_pair(wu[i], q), xk[i & 1][q], du[i >> 1]);
                }
            const uint32_t sgw[2] = {sg[m].x, sg[m].y}, suw[2] = {su[m].x, su[m].y};
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                ag[r] = fmaf(bf16_lo(sgw[r]), fmaf(-128.f, xs, dg[r]), fmaf(bf16_hi(sgw[r]), xs, ag[r]));
                au[r] = fmaf(bf16_lo(suw[r]), fmaf(-128.f, xs, du[r]), fmaf(bf16_hi(suw[r]), xs, au[r]));
            }
        }
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const float vg = sum_kb(ag[r]), vu = sum_kb(au[r]);
        if (kb == 0) {
            sh.red[wave][0][16 * r + lane] = vg;
            sh.red[wave][1][16 * r + lane] = vu;
        }
    }
    __syncthreads();
    if (threadIdx.x < 32) {
        const int r = threadIdx.x;
        float gv = 0.f, uv = 0.f;
        for (int w = 0; w < kWaves; ++w) {
            gv += sh.red[w][0][r];
            uv += sh.red[w][1][r];
        }
        const float h = gelu_tanh(gv) * uv;
        const uint16_t h1 = f32_to_bf16(h);
        const uint16_t h2 = f32_to_bf16(h - bf16_to_f32(h1));
        st_word(hout + r, tag, ((uint32_t)h1 << 16) | h2);
    }
    __syncthreads();
}

// Down bundle: output half tiles 4b .. 4b+3 (rows of H) from one source.
// Source src < k: routed expert slot src (its G_I groups); else shared chunk
// src - k (groups (src-k)*G_I .. +G_I of the shared intermediate).
__device__ __forceinline__ void unit_down(const Plan& p, FusedShared& sh, int b, int src, uint32_t tag) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, kb = lane >> 4;
    const bool routed = src < p.k;
    int g0, ng, gtot;
    const uint8_t* dw;
    const uint64_t* hsrc;
    if (routed) {
        g0 = 0;
        ng = p.G_I;
        gtot = p.G_I;
        dw = p.pool_base + (int64_t)sh.ids[src] * p.expert_stride + p.down_off;
        hsrc = p.f_h + (int64_t)src * p.I;
    } else {
        g0 = (src - p.k) * p.G_I;
        ng = min(p.G_I, p.G_s - g0);
        gtot = p.G_s;
        dw = p.sh_down;
        hsrc = p.f_hs;
    }
    const int nho = min(4, 2 * p.G_H - 4 * b);    // output half tiles in this bundle
    const int npairs = nho * ng;
    // issue the weight loads first: they do not depend on the activations
    constexpr int kMaxP = 8;                      // (half tile, group) pairs per wave (<= 64 in a bundle)
    uint4 c[kMaxP];
    uint2 sbv[kMaxP];
#pragma unroll
    for (int m = 0; m < kMaxP; ++m) {
        const int q = wave + kWaves * m;
        if (q < npairs) {
            const int ol = q % nho, gl = q / nho;
            const int ho = 4 * b + ol;
            const uint8_t* blk = dw + ((int64_t)(ho >> 1) * gtot + g0 + gl) * kBlk4;
            c[m] = ld_stream16(blk + (ho & 1) * 1024 + lane * 16);
            sbv[m] = *(const uint2*)(blk + kCodes4 + (lane & 15) * 16 + 8 * (ho & 1));
        }
    }
    // activations of this source: 64 words per group
    for (int q = threadIdx.x; q < ng * 64; q += kFusedThreads) {
        const uint32_t v = wait_word(hsrc + 64 * g0 + q, tag, p.f_err);
        sh.hhi[q] = (uint16_t)(v >> 16);
        sh.hlo[q] = (uint16_t)(v & 0xFFFFu);
    }
    __syncthreads();
    for (int q = threadIdx.x; q < ng * 4; q += kFusedThreads) {
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
    const float wf = routed ? sh.wts[src] : 1.0f;
    float acc[4][2];
#pragma unroll
    for (int o = 0; o < 4; ++o) acc[o][0] = acc[o][1] = 0.f;
#pragma unroll
    for (int m = 0; m < kMaxP; ++m) {
        const int q = wave + kWaves * m;
        if (q < npairs) {
            const int ol = q % nho, gl = q / nho;
            const uint4 ha = *(const uint4*)(sh.hhi + 64 * gl + 8 * kb);
            const uint4 hb = *(const uint4*)(sh.hhi + 64 * gl + 32 + 8 * kb);
            const uint4 la = *(const uint4*)(sh.hlo + 64 * gl + 8 * kb);
            const uint4 lb = *(const uint4*)(sh.hlo + 64 * gl + 32 + 8 * kb);
            const float hs = sh.hsum[gl * 4 + kb];
            const uint32_t w[4] = {c[m].x, c[m].y, c[m].z, c[m].w};
            const uint32_t hk[2][4] = {{ha.x, ha.y, ha.z, ha.w}, {hb.x, hb.y, hb.z, hb.w}};
            const uint32_t lk[2][4] = {{la.x, la.y, la.z, la.w}, {lb.x, lb.y, lb.z, lb.w}};
            float d[2] = {0.f, 0.f};
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int qq = 0; qq < 4; ++qq) {
                    const uint32_t pr = q4_pair(w[i], qq);
                    d[i >> 1] = dot2_bf16(pr, hk[i & 1][qq], d[i >> 1]);
                    d[i >> 1] = dot2_bf16(pr, lk[i & 1][qq], d[i >> 1]);
                }
            const uint32_t sw[2] = {sbv[m].x, sbv[m].y};
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const float v = fmaf(bf16_lo(sw[r]), fmaf(-128.f, hs, d[r]), bf16_hi(sw[r]) * hs);
#pragma unroll
                for (int o = 0; o < 4; ++o)
                    if (o == ol) acc[o][r] = fmaf(wf, v, acc[o][r]);
            }
        }
    }
#pragma unroll
    for (int o = 0; o < 4; ++o)
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const float v = sum_kb(acc[o][r]);
            if (kb == 0) sh.red2[wave][o][16 * r + lane] = v;
        }
    __syncthreads();
    uint64_t* piece = p.f_piece + ((int64_t)b * p.n_src + src) * 128;
    if (threadIdx.x < 128) {
        const int o = threadIdx.x >> 5, r = threadIdx.x & 31;
        float v = 0.f;
        for (int w = 0; w < kWaves; ++w) v += sh.red2[w][o][r];
        if (o < nho) st_word(piece + threadIdx.x, tag, __float_as_uint(v));
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t old = atomicAdd(p.f_bundle + b, 1u);
        sh.flag = old + 1 == tag * (uint32_t)p.n_src;   // n_src arrivals per bundle per call
    }
    __syncthreads();
    if (sh.flag && threadIdx.x < nho * 32) {
        // last source of this output range: fixed-order sum of all pieces
        const int o = threadIdx.x >> 5, r = threadIdx.x & 31;
        float v = 0.f;
        for (int s2 = 0; s2 < p.n_src; ++s2)
            v += __uint_as_float(
                wait_word(p.f_piece + ((int64_t)b * p.n_src + s2) * 128 + threadIdx.x, tag, p.f_err));
        const int row = (4 * b + o) * 32 + r;
        if (p.out_f32)
            ((float*)p.out)[row] = v;
        else
            ((uint16_t*)p.out)[row] = f32_to_bf16(v);
    }
    __syncthreads();
}

__global__ __launch_bounds__(kFusedThreads) void k_decode(Plan p) {
    __shared__ FusedShared sh;
    if (threadIdx.x == 0) sh.have_ids = 0;
    const uint32_t epoch = __hip_atomic_load(p.f_epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t tag = epoch + 1;
    const int nwg = gridDim.x;
    const int n_dyn = max(0, p.n_units - nwg);
    const uint32_t qbase = epoch * (uint32_t)(n_dyn + nwg);
    stage_token(p, sh, true);
    int u = blockIdx.x;
    bool first = true;
    __syncthreads();
    while (true) {
        if (!first) {
            if (threadIdx.x == 0) {
                const uint32_t v = atomicAdd(p.f_queue, 1u) - qbase;
                sh.unit = (int)v < n_dyn ? nwg + (int)v : -1;
            }
            __syncthreads();
            u = sh.unit;
            __syncthreads();
            if (u < 0) break;
        } else {
            first = false;
            if (u >= p.n_units) continue;   // no static unit: go take (and overshoot) the queue once
        }
        int v = u;
        if (v < p.n_router) {
            unit_router(p, sh, v, tag);
            continue;
        }
        v -= p.n_router;
        if (v < p.n_sg) {
            unit_gateup(p, sh, p.sh_gate, p.sh_up, v >> 1, v & 1, p.f_hs + 32 * v, tag);
            continue;
        }
        v -= p.n_sg;
        if (v < p.n_rg) {
            if (!sh.have_ids) fetch_topk(p, sh, tag);
            const int per = 2 * p.G_I, j = v / per, ht = v % per;
            if (v == 0 && threadIdx.x < p.k) {
                if (p.ids_out) p.ids_out[threadIdx.x] = sh.ids[threadIdx.x];
                if (p.w_out) p.w_out[threadIdx.x] = sh.wts[threadIdx.x];
            }
            const uint8_t* blob = p.pool_base + (int64_t)sh.ids[j] * p.expert_stride;
            unit_gateup(p, sh, blob + p.gate_off, blob + p.up_off, ht >> 1, ht & 1,
                        p.f_h + (int64_t)j * p.I + 32 * ht, tag);
            continue;
        }
        v -= p.n_rg;
        const int b = v / p.n_src, src = v % p.n_src;
        if (src < p.k && !sh.have_ids) fetch_topk(p, sh, tag);
        unit_down(p, sh, b, src, tag);
    }
    // the last workgroup to finish advances the epoch for the next call
    if (threadIdx.x == 0) {
        const uint32_t old = atomicAdd(p.f_done, 1u);
        if (old + 1 == (epoch + 1) * (uint32_t)nwg)
            __hip_atomic_store(p.f_epoch, epoch + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

}  // namespace mq
