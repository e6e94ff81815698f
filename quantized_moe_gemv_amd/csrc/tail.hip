// The layer tail on the multi-launch paths: one workgroup per token row
// takes the shared branch s and the weighted routed sum r from the path's
// partial results, and writes
//     out = scalar * (residual + N_o(N_s(s) + N_r(r))),
//     N(v) = v / sqrt(mean(v^2) + eps) * w   (no norm where w is null),
// in fp32, rounded once ("Decode", phase table cb2: post-FFN norms,
// residual and layer scalar after the combine).
#include <math.h>

#include "device.h"
#include "plan.h"

namespace mq {

constexpr int kTailThreads = 1024;
constexpr int kTailIters = 4;      // H <= 4 * 4 * 1024

// Sums of two values over the workgroup (every thread gets both totals).
__device__ __forceinline__ float2 block_sum2(float a, float b, float2* buf) {
    a = wave_sum(a);
    b = wave_sum(b);
    const int w = threadIdx.x >> 6;
    __syncthreads();   // buf may still be read from a previous use
    if ((threadIdx.x & 63) == 0) buf[w] = make_float2(a, b);
    __syncthreads();
    float2 t = make_float2(0.f, 0.f);
    for (int i = 0; i < kTailThreads / 64; ++i) {
        t.x += buf[i].x;
        t.y += buf[i].y;
    }
    return t;
}

__device__ __forceinline__ float4 ld4(const float* p) { return *(const float4*)p; }
__device__ __forceinline__ void add4(float4& a, const float4& b) {
    a.x += b.x;
    a.y += b.y;
    a.z += b.z;
    a.w += b.w;
}

// SRC 0: the GEMV path's down-projection splits (dpart[t][split][H]: splits
// 0..2 routed, split 3 shared when the layer has a shared expert, else all
// four routed).  SRC 1: the grouped path's weighted pair outputs (ysort:
// the k slots of the token through inv, then its shared virtual experts).
template <int SRC>
__device__ __forceinline__ void tail_rows(const Plan& p) {
    __shared__ float2 buf[kTailThreads / 64];
    const int t = blockIdx.x;
    float4 s[kTailIters], r[kTailIters];
    float ss = 0.f, rr = 0.f;
#pragma unroll
    for (int m = 0; m < kTailIters; ++m) {
        const int i = 4 * (threadIdx.x + kTailThreads * m);
        s[m] = r[m] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (i >= p.H) continue;
        if (SRC == 0) {
            const float* d = p.dpart + (int64_t)t * kDownSplits * p.H + i;
            const int nrs = p.has_shared ? kDownSplits - 1 : kDownSplits;
            for (int q = 0; q < nrs; ++q) add4(r[m], ld4(d + (int64_t)q * p.H));
            if (p.has_shared) s[m] = ld4(d + (int64_t)(kDownSplits - 1) * p.H);
        } else {
            for (int j = 0; j < p.k; ++j) add4(r[m], ld4(p.ysort + (int64_t)p.inv[t * p.k + j] * p.H + i));
            for (int j = 0; j < p.n_vs_dn; ++j)
                add4(s[m], ld4(p.ysort + ((int64_t)p.T * p.k + (int64_t)j * p.T + t) * p.H + i));
        }
        ss += (s[m].x * s[m].x + s[m].y * s[m].y) + (s[m].z * s[m].z + s[m].w * s[m].w);
        rr += (r[m].x * r[m].x + r[m].y * r[m].y) + (r[m].z * r[m].z + r[m].w * r[m].w);
    }
    const float2 tot = block_sum2(ss, rr, buf);
    const float a = p.tn_s ? 1.0f / sqrtf(tot.x / (float)p.H + p.t_eps) : 1.0f;
    const float b = p.tn_r ? 1.0f / sqrtf(tot.y / (float)p.H + p.t_eps) : 1.0f;
    float4 f[kTailIters];
    float ff = 0.f;
#pragma unroll
    for (int m = 0; m < kTailIters; ++m) {
        const int i = 4 * (threadIdx.x + kTailThreads * m);
        f[m] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (i >= p.H) continue;
        const float4 ws = p.tn_s ? ld4(p.tn_s + i) : make_float4(1.f, 1.f, 1.f, 1.f);
        const float4 wr = p.tn_r ? ld4(p.tn_r + i) : make_float4(1.f, 1.f, 1.f, 1.f);
        f[m].x = a * ws.x * s[m].x + b * wr.x * r[m].x;
        f[m].y = a * ws.y * s[m].y + b * wr.y * r[m].y;
        f[m].z = a * ws.z * s[m].z + b * wr.z * r[m].z;
        f[m].w = a * ws.w * s[m].w + b * wr.w * r[m].w;
        ff += (f[m].x * f[m].x + f[m].y * f[m].y) + (f[m].z * f[m].z + f[m].w * f[m].w);
    }
    float c = p.tn_o ? 1.0f / sqrtf(block_sum2(ff, 0.f, buf).x / (float)p.H + p.t_eps) : 1.0f;
    // the grouped path's single GEMM launch gave up a wait: NaN rows rather
    // than plausible ones
    if (SRC == 1 && (*p.f_err & kErrWait)) c = __builtin_nanf("");
#pragma unroll
    for (int m = 0; m < kTailIters; ++m) {
        const int i = 4 * (threadIdx.x + kTailThreads * m);
        if (i >= p.H) continue;
        const float4 wo = p.tn_o ? ld4(p.tn_o + i) : make_float4(1.f, 1.f, 1.f, 1.f);
        float res[4] = {0.f, 0.f, 0.f, 0.f};
        if (p.t_res) {
            const uint2 rv = *(const uint2*)(p.t_res + (int64_t)t * p.t_res_stride + i);
            res[0] = bf16_lo(rv.x);
            res[1] = bf16_hi(rv.x);
            res[2] = bf16_lo(rv.y);
            res[3] = bf16_hi(rv.y);
        }
        const float o[4] = {p.t_scalar * (res[0] + c * wo.x * f[m].x), p.t_scalar * (res[1] + c * wo.y * f[m].y),
                            p.t_scalar * (res[2] + c * wo.z * f[m].z), p.t_scalar * (res[3] + c * wo.w * f[m].w)};
        const int64_t off = (int64_t)t * p.out_stride + i;
        if (p.out_f32) {
#pragma unroll
            for (int e = 0; e < 4; ++e) ((float*)p.out)[off + e] = o[e];
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) ((uint16_t*)p.out)[off + e] = f32_to_bf16(o[e]);
        }
    }
}

// grid (T), block kTailThreads.
__global__ __launch_bounds__(kTailThreads) void k_tail_gemv(Plan p) { tail_rows<0>(p); }
__global__ __launch_bounds__(kTailThreads) void k_tail_grouped(Plan p) { tail_rows<1>(p); }

}  // namespace mq
