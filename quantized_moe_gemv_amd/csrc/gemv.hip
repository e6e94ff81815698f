// Router, top-k and the GEMV expert path (few tokens per call).
//
// All weights are read in the DEV_V1 block layout; each lane of a wave owns
// four rows of a 64-row tile and 16 columns of every group block, so a
// block costs each lane two 16-byte code loads and one 16-byte load of
// (scale, bias) pairs, and the dot products need no dequantised weights:
//   sum_c (s q_c + b) x_c = s * sum_c q_c x_c + b * sum_c x_c.
#include <math.h>

#include "device.h"
#include "plan.h"

namespace mq {


// Per token: scaled router input r = x / sqrt(mean(x^2) + eps) * router_scale / sqrt(H),
// and the per-lane column sums used by the 8-bit (r) and 4-bit (x) block dots.
__global__ __launch_bounds__(256) void k_prep(Plan p) {
    const int t = blockIdx.x;
    const uint16_t* x = p.x + (int64_t)t * p.x_stride;
    __shared__ float red[4];
    float ss = 0.f;
    for (int i = threadIdx.x; i < p.H; i += 256) {
        float v = bf16_to_f32(x[i]);
        ss += v * v;
    }
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    ss = (red[0] + red[1]) + (red[2] + red[3]);
    const float c = (1.0f / sqrtf(ss / (float)p.H + p.eps)) * (1.0f / sqrtf((float)p.H));
    float* r = p.r + (int64_t)t * p.H;
    for (int i = threadIdx.x; i < p.H; i += 256) {
        float rs = p.router_scale ? p.router_scale[i] : 1.0f;
        r[i] = bf16_to_f32(x[i]) * c * rs;
    }
    for (int q = threadIdx.x; q < p.G_H * 4; q += 256) {
        const int g = q >> 2, kb = q & 3;
        float s8 = 0.f, s4 = 0.f;
        for (int ks = 0; ks < 4; ++ks)
            for (int e = 0; e < 4; ++e) {
                int i = 64 * g + 16 * ks + 4 * kb + e;
                float rs = p.router_scale ? p.router_scale[i] : 1.0f;
                s8 += bf16_to_f32(x[i]) * c * rs;
            }
        for (int ks = 0; ks < 2; ++ks)
            for (int e = 0; e < 8; ++e) s4 += bf16_to_f32(x[64 * g + 32 * ks + 8 * kb + e]);
        p.rsum8[((int64_t)t * p.G_H + g) * 4 + kb] = s8;
        p.xsum4[((int64_t)t * p.G_H + g) * 4 + kb] = s4;
        if (p.ebits == 8) {   // the same sums over the 8-bit blocks' lane columns
            float x8 = 0.f;
            for (int ks = 0; ks < 4; ++ks)
                for (int e = 0; e < 4; ++e) x8 += bf16_to_f32(x[64 * g + 16 * ks + 4 * kb + e]);
            p.xsum8[((int64_t)t * p.G_H + g) * 4 + kb] = x8;
        }
    }
}

// Partial router scores: grid (E_pad/64 row tiles, rsplit column splits,
// ceil(T / kRouterTokens) token chunks), 4 waves splitting the groups.
__global__ __launch_bounds__(256) void k_router(Plan p) {
    const int tile = blockIdx.x, split = blockIdx.y, t0 = blockIdx.z * kRouterTokens;
    const int wave = wave_id(), lane = threadIdx.x & 63, kb = lane >> 4;
    const int g0 = split * p.rgroups, g1 = min(p.G_H, g0 + p.rgroups);
    const int nt = min(kRouterTokens, p.T - t0);
    float acc[kRouterTokens][4];
#pragma unroll
    for (int tt = 0; tt < kRouterTokens; ++tt)
#pragma unroll
        for (int m = 0; m < 4; ++m) acc[tt][m] = 0.f;
    const uint8_t* base = p.router_w + (int64_t)tile * p.G_H * kBlk8;
    for (int g = g0 + wave; g < g1; g += 4) {
        const uint8_t* blk = base + (int64_t)g * kBlk8;
        uint4 c[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) c[j] = *(const uint4*)(blk + (j * 64 + lane) * 16);
        const uint4 sb = *(const uint4*)(blk + kCodes8 + (lane & 15) * 16);
        const uint32_t sbw[4] = {sb.x, sb.y, sb.z, sb.w};
#pragma unroll
        for (int tt = 0; tt < kRouterTokens; ++tt) {
            if (tt < nt) {
                const float* r = p.r + (int64_t)(t0 + tt) * p.H + 64 * g + 4 * kb;
                float4 rv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) rv[i] = *(const float4*)(r + 16 * i);
                const float rs = p.rsum8[((int64_t)(t0 + tt) * p.G_H + g) * 4 + kb];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t cw[4] = {c[j].x, c[j].y, c[j].z, c[j].w};
                    float d = 0.f;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        d = fmaf((float)(cw[i] & 0xFFu), rv[i].x, d);
                        d = fmaf((float)((cw[i] >> 8) & 0xFFu), rv[i].y, d);
                        d = fmaf((float)((cw[i] >> 16) & 0xFFu), rv[i].z, d);
                        d = fmaf((float)(cw[i] >> 24), rv[i].w, d);
                    }
                    acc[tt][j] = fmaf(bf16_lo(sbw[j]), d, fmaf(bf16_hi(sbw[j]), rs, acc[tt][j]));
                }
            }
        }
    }
    __shared__ float red[4][kRouterTokens][64];
#pragma unroll
    for (int tt = 0; tt < kRouterTokens; ++tt)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            float v = sum_kb(acc[tt][m]);
            if (kb == 0) red[wave][tt][16 * m + lane] = v;
        }
    __syncthreads();
    for (int q = threadIdx.x; q < nt * 64; q += 256) {
        const int tt = q >> 6, row = q & 63;
        float v = (red[0][tt][row] + red[1][tt][row]) + (red[2][tt][row] + red[3][tt][row]);
        p.plog[((int64_t)split * p.T + t0 + tt) * p.E_pad + tile * 64 + row] = v;
    }
}

// Scores, top-k (higher score first, ties to the lower expert) and the
// softmax weights over the selected scores times per_expert_scale.  One
// workgroup per token: each expert's rank is the number of scores that beat
// it, and the experts of rank < k are the selection, in rank order.
__global__ __launch_bounds__(256) void k_topk(Plan p) {
    const int t = blockIdx.x;
    __shared__ float lg[kMaxExperts];
    __shared__ float selv[kMaxTopK];
    __shared__ int seli[kMaxTopK];
    for (int e = threadIdx.x; e < p.E; e += 256) {
        float s = 0.f;
        for (int sp = 0; sp < p.rsplit; ++sp) s += p.plog[((int64_t)sp * p.T + t) * p.E_pad + e];
        if (p.logit_bias) s += p.logit_bias[e];
        if (p.logits_out) p.logits_out[(int64_t)t * p.E + e] = s;
        lg[e] = (s == s) ? s : -INFINITY;   // a NaN score ranks last; ids stay distinct
    }
    __syncthreads();
    for (int e = threadIdx.x; e < p.E; e += 256) {
        const float v = lg[e];
        int rank = 0;
        for (int o = 0; o < p.E; ++o) rank += (lg[o] > v) || (lg[o] == v && o < e);
        if (rank < p.k) {
            selv[rank] = v;
            seli[rank] = e;
        }
    }
    __syncthreads();
    if (threadIdx.x < p.k) {
        const int j = threadIdx.x;
        float den = 0.f;
        for (int i = 0; i < p.k; ++i) den += expf(selv[i] - selv[0]);
        const int e = seli[j];
        const float w = expf(selv[j] - selv[0]) / den * (p.pes ? p.pes[e] : 1.0f);
        p.ids[t * p.k + j] = e;
        p.wts[t * p.k + j] = w;
        if (p.ids_out) p.ids_out[t * p.k + j] = e;
        if (p.w_out) p.w_out[t * p.k + j] = w;
    }
}

// Partial dots of one lane over one 8-bit DEV_V1 block: rows 16*m + lane%16
// (m = 0..3), over the lane's 16 columns 16*i + 4*(lane/16) + 0..3 (i = 0..3).
// c[m]: the lane's code words of row block m; xv[i]: four fp32 inputs of
// columns 16*i + 4*(lane/16)... Adds sum(q * x) of row m to d[m].
__device__ __forceinline__ void q8_block_dot(const uint4 c[4], const float xv[4][4], float d[4]) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const uint32_t cw[4] = {c[m].x, c[m].y, c[m].z, c[m].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            d[m] = fmaf((float)(cw[i] & 0xFFu), xv[i][0], d[m]);
            d[m] = fmaf((float)((cw[i] >> 8) & 0xFFu), xv[i][1], d[m]);
            d[m] = fmaf((float)((cw[i] >> 16) & 0xFFu), xv[i][2], d[m]);
            d[m] = fmaf((float)(cw[i] >> 24), xv[i][3], d[m]);
        }
    }
}

// Gate and up projections of one 64-row tile for one (token, expert) pair,
// or for the shared expert, with GeGLU: h = gelu_tanh(g) * u.  h is stored
// as a bf16 high/low pair (h ~= hi + lo to 2^-16) for the down projection,
// with the sums of each lane set's columns of it (the lane columns of
// BITS-bit blocks).  grid (T, k * I/64 + Is/64).
template <int BITS>
__device__ __forceinline__ void gateup_tile(const Plan& p) {
    constexpr int BLK = blk_bytes(BITS);
    const int t = blockIdx.x, item = blockIdx.y + p.gu_item0;
    const int wave = wave_id(), lane = threadIdx.x & 63, kb = lane >> 4;
    const int It = p.I / 64, routed = p.k * It;
    const uint8_t *gw, *uw;
    uint16_t *hi, *lo;
    float* hsum;
    if (item < routed) {
        const int j = item / It, rt = item % It;
        const int e = p.slots ? p.slots[t * p.k + j] : p.ids[t * p.k + j];
        const uint8_t* blob = p.pool_base + (int64_t)e * p.expert_stride;
        gw = blob + p.gate_off + (int64_t)rt * p.G_H * BLK;
        uw = blob + p.up_off + (int64_t)rt * p.G_H * BLK;
        const int64_t hrow = ((int64_t)t * p.k + j) * p.I + rt * 64;
        hi = p.hhi + hrow;
        lo = p.hlo + hrow;
        hsum = p.hsum + (((int64_t)t * p.k + j) * p.G_I + rt) * 4;
    } else {
        const int rt = item - routed;
        gw = p.sh_gate + (int64_t)rt * p.G_H * BLK;
        uw = p.sh_up + (int64_t)rt * p.G_H * BLK;
        hi = p.shi + (int64_t)t * p.Is + rt * 64;
        lo = p.slo + (int64_t)t * p.Is + rt * 64;
        hsum = p.ssum + ((int64_t)t * p.G_s + rt) * 4;
    }
    const uint16_t* x = p.x + (int64_t)t * p.x_stride;
    const float* xsum = BITS == 4 ? p.xsum4 : p.xsum8;
    float ag[4] = {0.f, 0.f, 0.f, 0.f}, au[4] = {0.f, 0.f, 0.f, 0.f};
    for (int g = wave; g < p.G_H; g += 4) {
        const uint8_t* bg = gw + (int64_t)g * BLK;
        const uint8_t* bu = uw + (int64_t)g * BLK;
        const uint4 sg = *(const uint4*)(bg + code_bytes(BITS) + (lane & 15) * 16);
        const uint4 su = *(const uint4*)(bu + code_bytes(BITS) + (lane & 15) * 16);
        const float xs = xsum[((int64_t)t * p.G_H + g) * 4 + kb];
        float dg[4] = {0.f, 0.f, 0.f, 0.f}, du[4] = {0.f, 0.f, 0.f, 0.f};
        const uint32_t sgw[4] = {sg.x, sg.y, sg.z, sg.w}, suw[4] = {su.x, su.y, su.z, su.w};
        if constexpr (BITS == 4) {
            const uint4 g0 = *(const uint4*)(bg + lane * 16), g1 = *(const uint4*)(bg + 1024 + lane * 16);
            const uint4 u0 = *(const uint4*)(bu + lane * 16), u1 = *(const uint4*)(bu + 1024 + lane * 16);
            const uint4 xa = *(const uint4*)(x + 64 * g + 8 * kb);
            const uint4 xb = *(const uint4*)(x + 64 * g + 32 + 8 * kb);
            q4_block_dot(g0, g1, xa, xb, dg);
            q4_block_dot(u0, u1, xa, xb, du);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                ag[m] = fmaf(bf16_lo(sgw[m]), fmaf(-128.f, xs, dg[m]), fmaf(bf16_hi(sgw[m]), xs, ag[m]));
                au[m] = fmaf(bf16_lo(suw[m]), fmaf(-128.f, xs, du[m]), fmaf(bf16_hi(suw[m]), xs, au[m]));
            }
        } else {
            uint4 gc[4], uc[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                gc[m] = *(const uint4*)(bg + (m * 64 + lane) * 16);
                uc[m] = *(const uint4*)(bu + (m * 64 + lane) * 16);
            }
            float xv[4][4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint2 v = *(const uint2*)(x + 64 * g + 16 * i + 4 * kb);
                xv[i][0] = bf16_lo(v.x);
                xv[i][1] = bf16_hi(v.x);
                xv[i][2] = bf16_lo(v.y);
                xv[i][3] = bf16_hi(v.y);
            }
            q8_block_dot(gc, xv, dg);
            q8_block_dot(uc, xv, du);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                ag[m] = fmaf(bf16_lo(sgw[m]), dg[m], fmaf(bf16_hi(sgw[m]), xs, ag[m]));
                au[m] = fmaf(bf16_lo(suw[m]), du[m], fmaf(bf16_hi(suw[m]), xs, au[m]));
            }
        }
    }
    __shared__ float red[4][2][64];
    __shared__ float hh[64];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        float vg = sum_kb(ag[m]), vu = sum_kb(au[m]);
        if (kb == 0) {
            red[wave][0][16 * m + lane] = vg;
            red[wave][1][16 * m + lane] = vu;
        }
    }
    __syncthreads();
    if (threadIdx.x < 64) {
        const int r = threadIdx.x;
        const float gv = (red[0][0][r] + red[1][0][r]) + (red[2][0][r] + red[3][0][r]);
        const float uv = (red[0][1][r] + red[1][1][r]) + (red[2][1][r] + red[3][1][r]);
        const float h = gelu_tanh(gv) * uv;
        const uint16_t h1 = f32_to_bf16(h);
        const uint16_t h2 = f32_to_bf16(h - bf16_to_f32(h1));
        hi[r] = h1;
        lo[r] = h2;
        hh[r] = bf16_to_f32(h1) + bf16_to_f32(h2);
    }
    __syncthreads();
    if (threadIdx.x < 4) {
        const int q = threadIdx.x;
        float s = 0.f;
        if (BITS == 4) {
            for (int ks = 0; ks < 2; ++ks)
                for (int e = 0; e < 8; ++e) s += hh[32 * ks + 8 * q + e];
        } else {
            for (int ks = 0; ks < 4; ++ks)
                for (int e = 0; e < 4; ++e) s += hh[16 * ks + 4 * q + e];
        }
        hsum[q] = s;
    }
}

__global__ __launch_bounds__(256) void k_gateup(Plan p) { gateup_tile<4>(p); }
__global__ __launch_bounds__(256) void k_gateup8(Plan p) { gateup_tile<8>(p); }

// Down projections of one 64-row tile of the output for one token: the k
// routed experts (weighted) and the shared expert, split over kDownSplits
// workgroups whose partial sums k_combine adds in a fixed order.  With a
// shared expert, splits 0 .. kDownSplits-2 take the routed sources and the
// last split the shared expert's, so the two branches stay apart for the
// layer tail.  grid (T, H/64, kDownSplits).
template <int BITS>
__device__ __forceinline__ void down_tile(const Plan& p) {
    constexpr int BLK = blk_bytes(BITS);
    const int t = blockIdx.x, rt = blockIdx.y, split = blockIdx.z + p.dn_split0;
    const int wave = wave_id(), lane = threadIdx.x & 63, kb = lane >> 4;
    const int nr = p.k * p.G_I;
    int b0, b1;
    if (!p.has_shared) {
        b0 = split * nr / kDownSplits;
        b1 = (split + 1) * nr / kDownSplits;
    } else if (split < kDownSplits - 1) {
        b0 = split * nr / (kDownSplits - 1);
        b1 = (split + 1) * nr / (kDownSplits - 1);
    } else {
        b0 = nr;
        b1 = nr + p.G_s;
    }
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int b = b0 + wave; b < b1; b += 4) {
        const uint8_t* blk;
        const uint16_t *hi, *lo;
        float hs, wf;
        if (b < nr) {
            const int j = b / p.G_I, g = b % p.G_I;
            const int e = p.slots ? p.slots[t * p.k + j] : p.ids[t * p.k + j];
            blk = p.pool_base + (int64_t)e * p.expert_stride + p.down_off + ((int64_t)rt * p.G_I + g) * BLK;
            const int64_t hrow = ((int64_t)t * p.k + j) * p.I + 64 * g;
            hi = p.hhi + hrow;
            lo = p.hlo + hrow;
            hs = p.hsum[(((int64_t)t * p.k + j) * p.G_I + g) * 4 + kb];
            wf = p.wts[t * p.k + j];
        } else {
            const int g = b - nr;
            blk = p.sh_down + ((int64_t)rt * p.G_s + g) * BLK;
            hi = p.shi + (int64_t)t * p.Is + 64 * g;
            lo = p.slo + (int64_t)t * p.Is + 64 * g;
            hs = p.ssum[((int64_t)t * p.G_s + g) * 4 + kb];
            wf = 1.0f;
        }
        const uint4 sb = *(const uint4*)(blk + code_bytes(BITS) + (lane & 15) * 16);
        const uint32_t sbw[4] = {sb.x, sb.y, sb.z, sb.w};
        float d[4] = {0.f, 0.f, 0.f, 0.f};
        if constexpr (BITS == 4) {
            const uint4 c0 = *(const uint4*)(blk + lane * 16), c1 = *(const uint4*)(blk + 1024 + lane * 16);
            const uint4 ha = *(const uint4*)(hi + 8 * kb), hb = *(const uint4*)(hi + 32 + 8 * kb);
            const uint4 la = *(const uint4*)(lo + 8 * kb), lb = *(const uint4*)(lo + 32 + 8 * kb);
            q4_block_dot(c0, c1, ha, hb, d);
            q4_block_dot(c0, c1, la, lb, d);
#pragma unroll
            for (int m = 0; m < 4; ++m)
                acc[m] = fmaf(wf, fmaf(bf16_lo(sbw[m]), fmaf(-128.f, hs, d[m]), bf16_hi(sbw[m]) * hs), acc[m]);
        } else {
            uint4 c[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) c[m] = *(const uint4*)(blk + (m * 64 + lane) * 16);
            float hv[4][4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint2 vh = *(const uint2*)(hi + 16 * i + 4 * kb), vl = *(const uint2*)(lo + 16 * i + 4 * kb);
                hv[i][0] = bf16_lo(vh.x) + bf16_lo(vl.x);
                hv[i][1] = bf16_hi(vh.x) + bf16_hi(vl.x);
                hv[i][2] = bf16_lo(vh.y) + bf16_lo(vl.y);
                hv[i][3] = bf16_hi(vh.y) + bf16_hi(vl.y);
            }
            q8_block_dot(c, hv, d);
#pragma unroll
            for (int m = 0; m < 4; ++m)
                acc[m] = fmaf(wf, fmaf(bf16_lo(sbw[m]), d[m], bf16_hi(sbw[m]) * hs), acc[m]);
        }
    }
    __shared__ float red[4][64];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        float v = sum_kb(acc[m]);
        if (kb == 0) red[wave][16 * m + lane] = v;
    }
    __syncthreads();
    if (threadIdx.x < 64) {
        const int r = threadIdx.x;
        p.dpart[((int64_t)t * kDownSplits + split) * p.H + rt * 64 + r] =
            (red[0][r] + red[1][r]) + (red[2][r] + red[3][r]);
    }
}

__global__ __launch_bounds__(256) void k_down(Plan p) { down_tile<4>(p); }
__global__ __launch_bounds__(256) void k_down8(Plan p) { down_tile<8>(p); }

// out[t][i] = sum of the kDownSplits partials, rounded once.  grid (T, ceil(H/256)).
__global__ __launch_bounds__(256) void k_combine(Plan p) {
    const int t = blockIdx.x, i = blockIdx.y * 256 + threadIdx.x;
    if (i >= p.H) return;
    const float* d = p.dpart + (int64_t)t * kDownSplits * p.H + i;
    float v = 0.f;
#pragma unroll
    for (int s = 0; s < kDownSplits; ++s) v += d[(int64_t)s * p.H];
    if (p.out_f32)
        ((float*)p.out)[(int64_t)t * p.out_stride + i] = v;
    else
        ((uint16_t*)p.out)[(int64_t)t * p.out_stride + i] = f32_to_bf16(v);
}

// Unit-weight RMS norm of bf16 rows.  grid (T).
__global__ __launch_bounds__(256) void k_rmsnorm(const uint16_t* x, int64_t xs, uint16_t* y, int64_t ys, int H,
                                                 float eps) {
    const int t = blockIdx.x;
    const uint16_t* xr = x + (int64_t)t * xs;
    __shared__ float red[4];
    float ss = 0.f;
    for (int i = threadIdx.x; i < H; i += 256) {
        float v = bf16_to_f32(xr[i]);
        ss += v * v;
    }
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    ss = (red[0] + red[1]) + (red[2] + red[3]);
    const float inv = 1.0f / sqrtf(ss / (float)H + eps);
    __syncthreads();
    for (int i = threadIdx.x; i < H; i += 256) y[(int64_t)t * ys + i] = f32_to_bf16(bf16_to_f32(xr[i]) * inv);
}

// Parity hooks: every code, or every fp32 weight, of a DEV_V1 tensor.
// grid (row tiles * groups), block 256: thread q handles words q, q+256, ...
__global__ __launch_bounds__(256) void k_debug_read(const uint8_t* data, int rows, int cols, int bits,
                                                    uint8_t* codes_out, float* w_out) {
    const int G = cols / 64;
    const int tile = blockIdx.x / G, g = blockIdx.x % G;
    const uint8_t* blk = data + (int64_t)blockIdx.x * (bits == 4 ? kBlk4 : kBlk8);
    const uint32_t* wd = (const uint32_t*)blk;
    const uint32_t* sb = (const uint32_t*)(blk + (bits == 4 ? kCodes4 : kCodes8));
    const int nwords = bits == 4 ? 512 : 1024;
    for (int q = threadIdx.x; q < nwords; q += 256) {
        const int j = q >> 8, lane = (q >> 2) & 63, i = q & 3, a = 4 * j + i;
        int r, c0, n;
        if (bits == 4) {
            r = 16 * (a >> 1) + (lane & 15);
            c0 = 32 * (a & 1) + 8 * (lane >> 4);
            n = 8;
        } else {
            r = 16 * (a >> 2) + (lane & 15);
            c0 = 16 * (a & 3) + 4 * (lane >> 4);
            n = 4;
        }
        const int64_t row = (int64_t)tile * 64 + r;
        if (row >= rows) continue;
        const uint32_t w = wd[q];
        const uint32_t pr = sb[(r & 15) * 4 + (r >> 4)];
        const float s = bf16_lo(pr), b = bf16_hi(pr);
        for (int e = 0; e < n; ++e) {
            const uint32_t code = bits == 4 ? (w >> (4 * (e >> 1) + 16 * (e & 1))) & 0xFu : (w >> (8 * e)) & 0xFFu;
            const int64_t o = row * cols + 64 * g + c0 + e;
            if (codes_out) codes_out[o] = (uint8_t)code;
            if (w_out) w_out[o] = fmaf(s, (float)code, b);
        }
    }
}

}  // namespace mq
