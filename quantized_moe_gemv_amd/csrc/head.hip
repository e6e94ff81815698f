// Quantized GEMV at any shape, for the tied head at the end of decode
// ("Why the runtime has this shape": embedding and head share quantized
// weights, final logit softcap 30.0; "Decode": after the last layer the
// head returns the argmax token directly in the greedy configuration).
//
// y[t][r] = sum_c (s q + b)[r][c] x[t][c], then cap * tanh(y / cap) when a
// cap is given, and the argmax over r per token (equal values to the lower
// row, NaN ranks last).  Each wave owns one 64-row tile and streams its
// blocks group by group, kHeadDepth groups in flight; the weights of a group
// are used for every token of the call, so T tokens cost one pass over W.
// Each workgroup (4 tiles) leaves its best (value, row) per token in the
// workspace and k_head_argmax reduces those.
#include <math.h>

#include "../../include/moegemv.h"
#include "device.h"
#include "plan.h"

namespace mq {

constexpr int kHeadDepth = 4;      // groups in flight per wave

// One group's loads of one lane: the block's codes (2 or 4 16-byte pieces)
// and its (scale, bias) pairs for the lane's four rows.
template <int BITS>
struct HeadLoad {
    uint4 c[BITS == 4 ? 2 : 4];
    uint4 sb;
};

template <int BITS>
__device__ __forceinline__ void head_load(HeadLoad<BITS>& L, const uint8_t* blk, int lane) {
    constexpr int nc = BITS == 4 ? 2 : 4;
#pragma unroll
    for (int j = 0; j < nc; ++j) L.c[j] = ld_stream16(blk + (j * 64 + lane) * 16);
    L.sb = ld_stream16(blk + code_bytes(BITS) + (lane & 15) * 16);
}

// Order key of a value (NaN lowest) with ties to the lower row: larger is better.
__device__ __forceinline__ uint64_t head_key(float v, int row) {
    if (!(v == v)) v = -INFINITY;
    if (v == 0.f) v = 0.f;
    uint32_t u = __float_as_uint(v);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)u << 32) | (uint32_t)(0x7FFFFFFF - row);
}

template <int BITS>
__global__ __launch_bounds__(256) void k_head(HeadArgs a) {
    // dynamic LDS: the token rows [T][cols] (bf16), then per token, group and
    // lane set the sum of the lane's columns [T][G][4] (fp32)
    extern __shared__ uint16_t xs_lds[];
    __shared__ uint64_t best[4][kHeadTokens];
    const int wave = wave_id(), lane = threadIdx.x & 63, kb = lane >> 4;
    const int G = a.cols / 64;
    float* xsum = (float*)(xs_lds + a.T * a.cols);
    for (int q = threadIdx.x; q < a.T * a.cols / 8; q += 256) {
        const int t = q / (a.cols / 8), c8 = q % (a.cols / 8);
        *(uint4*)(xs_lds + t * a.cols + 8 * c8) = *(const uint4*)(a.x + t * a.x_stride + 8 * c8);
    }
    __syncthreads();
    for (int q = threadIdx.x; q < a.T * G * 4; q += 256) {
        const int t = q / (G * 4), g = (q >> 2) % G, k4 = q & 3;
        const uint16_t* xr = xs_lds + t * a.cols + 64 * g;
        float v = 0.f;
        if (BITS == 4) {
            for (int e = 0; e < 8; ++e) v += bf16_to_f32(xr[8 * k4 + e]) + bf16_to_f32(xr[32 + 8 * k4 + e]);
        } else {
            for (int i = 0; i < 4; ++i)
                for (int e = 0; e < 4; ++e) v += bf16_to_f32(xr[16 * i + 4 * k4 + e]);
        }
        xsum[(t * G + g) * 4 + k4] = v;
    }
    __syncthreads();

    const int tile = blockIdx.x * 4 + wave;
    const int ntiles = (a.rows + 63) / 64;
    const bool live = tile < ntiles;
    const uint8_t* base = a.w + (int64_t)(live ? tile : 0) * G * blk_bytes(BITS);
    float acc[kHeadTokens][4];
#pragma unroll
    for (int t = 0; t < kHeadTokens; ++t)
#pragma unroll
        for (int m = 0; m < 4; ++m) acc[t][m] = 0.f;
    HeadLoad<BITS> buf[kHeadDepth];
#pragma unroll
    for (int d = 0; d < kHeadDepth; ++d) head_load<BITS>(buf[d], base + (int64_t)min(d, G - 1) * blk_bytes(BITS), lane);
    for (int g0 = 0; g0 < G; g0 += kHeadDepth) {
#pragma unroll
        for (int d = 0; d < kHeadDepth; ++d) {
            const int g = g0 + d;
            const HeadLoad<BITS> L = buf[d];
            // refill: group g + depth (clamped: an unused load stays in bounds)
            head_load<BITS>(buf[d], base + (int64_t)min(g + kHeadDepth, G - 1) * blk_bytes(BITS), lane);
            if (g < G) {
                const uint32_t sbw[4] = {L.sb.x, L.sb.y, L.sb.z, L.sb.w};
#pragma unroll
                for (int t = 0; t < kHeadTokens; ++t) {
                    if (t < a.T) {
                        const uint16_t* xr = xs_lds + t * a.cols + 64 * g;
                        const float xsv = xsum[(t * G + g) * 4 + kb];
                        float d4[4] = {0.f, 0.f, 0.f, 0.f};
                        if (BITS == 4) {
                            const uint4 xa = *(const uint4*)(xr + 8 * kb), xb = *(const uint4*)(xr + 32 + 8 * kb);
                            q4_block_dot(L.c[0], L.c[1], xa, xb, d4);
#pragma unroll
                            for (int m = 0; m < 4; ++m)
                                acc[t][m] += fmaf(bf16_lo(sbw[m]), fmaf(-128.f, xsv, d4[m]), bf16_hi(sbw[m]) * xsv);
                        } else {
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const uint2 xv = *(const uint2*)(xr + 16 * i + 4 * kb);
                                const float x4[4] = {bf16_lo(xv.x), bf16_hi(xv.x), bf16_lo(xv.y), bf16_hi(xv.y)};
#pragma unroll
                                for (int j = 0; j < 4; ++j) {
                                    const uint32_t cw = (&L.c[j].x)[i];
                                    d4[j] = fmaf((float)(cw & 0xFFu), x4[0], d4[j]);
                                    d4[j] = fmaf((float)((cw >> 8) & 0xFFu), x4[1], d4[j]);
                                    d4[j] = fmaf((float)((cw >> 16) & 0xFFu), x4[2], d4[j]);
                                    d4[j] = fmaf((float)(cw >> 24), x4[3], d4[j]);
                                }
                            }
#pragma unroll
                            for (int m = 0; m < 4; ++m)
                                acc[t][m] += fmaf(bf16_lo(sbw[m]), d4[m], bf16_hi(sbw[m]) * xsv);
                        }
                    }
                }
            }
        }
    }
    // rows 16 m + lane % 16 of the tile; the four lane sets hold parts of each
#pragma unroll
    for (int t = 0; t < kHeadTokens; ++t) {
        if (t >= a.T) break;
        uint64_t key = 0;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            float v = sum_kb(acc[t][m]);
            const int row = tile * 64 + 16 * m + (lane & 15);
            if (a.cap > 0.f) v = a.cap * tanhf(v / a.cap);
            if (live && row < a.rows) {
                if (kb == 0 && a.y) {
                    const int64_t o = (int64_t)t * a.y_stride + row;
                    if (a.y_f32)
                        ((float*)a.y)[o] = v;
                    else
                        ((uint16_t*)a.y)[o] = f32_to_bf16(v);
                }
                const uint64_t k2 = head_key(v, row);
                key = k2 > key ? k2 : key;
            }
        }
        if (a.part) {
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) {
                const uint64_t other = __shfl_xor(key, o, 64);
                key = other > key ? other : key;
            }
            if (lane == 0) best[wave][t] = key;
        }
    }
    if (a.part) {
        __syncthreads();
        if (threadIdx.x < a.T) {
            const int t = threadIdx.x;
            uint64_t k = best[0][t];
#pragma unroll
            for (int w = 1; w < 4; ++w) k = best[w][t] > k ? best[w][t] : k;
            uint32_t u = (uint32_t)(k >> 32);
            u = (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u;   // back to the float bits
            const int row = k == 0 ? -1 : 0x7FFFFFFF - (int)(uint32_t)k;
            a.part[(int64_t)t * gridDim.x + blockIdx.x] = make_float2(__uint_as_float(u), __int_as_float(row));
        }
    }
}

// The argmax over the workgroups' partials: one workgroup per token.
__global__ __launch_bounds__(256) void k_head_argmax(const float2* part, int nparts, int32_t* argmax) {
    const int t = blockIdx.x;
    uint64_t key = 0;
    for (int i = threadIdx.x; i < nparts; i += 256) {
        const float2 v = part[(int64_t)t * nparts + i];
        const int row = __float_as_int(v.y);
        if (row >= 0) {
            const uint64_t k2 = head_key(v.x, row);
            key = k2 > key ? k2 : key;
        }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const uint64_t other = __shfl_xor(key, o, 64);
        key = other > key ? other : key;
    }
    __shared__ uint64_t w4[4];
    if ((threadIdx.x & 63) == 0) w4[threadIdx.x >> 6] = key;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint64_t k = w4[0];
        for (int w = 1; w < 4; ++w) k = w4[w] > k ? w4[w] : k;
        argmax[t] = k == 0 ? -1 : 0x7FFFFFFF - (int)(uint32_t)k;
    }
}

int head_groups(int rows) { return (rows + 255) / 256; }

mq_status launch_head(const HeadArgs& a, int32_t* argmax, hipStream_t s) {
    const int nwg = head_groups(a.rows);
    const size_t lds = head_lds_bytes(a.T, a.cols);
    if (a.bits == 4)
        hipLaunchKernelGGL(k_head<4>, dim3(nwg), dim3(256), lds, s, a);
    else
        hipLaunchKernelGGL(k_head<8>, dim3(nwg), dim3(256), lds, s, a);
    if (argmax) hipLaunchKernelGGL(k_head_argmax, dim3(a.T), dim3(256), 0, s, a.part, nwg, argmax);
    return hipGetLastError() == hipSuccess ? MQ_OK : MQ_ERR_HIP;
}

}  // namespace mq
