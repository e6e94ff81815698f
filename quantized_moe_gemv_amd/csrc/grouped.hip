// Grouped path (many tokens per call): token -> expert permutation, grouped
// dequant-GEMMs on the matrix cores, and the combine.
//
// The weight operand of each MFMA is dequantised in registers from one
// DEV_V1 word per lane: the word holds the eight 4-bit codes of one row and
// eight consecutive columns, which is exactly the A fragment of
// v_mfma_f32_16x16x32_f16 for lane (row % 16, column block lane / 16).
// Codes become fp16 through the exponent trick (0x6400 | q = 1024 + q),
// then w = s * q + b in fp16 (bounded FP16 staging of dequantised weights,
// as the staged-affine prefill of the pages does), and accumulation is fp32.
#include "device.h"
#include "plan.h"

#include "../../include/moegemv.h"

namespace mq {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));

// Prefix sum of v[0 .. n) (n <= 1024) in LDS, one value per thread: the
// thread's exclusive prefix in *excl_out, the total as the return value.
// Every thread of the block must call it.
__device__ __forceinline__ int block_scan_total(int* buf, int n, int v, int* excl_out) {
    const int t = threadIdx.x;
    buf[t] = t < n ? v : 0;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {
        const int add = t >= d ? buf[t - d] : 0;
        __syncthreads();
        buf[t] += add;
        __syncthreads();
    }
    const int total = buf[1023];
    *excl_out = buf[t] - (t < n ? v : 0);
    __syncthreads();
    return total;
}

// Stable counting sort of the (token, slot) pairs by expert, one workgroup.
// The selected experts of one token are distinct, so the rank of pair
// (t, j) among the pairs of expert e is the number of tokens before t that
// chose e: a popcount over a per-expert token bitmap.  Expert offsets and
// the tile schedule (expert << 16 | tile) come from block-wide prefix sums.
__global__ __launch_bounds__(1024) void k_permute(Plan p) {
    __shared__ int scan[1024];
    __shared__ int offs[kMaxExperts + 1];
    uint32_t* bitmap = p.bitmap;
    int32_t* wpre = p.wpre;
    const int T = p.T, k = p.k, E = p.E, W = (T + 31) / 32;
    const int P = T * k;
    for (int q = threadIdx.x; q < E * W; q += 1024) bitmap[q] = 0u;
    __syncthreads();
    for (int q = threadIdx.x; q < P; q += 1024) {
        const int t = q / k, e = p.ids[q];
        atomicOr(&bitmap[e * W + (t >> 5)], 1u << (t & 31));
    }
    __syncthreads();
    int cnt = 0;
    if (threadIdx.x < E) {
        const int e = threadIdx.x;
        for (int w = 0; w < W; ++w) {
            wpre[e * W + w] = cnt;
            cnt += __popc(bitmap[e * W + w]);
        }
        p.counts[e] = cnt;
    }
    int off;
    block_scan_total(scan, E, cnt, &off);   // E <= kMaxExperts <= 1024
    if (threadIdx.x < E) {
        offs[threadIdx.x] = off;
        p.offsets[threadIdx.x] = off;
    }
    if (threadIdx.x == 0) {
        offs[E] = P;
        p.offsets[E] = P;
    }
    const int ntiles = threadIdx.x < E ? (cnt + p.ntile - 1) / p.ntile : 0;
    int toff;
    const int nsched = block_scan_total(scan, E, ntiles, &toff);
    if (threadIdx.x < E)
        for (int tile = 0; tile < ntiles; ++tile) p.sched[toff + tile] = (threadIdx.x << 16) | tile;
    if (threadIdx.x == 0) *p.nsched = nsched;
    for (int q = threadIdx.x; q < P; q += 1024) {
        const int t = q / k, e = p.ids[q];
        const uint32_t word = bitmap[e * W + (t >> 5)];
        const int rank = wpre[e * W + (t >> 5)] + __popc(word & ((1u << (t & 31)) - 1u));
        const int pos = offs[e] + rank;
        p.perm[pos] = q;
        p.inv[q] = pos;
    }
}

// Eight fp16 weights s*q + b from one DEV_V1 4-bit word (column order 0..7).
__device__ __forceinline__ half8_t dequant8(uint32_t w, half2_t s2, half2_t b2) {
    half8_t r;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const uint32_t v = ((w >> (4 * m)) & 0x000F000Fu) | 0x64006400u;  // 1024 + q, two lanes
        half2_t q = __builtin_bit_cast(half2_t, v) - (half2_t){(_Float16)1024.0f, (_Float16)1024.0f};
        half2_t d = q * s2 + b2;
        r[2 * m] = d[0];
        r[2 * m + 1] = d[1];
    }
    return r;
}

__device__ __forceinline__ void sb_half2(uint32_t pr, half2_t* s2, half2_t* b2) {
    const _Float16 s = (_Float16)bf16_lo(pr), b = (_Float16)bf16_hi(pr);
    *s2 = (half2_t){s, s};
    *b2 = (half2_t){b, b};
}

// One 16-row slice (wave ms) x 16 tokens of W . X^T over K = 64 * G
// columns, for NM matrices at once (gate and up share the token operand).
// The column-group loop is software-pipelined: the loads of the next kBatch
// groups are in flight while the current kBatch groups are dequantised and
// multiplied, so a wave keeps up to 2 kBatch groups of loads outstanding
// instead of waiting for each group's loads in turn.
// xrow: this lane's token row (fp16, K long); lanes past the tile's tokens
// read a valid row too and their results are not stored, so every load is
// unconditional.
constexpr int kBatch = 4;

template <int NM>
struct TileLoads {
    uint2 c[NM][kBatch];
    uint32_t s[NM][kBatch];
    half8_t x0[kBatch], x1[kBatch];
};

template <int NM>
__device__ __forceinline__ void tile_load(TileLoads<NM>& L, const uint8_t* const* wbase, const uint8_t* const* sbase,
                                          const _Float16* xrow, int kb, int g0, int G) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
        const int g = g0 + u;
        if (g < G) {
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                L.c[m][u] = *(const uint2*)(wbase[m] + (int64_t)g * kBlk4);
                L.s[m][u] = *(const uint32_t*)(sbase[m] + (int64_t)g * kBlk4);
            }
            L.x0[u] = *(const half8_t*)(xrow + 64 * g + 8 * kb);
            L.x1[u] = *(const half8_t*)(xrow + 64 * g + 32 + 8 * kb);
        }
    }
}

template <int NM>
__device__ __forceinline__ void tile_mma(const TileLoads<NM>& L, float4_t* acc, int g0, int G) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
        if (g0 + u < G) {
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                half2_t s2, b2;
                sb_half2(L.s[m][u], &s2, &b2);
                acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(dequant8(L.c[m][u].x, s2, b2), L.x0[u], acc[m], 0, 0, 0);
                acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(dequant8(L.c[m][u].y, s2, b2), L.x1[u], acc[m], 0, 0, 0);
            }
        }
    }
}

template <int NM>
__device__ __forceinline__ void mma_tiles(const uint8_t* const* tiles, int G, int ms, int lane, const _Float16* xrow,
                                          float4_t* acc) {
    const int kb = lane >> 4;
    const uint8_t* wbase[NM];
    const uint8_t* sbase[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        wbase[m] = tiles[m] + ((ms >> 1) * 64 + lane) * 16 + 8 * (ms & 1);
        sbase[m] = tiles[m] + kCodes4 + (lane & 15) * 16 + 4 * ms;
    }
    TileLoads<NM> A, B;
    tile_load(A, wbase, sbase, xrow, kb, 0, G);
    for (int g0 = 0; g0 < G; g0 += 2 * kBatch) {
        tile_load(B, wbase, sbase, xrow, kb, g0 + kBatch, G);
        tile_mma(A, acc, g0, G);
        tile_load(A, wbase, sbase, xrow, kb, g0 + 2 * kBatch, G);
        tile_mma(B, acc, g0 + kBatch, G);
    }
}

// Gate/up + GeGLU for one (expert, token tile) or, with shared = 1, for the
// shared expert over a tile of all tokens.  grid (I/64, tiles), block 256.
__global__ __launch_bounds__(256) void k_gg_gateup(Plan p, int shared) {
    const int rt = blockIdx.x, wave = wave_id(), lane = threadIdx.x & 63;
    const int n = lane & 15;
    int count, first;   // tokens of this tile, position of its first pair
    const uint8_t *gw, *uw;
    int rows;
    if (shared) {
        first = blockIdx.y * p.ntile;
        count = min(p.ntile, p.T - first);
        gw = p.sh_gate + (int64_t)rt * p.G_H * kBlk4;
        uw = p.sh_up + (int64_t)rt * p.G_H * kBlk4;
        rows = p.Is;
    } else {
        if ((int)blockIdx.y >= *p.nsched) return;
        const int sc = p.sched[blockIdx.y], e = sc >> 16, tile = sc & 0xFFFF;
        first = p.offsets[e] + tile * p.ntile;
        count = min(p.ntile, p.offsets[e + 1] - first);
        const uint8_t* blob = p.pool_base + (int64_t)e * p.expert_stride;
        gw = blob + p.gate_off + (int64_t)rt * p.G_H * kBlk4;
        uw = blob + p.up_off + (int64_t)rt * p.G_H * kBlk4;
        rows = p.I;
    }
    // lanes past the tile's tokens use the tile's first token (not stored)
    const int nn = n < count ? n : 0;
    const int tok = shared ? first + nn : p.perm[first + nn] / p.k;
    const _Float16* xrow = p.x16 + (int64_t)tok * p.H;
    float4_t acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    const uint8_t* tiles[2] = {gw, uw};
    mma_tiles<2>(tiles, p.G_H, wave, lane, xrow, acc);
    const float4_t ag = acc[0], au = acc[1];
    if (n < count) {
        _Float16* dst = shared ? p.hs16 + (int64_t)(first + n) * p.Is : p.hg + (int64_t)(first + n) * p.I;
        const int r0 = rt * 64 + 16 * wave + 4 * (lane >> 4);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (r0 + i < rows) dst[r0 + i] = (_Float16)(gelu_tanh(ag[i]) * au[i]);
    }
}

// Down projection for one (expert, token tile): ysort[pos] = w_pair * (W_down . h),
// or with shared = 1 the shared expert: ysh[t] = W_sdown . hs.  grid (H/64, tiles).
__global__ __launch_bounds__(256) void k_gg_down(Plan p, int shared) {
    const int rt = blockIdx.x, wave = wave_id(), lane = threadIdx.x & 63;
    const int n = lane & 15;
    int count, first, G, K;
    const uint8_t* dw;
    const _Float16* hbase;
    if (shared) {
        first = blockIdx.y * p.ntile;
        count = min(p.ntile, p.T - first);
        dw = p.sh_down + (int64_t)rt * p.G_s * kBlk4;
        hbase = p.hs16;
        G = p.G_s;
        K = p.Is;
    } else {
        if ((int)blockIdx.y >= *p.nsched) return;
        const int sc = p.sched[blockIdx.y], e = sc >> 16, tile = sc & 0xFFFF;
        first = p.offsets[e] + tile * p.ntile;
        count = min(p.ntile, p.offsets[e + 1] - first);
        dw = p.pool_base + (int64_t)e * p.expert_stride + p.down_off + (int64_t)rt * p.G_I * kBlk4;
        hbase = p.hg;
        G = p.G_I;
        K = p.I;
    }
    const _Float16* hrow = hbase + (int64_t)(first + (n < count ? n : 0)) * K;   // padding lanes: not stored
    float4_t accv[1] = {{0.f, 0.f, 0.f, 0.f}};
    const uint8_t* tiles[1] = {dw};
    mma_tiles<1>(tiles, G, wave, lane, hrow, accv);
    const float4_t acc = accv[0];
    if (n < count) {
        const int r0 = rt * 64 + 16 * wave + 4 * (lane >> 4);
        if (shared) {
            float* dst = p.ysh + (int64_t)(first + n) * p.H;
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[r0 + i] = acc[i];
        } else {
            const float w = p.wts[p.perm[first + n]];
            float* dst = p.ysort + (int64_t)(first + n) * p.H;
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[r0 + i] = w * acc[i];
        }
    }
}

// out[t] = shared + sum_j ysort[inv[t][j]] (slot order), rounded once.  grid (T, ceil(H/256)).
__global__ __launch_bounds__(256) void k_gg_combine(Plan p) {
    const int t = blockIdx.x, i = blockIdx.y * 256 + threadIdx.x;
    if (i >= p.H) return;
    float v = p.has_shared ? p.ysh[(int64_t)t * p.H + i] : 0.f;
    for (int j = 0; j < p.k; ++j) v += p.ysort[(int64_t)p.inv[t * p.k + j] * p.H + i];
    if (p.out_f32)
        ((float*)p.out)[(int64_t)t * p.out_stride + i] = v;
    else
        ((uint16_t*)p.out)[(int64_t)t * p.out_stride + i] = f32_to_bf16(v);
}

mq_status launch_grouped(const Plan& p, hipStream_t s) {
    hipLaunchKernelGGL(k_permute, dim3(1), dim3(1024), 0, s, p);
    const int tshared = (p.T + p.ntile - 1) / p.ntile;
    hipLaunchKernelGGL(k_gg_gateup, dim3(p.I / 64, p.max_tiles), dim3(256), 0, s, p, 0);
    if (p.has_shared) hipLaunchKernelGGL(k_gg_gateup, dim3(p.Is / 64, tshared), dim3(256), 0, s, p, 1);
    hipLaunchKernelGGL(k_gg_down, dim3(p.H / 64, p.max_tiles), dim3(256), 0, s, p, 0);
    if (p.has_shared) hipLaunchKernelGGL(k_gg_down, dim3(p.H / 64, tshared), dim3(256), 0, s, p, 1);
    hipLaunchKernelGGL(k_gg_combine, dim3(p.T, (p.H + 255) / 256), dim3(256), 0, s, p);
    return MQ_OK;
}

}  // namespace mq
