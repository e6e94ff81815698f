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
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

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
// the schedule (expert << 16 | chunk) come from block-wide prefix sums.
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
    // then the chunks of the shared expert's virtual experts E .. E+n_vs-1
    const int nch = (T + p.ntile - 1) / p.ntile;
    for (int q = threadIdx.x; q < p.n_vs * nch; q += 1024) p.sched[nsched + q] = ((E + q / nch) << 16) | (q % nch);
    if (threadIdx.x == 0) *p.nsched = nsched + p.n_vs * nch;
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

// Grouped dequant-GEMM.  A work item is (64-row tile of one matrix, chunk
// of up to p.ntile tokens of one expert).  The shared expert takes part as
// n_sc virtual experts of I rows each (its gate/up rows, and the matching
// column slices of its down projection), applied to every token with
// weight 1, so it fills the machine together with the routed work.
//
// Wave ms owns rows 16 ms .. 16 ms + 15 of the tile.  The token operand (x
// for gate/up, h for down) is staged in LDS kKB column groups at a time for
// every token of the chunk; each dequantised weight fragment then feeds the
// MFMAs of all the chunk's 16-token tiles.  The weights and the token rows
// of the next batch are loaded into registers while the current batch is
// multiplied.
constexpr int kKB = 4;                    // most column groups per staged batch
constexpr int kXPitch = kKB * 64 + 8;     // LDS row pitch in halves (rows fall on different banks)

template <int NM, int KB>
struct WLoads {
    uint2 c[NM][KB];
    uint32_t s[NM][KB];
};

// Weight words of column groups g0 .. g0+KB-1.  A group past the end is
// read from group G-1 with its scale and bias forced to zero, so its
// dequantised fragment is exactly zero; no load is predicated.
template <int NM, int KB>
__device__ __forceinline__ void w_load(WLoads<NM, KB>& L, const uint8_t* const* wbase, const uint8_t* const* sbase,
                                       int g0, int G) {
#pragma unroll
    for (int u = 0; u < KB; ++u) {
        const int g = min(g0 + u, G - 1);
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            L.c[m][u] = *(const uint2*)(wbase[m] + (int64_t)g * kBlk4);
            const uint32_t sv = *(const uint32_t*)(sbase[m] + (int64_t)g * kBlk4);
            L.s[m][u] = g0 + u < G ? sv : 0u;
        }
    }
}

// Token-operand pieces (16 bytes) of one batch held by this thread: piece i
// is row tid / (8 KB) + (32 / KB) i, columns (tid % (8 KB)) * 8 .. + 7 of the
// batch.  Rows past the chunk repeat its last row and groups past the end
// repeat group G-1 (their weights are zero), so every load is in bounds and
// unmasked.
template <int NTT, int KB>
struct XLoads {
    u32x4_t v[NTT * KB / 2];
};

template <int NTT, int KB>
__device__ __forceinline__ void x_load(XLoads<NTT, KB>& X, const _Float16* src, int64_t stride, const int* rows,
                                       int count, int g0, int G) {
    const int q = threadIdx.x % (8 * KB), g = min(g0 + (q >> 3), G - 1);
    const int col = g * 64 + (q & 7) * 8;
#pragma unroll
    for (int i = 0; i < NTT * KB / 2; ++i) {
        const int n = min((int)threadIdx.x / (8 * KB) + (32 / KB) * i, count - 1);
        X.v[i] = *(const u32x4_t*)(src + (int64_t)rows[n] * stride + col);
    }
}

template <int NTT, int KB>
__device__ __forceinline__ void x_store(const XLoads<NTT, KB>& X, _Float16 (*xs)[kXPitch]) {
    const int q = threadIdx.x % (8 * KB);
#pragma unroll
    for (int i = 0; i < NTT * KB / 2; ++i)
        *(u32x4_t*)&xs[threadIdx.x / (8 * KB) + (32 / KB) * i][q * 8] = X.v[i];
}

template <int NM, int NTT, int MAXT, int KB>
__device__ __forceinline__ void w_mma(const WLoads<NM, KB>& L, _Float16 (*xs)[kXPitch], float4_t (*acc)[MAXT],
                                      int lane) {
    const int kb = lane >> 4, n = lane & 15;
#pragma unroll
    for (int u = 0; u < KB; ++u) {
        half8_t a0[NM], a1[NM];
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            half2_t s2, b2;
            sb_half2(L.s[m][u], &s2, &b2);
            a0[m] = dequant8(L.c[m][u].x, s2, b2);
            a1[m] = dequant8(L.c[m][u].y, s2, b2);
        }
#pragma unroll
        for (int t = 0; t < NTT; ++t) {
            const half8_t b0 = *(const half8_t*)&xs[16 * t + n][64 * u + 8 * kb];
            const half8_t b1 = *(const half8_t*)&xs[16 * t + n][64 * u + 32 + 8 * kb];
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                acc[m][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0[m], b0, acc[m][t], 0, 0, 0);
                acc[m][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1[m], b1, acc[m][t], 0, 0, 0);
            }
        }
    }
}

// One work item over all G column groups: acc[m][t] holds rows
// 16 ms + 4 (lane / 16) + i, token 16 t + lane % 16 of matrix m.
template <int NM, int NTT, int MAXT>
__device__ __forceinline__ void gg_tile_n(const uint8_t* const* tiles, int G, const _Float16* src, int64_t stride,
                                          const int* rows, int count, _Float16 (*xs)[kXPitch],
                                          float4_t (*acc)[MAXT]) {
    constexpr int KB = NTT <= 4 ? kKB : kKB / 2;   // keeps the prefetched rows within the register budget
    const int ms = wave_id(), lane = threadIdx.x & 63;
    const uint8_t* wbase[NM];
    const uint8_t* sbase[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        wbase[m] = tiles[m] + ((ms >> 1) * 64 + lane) * 16 + 8 * (ms & 1);
        sbase[m] = tiles[m] + kCodes4 + (lane & 15) * 16 + 4 * ms;
    }
    WLoads<NM, KB> A, B;
    XLoads<NTT, KB> X;
    x_load(X, src, stride, rows, count, 0, G);
    w_load(A, wbase, sbase, 0, G);
    // The loads for the batch after the last one re-read (clamped) groups
    // just read, which keeps every load unconditional.
    for (int g0 = 0;; g0 += 2 * KB) {
        x_store(X, xs);
        __syncthreads();
        x_load(X, src, stride, rows, count, g0 + KB, G);
        w_load(B, wbase, sbase, g0 + KB, G);
        w_mma<NM, NTT, MAXT, KB>(A, xs, acc, lane);
        __syncthreads();
        if (g0 + KB >= G) break;
        x_store(X, xs);
        __syncthreads();
        x_load(X, src, stride, rows, count, g0 + 2 * KB, G);
        w_load(A, wbase, sbase, g0 + 2 * KB, G);
        w_mma<NM, NTT, MAXT, KB>(B, xs, acc, lane);
        __syncthreads();
        if (g0 + 2 * KB >= G) break;
    }
}

// Dispatch on the chunk's number of 16-token tiles so that every MFMA
// sequence is straight-line code.
template <int NM, int MAXT>
__device__ __forceinline__ void gg_tile(const uint8_t* const* tiles, int G, const _Float16* src, int64_t stride,
                                        const int* rows, int count, _Float16 (*xs)[kXPitch], float4_t (*acc)[MAXT]) {
    const int ntt = (count + 15) / 16;
    if constexpr (MAXT <= 2) {
        if (ntt == 1) gg_tile_n<NM, 1, MAXT>(tiles, G, src, stride, rows, count, xs, acc);
        else gg_tile_n<NM, MAXT, MAXT>(tiles, G, src, stride, rows, count, xs, acc);
    } else {
        switch (ntt) {
            case 1: gg_tile_n<NM, 1, MAXT>(tiles, G, src, stride, rows, count, xs, acc); break;
            case 2: gg_tile_n<NM, 2, MAXT>(tiles, G, src, stride, rows, count, xs, acc); break;
            case 3: gg_tile_n<NM, 3, MAXT>(tiles, G, src, stride, rows, count, xs, acc); break;
            case 4: gg_tile_n<NM, 4, MAXT>(tiles, G, src, stride, rows, count, xs, acc); break;
            case 5: gg_tile_n<NM, 5, MAXT>(tiles, G, src, stride, rows, count, xs, acc); break;
            case 6: gg_tile_n<NM, 6, MAXT>(tiles, G, src, stride, rows, count, xs, acc); break;
            case 7: gg_tile_n<NM, 7, MAXT>(tiles, G, src, stride, rows, count, xs, acc); break;
            default: gg_tile_n<NM, MAXT, MAXT>(tiles, G, src, stride, rows, count, xs, acc); break;
        }
    }
}

// The work item of this workgroup: blockIdx.y indexes the schedule
// (expert << 16 | chunk), blockIdx.x the 64-row tile.  Experts E .. E+n_vs-1
// are the shared expert's virtual experts.  Returns false when the
// workgroup has nothing to do.
struct Item {
    int count;          // tokens of the chunk
    int pos0;           // row of chunk token 0 in hg / ysort
    int shared;         // 1 for a virtual shared expert
    int tok0;           // shared: first token of the chunk
    int G;              // column groups of the operand
    const uint8_t* w[2];
};

__device__ __forceinline__ bool gg_item(const Plan& p, bool down, Item* it) {
    if ((int)blockIdx.y >= *p.nsched) return false;
    const int sc = p.sched[blockIdx.y], ex = sc >> 16, c = sc & 0xFFFF, rt = blockIdx.x;
    if (ex < p.E) {
        const int first = p.offsets[ex] + c * p.ntile;
        it->count = min(p.ntile, p.offsets[ex + 1] - first);
        it->pos0 = first;
        it->shared = 0;
        it->tok0 = 0;
        const uint8_t* base = p.pool_base + (int64_t)ex * p.expert_stride;
        if (down) {
            it->G = p.G_I;
            it->w[0] = it->w[1] = base + p.down_off + (int64_t)rt * p.G_I * kBlk4;
        } else {
            it->G = p.G_H;
            it->w[0] = base + p.gate_off + (int64_t)rt * p.G_H * kBlk4;
            it->w[1] = base + p.up_off + (int64_t)rt * p.G_H * kBlk4;
        }
    } else {
        const int j = ex - p.E;
        it->tok0 = c * p.ntile;
        it->count = min(p.ntile, p.T - it->tok0);
        it->pos0 = p.T * p.k + j * p.T + it->tok0;
        it->shared = 1;
        if (down) {
            it->G = min(p.G_I, p.G_s - j * p.G_I);
            it->w[0] = it->w[1] = p.sh_down + ((int64_t)rt * p.G_s + (int64_t)j * p.G_I) * kBlk4;
        } else {
            if (rt * 64 >= p.Is - j * p.I) return false;   // the last virtual expert may be shorter
            it->G = p.G_H;
            it->w[0] = p.sh_gate + (int64_t)(j * p.G_I + rt) * p.G_H * kBlk4;
            it->w[1] = p.sh_up + (int64_t)(j * p.G_I + rt) * p.G_H * kBlk4;
        }
    }
    return true;
}

// Gate/up + GeGLU: hg[pos] = gelu(gate x) * (up x) in fp16.
// grid (I / 64, max_tiles), block 256.
template <int MAXT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_gg_gateup(Plan p) {
    __shared__ __attribute__((aligned(16))) _Float16 xs[MAXT * 16][kXPitch];
    __shared__ int rows[MAXT * 16];
    Item it;
    if (!gg_item(p, false, &it)) return;
    const int rt = blockIdx.x, wave = wave_id(), lane = threadIdx.x & 63;
    if ((int)threadIdx.x < it.count)
        rows[threadIdx.x] = it.shared ? it.tok0 + threadIdx.x : p.perm[it.pos0 + threadIdx.x] / p.k;
    __syncthreads();
    float4_t acc[2][MAXT];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int t = 0; t < MAXT; ++t) acc[m][t] = (float4_t){0.f, 0.f, 0.f, 0.f};
    gg_tile<2, MAXT>(it.w, it.G, p.x16, p.H, rows, it.count, xs, acc);
    const int r0 = rt * 64 + 16 * wave + 4 * (lane >> 4);
#pragma unroll
    for (int t = 0; t < MAXT; ++t) {
        const int n = 16 * t + (lane & 15);
        if (n < it.count) {
            _Float16* dst = p.hg + (int64_t)(it.pos0 + n) * p.I + r0;
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[i] = (_Float16)(gelu_tanh(acc[0][t][i]) * acc[1][t][i]);
        }
    }
}

// Down projection: ysort[pos] = w_pair * (W_down . h), weight 1 for the
// shared expert's slices.  grid (H / 64, max_tiles), block 256.
template <int MAXT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_gg_down(Plan p) {
    __shared__ __attribute__((aligned(16))) _Float16 xs[MAXT * 16][kXPitch];
    __shared__ int rows[MAXT * 16];
    __shared__ float wrow[MAXT * 16];
    Item it;
    if (!gg_item(p, true, &it)) return;
    const int rt = blockIdx.x, wave = wave_id(), lane = threadIdx.x & 63;
    if ((int)threadIdx.x < it.count) {
        rows[threadIdx.x] = it.pos0 + threadIdx.x;
        wrow[threadIdx.x] = it.shared ? 1.f : p.wts[p.perm[it.pos0 + threadIdx.x]];
    }
    __syncthreads();
    float4_t acc[1][MAXT];
#pragma unroll
    for (int t = 0; t < MAXT; ++t) acc[0][t] = (float4_t){0.f, 0.f, 0.f, 0.f};
    gg_tile<1, MAXT>(it.w, it.G, p.hg, p.I, rows, it.count, xs, acc);
    const int r0 = rt * 64 + 16 * wave + 4 * (lane >> 4);
#pragma unroll
    for (int t = 0; t < MAXT; ++t) {
        const int n = 16 * t + (lane & 15);
        if (n < it.count) {
            const float w = wrow[n];
            float* dst = p.ysort + (int64_t)(it.pos0 + n) * p.H + r0;
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[i] = w * acc[0][t][i];
        }
    }
}

// out[t] = sum_j ysort[inv[t][j]] (slot order) + the shared expert's
// slices, rounded once.  grid (T, ceil(H/256)).
__global__ __launch_bounds__(256) void k_gg_combine(Plan p) {
    const int t = blockIdx.x, i = blockIdx.y * 256 + threadIdx.x;
    if (i >= p.H) return;
    float v = 0.f;
    for (int j = 0; j < p.k; ++j) v += p.ysort[(int64_t)p.inv[t * p.k + j] * p.H + i];
    for (int j = 0; j < p.n_vs; ++j) v += p.ysort[((int64_t)p.T * p.k + (int64_t)j * p.T + t) * p.H + i];
    if (p.out_f32)
        ((float*)p.out)[(int64_t)t * p.out_stride + i] = v;
    else
        ((uint16_t*)p.out)[(int64_t)t * p.out_stride + i] = f32_to_bf16(v);
}

mq_status launch_grouped(const Plan& p, hipStream_t s) {
    hipLaunchKernelGGL(k_permute, dim3(1), dim3(1024), 0, s, p);
    const dim3 gu(p.I / 64, p.max_tiles), dn(p.H / 64, p.max_tiles);
    if (p.ntile <= 32) {
        hipLaunchKernelGGL(k_gg_gateup<2>, gu, dim3(256), 0, s, p);
        hipLaunchKernelGGL(k_gg_down<2>, dn, dim3(256), 0, s, p);
    } else {
        hipLaunchKernelGGL(k_gg_gateup<8>, gu, dim3(256), 0, s, p);
        hipLaunchKernelGGL(k_gg_down<8>, dn, dim3(256), 0, s, p);
    }
    hipLaunchKernelGGL(k_gg_combine, dim3(p.T, (p.H + 255) / 256), dim3(256), 0, s, p);
    return MQ_OK;
}

}  // namespace mq
