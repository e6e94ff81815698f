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

// Prefix sum of v[0 .. n) (n <= 1024), one value per thread of a 1024-thread
// block: the thread's exclusive prefix in *excl_out, the total as the return
// value.  Shuffle scans within each wave, then the 16 wave totals (buf holds
// 16 ints).  Every thread of the block must call it.
__device__ __forceinline__ int block_scan_total(int* buf, int n, int v, int* excl_out) {
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int x = t < n ? v : 0;
    int inc = x;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(inc, d, 64);
        if (lane >= d) inc += y;
    }
    if (lane == 63) buf[w] = inc;
    __syncthreads();
    int base = 0, total = 0;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int c = buf[q];
        base += q < w ? c : 0;
        total += c;
    }
    __syncthreads();
    *excl_out = base + inc - x;
    return total;
}

// ---------------------------------------------------------------------------
// Front of the grouped path in one launch: router input, router scores,
// top-k and softmax, and the token -> expert permutation with the work
// schedule.  grid (ceil(T / TG)), block 1024.
//
// Each workgroup scores all experts for its TG tokens and ranks them; the
// last workgroup to finish (a counter at a fixed workspace offset, returned
// to zero for the next call) sorts every (token, slot) pair by expert and
// writes the schedule.  Device-scope fences order the stores before the
// counter and the loads after it.
constexpr int kFrontStatic = 16 * 1024;   // bytes of static LDS in k_front (upper bound)

// Schedule entries (unit << 16 | tiles << 8 | chunk), tiles = the chunk's
// 16-token tiles, heaviest chunks first: the full chunks of every unit (the
// experts, then the shared expert's virtual experts E .. E+n_vs-1 over all T
// tokens), then the partial last chunks by decreasing number of tiles.
// Items are independent, so the order within a class does not matter.
// cnt: this thread's expert count (thread u < E); every thread calls it.
__device__ __forceinline__ void build_schedule(const Plan& p, int cnt, int* scan) {
    __shared__ int ccount[17], cfill[17];
    const int T = p.T, E = p.E, nu = E + p.n_vs;   // nu <= kMaxExperts + a few <= 1024
    const int u = threadIdx.x;
    const int ucnt = u < E ? cnt : (u < nu ? T : 0);
    const int nfull = ucnt / p.ntile, rem = ucnt - nfull * p.ntile;
    const int cls = rem > 0 ? (rem + 15) / 16 : 0;   // 1 .. ntile / 16
    int foff;
    const int tfull = block_scan_total(scan, nu, nfull, &foff);
    for (int c = 0; c < nfull; ++c) p.sched[foff + c] = (u << 16) | ((p.ntile / 16) << 8) | c;
    if (threadIdx.x < 17) ccount[threadIdx.x] = cfill[threadIdx.x] = 0;
    __syncthreads();
    if (cls > 0) atomicAdd(&ccount[cls], 1);
    __syncthreads();
    if (cls > 0) {
        int before = 0;   // partial chunks of heavier classes
        for (int q = cls + 1; q <= 16; ++q) before += ccount[q];
        p.sched[tfull + before + atomicAdd(&cfill[cls], 1)] = (u << 16) | (cls << 8) | nfull;
    }
    if (threadIdx.x == 0) {
        int np = 0;
        for (int q = 1; q <= 16; ++q) np += ccount[q];
        *p.nsched = tfull + np;
    }
}

template <int TG>
__global__ __launch_bounds__(1024) void k_front(Plan p) {
    extern __shared__ __attribute__((aligned(16))) float rr[];   // [TG][H] router input
    __shared__ float red[16][TG];
    __shared__ float part[16][TG][16];
    __shared__ float lg[TG][kMaxExperts];
    __shared__ float selv[TG][kMaxTopK];
    __shared__ int seli[TG][kMaxTopK];
    __shared__ int scan[16];
    __shared__ int ecount[kMaxExperts], efill[kMaxExperts], eoff[kMaxExperts];
    __shared__ int last;
    const int H = p.H, E = p.E, tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
    const int t0 = blockIdx.x * TG, nt = min(TG, p.T - t0);

    // router input r = x / sqrt(mean(x^2) + eps) * router_scale / sqrt(H),
    // all TG tokens at once
    {
        float ss[TG];
#pragma unroll
        for (int tt = 0; tt < TG; ++tt) ss[tt] = 0.f;
        for (int i = tid; i < H; i += 1024)
#pragma unroll
            for (int tt = 0; tt < TG; ++tt)
                if (tt < nt) {
                    const float v = bf16_to_f32(p.x[(int64_t)(t0 + tt) * p.x_stride + i]);
                    ss[tt] += v * v;
                }
#pragma unroll
        for (int tt = 0; tt < TG; ++tt) {
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) ss[tt] += __shfl_xor(ss[tt], o, 64);
            if (lane == 0) red[wave][tt] = ss[tt];
        }
        __syncthreads();
        float c[TG];
#pragma unroll
        for (int tt = 0; tt < TG; ++tt) {
            float t = 0.f;
#pragma unroll
            for (int w = 0; w < 16; ++w) t += red[w][tt];
            c[tt] = (1.0f / sqrtf(t / (float)H + p.eps)) * (1.0f / sqrtf((float)H));
        }
        for (int i = tid; i < H; i += 1024) {
            const float rs = p.router_scale ? p.router_scale[i] : 1.0f;
#pragma unroll
            for (int tt = 0; tt < TG; ++tt)
                if (tt < nt) {
                    const float xv = bf16_to_f32(p.x[(int64_t)(t0 + tt) * p.x_stride + i]);
                    rr[tt * H + i] = xv * c[tt] * rs;
                    p.x16[(int64_t)(t0 + tt) * H + i] = (_Float16)xv;
                }
        }
    }
    __syncthreads();

    // scores: slice sl of 16 experts (rows 16 sl .. of the router) per wave
    // set, lane owns expert row 16 sl + lane % 16 and columns
    // 16 i + 4 (lane / 16) + 0..3 of each group; the wps waves of a slice
    // split its groups
    const int nsl = p.E_pad / 16, wps = 16 / nsl;   // E_pad in {64, 128, 192, 256}
    {
        const int sl = wave % nsl, gw = wave / nsl, kb = lane >> 4, j4 = sl & 3;
        float acc[TG];
#pragma unroll
        for (int tt = 0; tt < TG; ++tt) acc[tt] = 0.f;
        if (wave < nsl * wps) {
            const uint8_t* base = p.router_w + (int64_t)(sl >> 2) * p.G_H * kBlk8 + (j4 * 64 + lane) * 16;
            const int sbo = kCodes8 + (lane & 15) * 16 + 4 * j4 - (j4 * 64 + lane) * 16;
            const int ng = (p.G_H - gw + wps - 1) / wps;   // this wave's groups gw + wps j
            // eight groups of loads in flight per batch (the last batch
            // re-reads, clamped, and skips what lies past the end)
            constexpr int kRB = 8;
            for (int j0 = 0; j0 < ng; j0 += kRB) {
                u32x4_t cw[kRB];
                uint32_t sb[kRB];
#pragma unroll
                for (int u = 0; u < kRB; ++u) {
                    const int g = gw + wps * min(j0 + u, ng - 1);
                    cw[u] = *(const u32x4_t*)(base + (int64_t)g * kBlk8);
                    sb[u] = *(const uint32_t*)(base + (int64_t)g * kBlk8 + sbo);
                }
#pragma unroll
                for (int u = 0; u < kRB; ++u) {
                    if (j0 + u >= ng) break;
                    const int g = gw + wps * (j0 + u);
#pragma unroll
                    for (int tt = 0; tt < TG; ++tt) {
                        float d = 0.f, rs = 0.f;
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float4_t rv = *(const float4_t*)&rr[tt * H + 64 * g + 16 * i + 4 * kb];
                            d = fmaf((float)(cw[u][i] & 0xFFu), rv[0], d);
                            d = fmaf((float)((cw[u][i] >> 8) & 0xFFu), rv[1], d);
                            d = fmaf((float)((cw[u][i] >> 16) & 0xFFu), rv[2], d);
                            d = fmaf((float)(cw[u][i] >> 24), rv[3], d);
                            rs += (rv[0] + rv[1]) + (rv[2] + rv[3]);
                        }
                        acc[tt] = fmaf(bf16_lo(sb[u]), d, fmaf(bf16_hi(sb[u]), rs, acc[tt]));
                    }
                }
            }
        }
#pragma unroll
        for (int tt = 0; tt < TG; ++tt) {
            const float v = sum_kb(acc[tt]);
            if (kb == 0) part[wave][tt][lane] = v;
        }
    }
    __syncthreads();
    for (int q = tid; q < TG * E; q += 1024) {
        const int tt = q / E, e = q - tt * E, sl = e >> 4;
        if (tt < nt) {
            float s = 0.f;
            for (int w = 0; w < wps; ++w) s += part[sl + w * nsl][tt][e & 15];
            if (p.logit_bias) s += p.logit_bias[e];
            if (p.logits_out) p.logits_out[(int64_t)(t0 + tt) * E + e] = s;
            lg[tt][e] = (s == s) ? s : -INFINITY;   // a NaN score ranks last; ids stay distinct
        }
    }
    __syncthreads();
    // rank: four threads per expert each count a quarter of the others
    for (int tt = 0; tt < nt; ++tt) {
        const int e = tid >> 2, qq = tid & 3;
        int beat = 0;
        float v = 0.f;
        if (e < E) {
            v = lg[tt][e];
            for (int o = qq; o < E; o += 4) beat += (lg[tt][o] > v) || (lg[tt][o] == v && o < e);
        }
        beat += __shfl_xor(beat, 1, 64);
        beat += __shfl_xor(beat, 2, 64);
        if (e < E && qq == 0 && beat < p.k) {
            selv[tt][beat] = v;
            seli[tt][beat] = e;
        }
    }
    __syncthreads();
    if (tid < nt * p.k) {
        const int tt = tid / p.k, j = tid - tt * p.k, t = t0 + tt;
        float den = 0.f;
        for (int i = 0; i < p.k; ++i) den += expf(selv[tt][i] - selv[tt][0]);
        const int e = seli[tt][j];
        const float w = expf(selv[tt][j] - selv[tt][0]) / den * (p.pes ? p.pes[e] : 1.0f);
        p.ids[t * p.k + j] = e;
        p.wts[t * p.k + j] = w;
        if (p.ids_out) p.ids_out[t * p.k + j] = e;
        if (p.w_out) p.w_out[t * p.k + j] = w;
    }

    // the last workgroup sorts every pair by expert and builds the schedule.
    // One thread fences for the workgroup: the barrier orders the other
    // threads' stores before its release and its acquire before their loads.
    __syncthreads();
    if (tid == 0) {
        __threadfence();
        last = atomicAdd(&p.fcnt[kFrontMaxGroups], 1u) + 1 == gridDim.x;
        if (last) {
            p.fcnt[kFrontMaxGroups] = 0u;
            __threadfence();
        }
    }
    __syncthreads();
    if (!last) return;
    const int P = p.T * p.k;
    for (int e = tid; e < E; e += 1024) ecount[e] = efill[e] = 0;
    __syncthreads();
    for (int q = tid; q < P; q += 1024) atomicAdd(&ecount[p.ids[q]], 1);
    __syncthreads();
    const int cnt = tid < E ? ecount[tid] : 0;
    int off;
    block_scan_total(scan, E, cnt, &off);   // E <= kMaxExperts <= 1024
    if (tid < E) {
        eoff[tid] = off;
        p.offsets[tid] = off;
        p.counts[tid] = cnt;
    }
    if (tid == 0) p.offsets[E] = P;
    __syncthreads();
    // positions within an expert's segment come from LDS atomics; every item
    // computes each token independently, so their order changes no result
    for (int q = tid; q < P; q += 1024) {
        const int e = p.ids[q];
        const int pos = eoff[e] + atomicAdd(&efill[e], 1);
        p.perm[pos] = q;
        p.inv[q] = pos;
    }
    build_schedule(p, cnt, scan);
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
// of up to p.ntile = 128 tokens of one expert); for the down projection a
// workgroup takes kDnTiles consecutive row tiles of the item.  The shared
// expert takes part as n_sc virtual experts of I rows each (its gate/up
// rows, and the matching column slices of its down projection), applied to
// every token with weight 1, so it fills the machine together with the
// routed work.  The schedule puts the heaviest chunks first.
//
// Two ways through an item, by its token count:
//  * up to 32 tokens, the loop is bound by load latency: the four waves
//    split the column groups (gate/up) or own 16 rows each over an operand
//    staged once (down), keep several groups of weights in flight and take
//    no workgroup barrier;
//  * more tokens: the token operand is staged in LDS a batch of column
//    groups at a time for the whole chunk, and each dequantised weight
//    fragment feeds the MFMAs of all the chunk's 16-token tiles (wave ms
//    owns rows 16 ms .. 16 ms + 15 of the tile).
constexpr int kBigKB = 4;                     // most column groups per staged batch (gate/up)
constexpr int kDnKB = 2;                      // column groups per staged batch (down)
constexpr int kDnTiles = 4;                   // 64-row output tiles per down workgroup

template <int KB>
constexpr int pitch_of() { return KB * 64 + 8; }   // LDS row pitch in halves (rows fall on different banks)

template <int NM, int KB>
struct WLoads {
    uint2 c[NM][KB];
    uint32_t s[NM][KB];
};

// Weight words of column groups g0 .. g0+KB-1.  A group past the end is
// read from group G-1 (in bounds, no load is predicated); the multiply
// forces its scale and bias to zero, so its fragment is exactly zero.
template <int NM, int KB>
__device__ __forceinline__ void w_load(WLoads<NM, KB>& L, const uint8_t* const* wbase, const uint8_t* const* sbase,
                                       int g0, int G) {
#pragma unroll
    for (int u = 0; u < KB; ++u) {
        const int g = min(g0 + u, G - 1);
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            L.c[m][u] = *(const uint2*)(wbase[m] + (int64_t)g * kBlk4);
            L.s[m][u] = *(const uint32_t*)(sbase[m] + (int64_t)g * kBlk4);
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

template <int NTT, int KB, int P>
__device__ __forceinline__ void x_store(const XLoads<NTT, KB>& X, _Float16 (*xs)[P]) {
    const int q = threadIdx.x % (8 * KB);
#pragma unroll
    for (int i = 0; i < NTT * KB / 2; ++i)
        *(u32x4_t*)&xs[threadIdx.x / (8 * KB) + (32 / KB) * i][q * 8] = X.v[i];
}

template <int NM, int NTT, int KB, int P>
__device__ __forceinline__ void w_mma(const WLoads<NM, KB>& L, _Float16 (*xs)[P], float4_t (*acc)[8], int lane,
                                      int g0, int G) {
    const int kb = lane >> 4, n = lane & 15;
#pragma unroll
    for (int u = 0; u < KB; ++u) {
        half8_t a0[NM], a1[NM];
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            half2_t s2, b2;
            sb_half2(g0 + u < G ? L.s[m][u] : 0u, &s2, &b2);
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

// One row tile of a staged item over all G column groups: acc[m][t] holds
// rows 16 ms + 4 (lane / 16) + i, token 16 t + lane % 16 of matrix m.
// KBM is the widest batch the LDS rows hold; NTT > 4 halves the batch to
// keep the prefetched token rows within the register budget.
template <int NM, int NTT, int KBM>
__device__ __forceinline__ void gg_tile_n(const uint8_t* const* tiles, int G, const _Float16* src, int64_t stride,
                                          const int* rows, int count, _Float16 (*xs)[pitch_of<KBM>()],
                                          float4_t (*acc)[8]) {
    constexpr int KB = NTT <= 4 ? KBM : (KBM < 2 ? KBM : 2);
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
    // just read, which keeps every load unconditional.  sched_barrier keeps
    // the compiler from sinking the prefetch towards its use.
    for (int g0 = 0;; g0 += 2 * KB) {
        x_store(X, xs);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        x_load(X, src, stride, rows, count, g0 + KB, G);
        w_load(B, wbase, sbase, g0 + KB, G);
        __builtin_amdgcn_sched_barrier(0);
        w_mma<NM, NTT, KB>(A, xs, acc, lane, g0, G);
        __syncthreads();
        if (g0 + KB >= G) break;
        x_store(X, xs);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        x_load(X, src, stride, rows, count, g0 + 2 * KB, G);
        w_load(A, wbase, sbase, g0 + 2 * KB, G);
        __builtin_amdgcn_sched_barrier(0);
        w_mma<NM, NTT, KB>(B, xs, acc, lane, g0 + KB, G);
        __syncthreads();
        if (g0 + 2 * KB >= G) break;
    }
}

// Dispatch on the chunk's 16-token tiles (3 .. 8) so that every MFMA
// sequence is straight-line code.
template <int NM, int KBM>
__device__ __forceinline__ void gg_tile(const uint8_t* const* tiles, int G, const _Float16* src, int64_t stride,
                                        const int* rows, int count, _Float16 (*xs)[pitch_of<KBM>()],
                                        float4_t (*acc)[8]) {
    switch ((count + 15) / 16) {
        case 3: gg_tile_n<NM, 3, KBM>(tiles, G, src, stride, rows, count, xs, acc); break;
        case 4: gg_tile_n<NM, 4, KBM>(tiles, G, src, stride, rows, count, xs, acc); break;
        case 5: gg_tile_n<NM, 5, KBM>(tiles, G, src, stride, rows, count, xs, acc); break;
        case 6: gg_tile_n<NM, 6, KBM>(tiles, G, src, stride, rows, count, xs, acc); break;
        case 7: gg_tile_n<NM, 7, KBM>(tiles, G, src, stride, rows, count, xs, acc); break;
        default: gg_tile_n<NM, 8, KBM>(tiles, G, src, stride, rows, count, xs, acc); break;
    }
}

// The work item of this workgroup: blockIdx.y indexes the schedule
// (expert << 16 | tiles << 8 | chunk).  Experts E .. E+n_vs-1 are the shared expert's
// virtual experts.
struct Item {
    int ntt;            // 16-token tiles of the chunk
    int count;          // tokens of the chunk
    int pos0;           // row of chunk token 0 in hg / ysort
    int shared;         // 1 for a virtual shared expert
    int tok0;           // shared: first token of the chunk
    int G;              // column groups of the operand
    int64_t rstride;    // bytes from one 64-row tile of the matrices to the next
    const uint8_t* w[2];
};

// The matrices of the item's row tile rt, from the schedule entry alone, so
// that weight loads can start before the token bookkeeping arrives.
// Returns false when the workgroup has nothing to do.
__device__ __forceinline__ bool gg_weights(const Plan& p, bool down, int rt, Item* it) {
    if ((int)blockIdx.y >= *p.nsched) return false;
    const int sc = p.sched[blockIdx.y], ex = sc >> 16, c = sc & 0xFF;
    it->ntt = (sc >> 8) & 0xFF;
    it->tok0 = c;   // chunk index until gg_tokens
    if (ex < p.E) {
        it->shared = 0;
        it->pos0 = ex;   // expert until gg_tokens
        const uint8_t* base = p.pool_base + (int64_t)ex * p.expert_stride;
        if (down) {
            it->G = p.G_I;
            it->rstride = (int64_t)p.G_I * kBlk4;
            it->w[0] = it->w[1] = base + p.down_off + (int64_t)rt * p.G_I * kBlk4;
        } else {
            it->G = p.G_H;
            it->rstride = (int64_t)p.G_H * kBlk4;
            it->w[0] = base + p.gate_off + (int64_t)rt * p.G_H * kBlk4;
            it->w[1] = base + p.up_off + (int64_t)rt * p.G_H * kBlk4;
        }
    } else {
        const int j = ex - p.E;
        it->shared = 1;
        it->pos0 = j;    // virtual expert until gg_tokens
        if (down) {
            it->G = min(p.G_I, p.G_s - j * p.G_I);
            it->rstride = (int64_t)p.G_s * kBlk4;
            it->w[0] = it->w[1] = p.sh_down + ((int64_t)rt * p.G_s + (int64_t)j * p.G_I) * kBlk4;
        } else {
            if (rt * 64 >= p.Is - j * p.I) return false;   // the last virtual expert may be shorter
            it->G = p.G_H;
            it->rstride = (int64_t)p.G_H * kBlk4;
            it->w[0] = p.sh_gate + (int64_t)(j * p.G_I + rt) * p.G_H * kBlk4;
            it->w[1] = p.sh_up + (int64_t)(j * p.G_I + rt) * p.G_H * kBlk4;
        }
    }
    return true;
}

// The chunk's tokens: count, first sorted position and (shared) first token.
__device__ __forceinline__ void gg_tokens(const Plan& p, Item* it) {
    const int c = it->tok0;
    if (!it->shared) {
        const int ex = it->pos0;
        const int first = p.offsets[ex] + c * p.ntile;
        it->count = min(p.ntile, p.offsets[ex + 1] - first);
        it->pos0 = first;
        it->tok0 = 0;
    } else {
        const int j = it->pos0;
        it->tok0 = c * p.ntile;
        it->count = min(p.ntile, p.T - it->tok0);
        it->pos0 = p.T * p.k + j * p.T + it->tok0;
    }
}

// ---- gate/up, up to 32 tokens: the four waves split the column groups
// (wave w takes groups w, w+4, ...) over all 64 rows of the tile, so each
// wave loads only its own token fragments, straight into registers; the
// partial sums meet in LDS at the end.
struct GuW {
    u32x4_t c[2][2];     // [matrix][row-block pair]: codes, lane's 16 bytes of each half block
    u32x4_t s[2];        // [matrix]: scale|bias of row lane % 16 in each of the four row blocks
};
template <int NTT>
struct GuX {
    half8_t x[NTT][2];   // token fragments: columns 8 (lane / 16) .. +7 and 32 + that
};

__device__ __forceinline__ void gu_wload(GuW& L, const uint8_t* w0, const uint8_t* w1, int g, int lane) {
    const uint8_t* b[2] = {w0 + (int64_t)g * kBlk4, w1 + (int64_t)g * kBlk4};
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        L.c[m][0] = *(const u32x4_t*)(b[m] + lane * 16);
        L.c[m][1] = *(const u32x4_t*)(b[m] + 1024 + lane * 16);
        L.s[m] = *(const u32x4_t*)(b[m] + kCodes4 + (lane & 15) * 16);
    }
}

// xr[t]: element offset in x16 of the lane's first column of tile t.
template <int NTT>
__device__ __forceinline__ void gu_xload(GuX<NTT>& X, const _Float16* x16, const int* xr, int g) {
#pragma unroll
    for (int t = 0; t < NTT; ++t) {
        X.x[t][0] = *(const half8_t*)(x16 + (uint32_t)(xr[t] + g * 64));
        X.x[t][1] = *(const half8_t*)(x16 + (uint32_t)(xr[t] + g * 64 + 32));
    }
}

// One fragment is dequantised at a time (sched_barrier keeps the compiler
// from hoisting all eight), which bounds the registers they take.
template <int NTT>
__device__ __forceinline__ void gu_mma(const GuW& L, const GuX<NTT>& X, float4_t (*acc)[4][NTT]) {
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
            __builtin_amdgcn_sched_barrier(0);
            half2_t s2, b2;
            sb_half2(L.s[m][rb], &s2, &b2);
            const half8_t a0 = dequant8(L.c[m][rb >> 1][2 * (rb & 1)], s2, b2);
            const half8_t a1 = dequant8(L.c[m][rb >> 1][2 * (rb & 1) + 1], s2, b2);
#pragma unroll
            for (int t = 0; t < NTT; ++t) {
                acc[m][rb][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, X.x[t][0], acc[m][rb][t], 0, 0, 0);
                acc[m][rb][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, X.x[t][1], acc[m][rb][t], 0, 0, 0);
            }
        }
}

typedef float4_t GuRed[4][3][2][2][64];   // [row block][other wave][matrix][tile][lane]

// The wave's groups are w + 4 j, j < nj; WA and WB hold the weights of
// j = 0 and 1, loaded before the token bookkeeping.  sched_barrier pins each
// refill right after the multiply that frees its registers, so the next
// groups stay in flight behind the one in use: two of them for one token
// tile, one for two (register budget).  Prefetch past the end re-reads the
// last group; the loops have one exit, a multiply past the end is skipped.
template <int NTT>
__device__ __forceinline__ void gu_small_n(const Plan& p, const Item& it, GuW& WA, GuW& WB, GuRed& red) {
    const int w = wave_id(), lane = threadIdx.x & 63;
    const _Float16* x16 = p.x16;
    int xr[NTT];
#pragma unroll
    for (int t = 0; t < NTT; ++t) {
        const int n = min(16 * t + (lane & 15), it.count - 1);
        const int tok = it.shared ? it.tok0 + n : p.perm[it.pos0 + n] / p.k;
        xr[t] = tok * p.H + 8 * (lane >> 4);
    }
    const int G = it.G, nj = (G - w + 3) / 4;
    auto grp = [&](int j) { return min(w + 4 * j, G - 1); };
    const uint8_t *w0 = it.w[0], *w1 = it.w[1];
    float4_t acc[2][4][NTT];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
            for (int t = 0; t < NTT; ++t) acc[m][rb][t] = (float4_t){0.f, 0.f, 0.f, 0.f};
    GuX<NTT> XA, XB;
    gu_xload(XA, x16, xr, grp(0));
    gu_xload(XB, x16, xr, grp(1));
    if constexpr (NTT >= 2) {
        for (int j = 0; j < nj; j += 2) {
            __builtin_amdgcn_sched_barrier(0);
            gu_mma<NTT>(WA, XA, acc);
            __builtin_amdgcn_sched_barrier(0);
            gu_wload(WA, w0, w1, grp(j + 2), lane);
            gu_xload(XA, x16, xr, grp(j + 2));
            __builtin_amdgcn_sched_barrier(0);
            if (j + 1 < nj) gu_mma<NTT>(WB, XB, acc);
            __builtin_amdgcn_sched_barrier(0);
            gu_wload(WB, w0, w1, grp(j + 3), lane);
            gu_xload(XB, x16, xr, grp(j + 3));
        }
    } else {
        GuW WC;
        GuX<NTT> XC;
        gu_wload(WC, w0, w1, grp(2), lane);
        gu_xload(XC, x16, xr, grp(2));
        for (int j = 0; j < nj; j += 3) {
            __builtin_amdgcn_sched_barrier(0);
            gu_mma<NTT>(WA, XA, acc);
            __builtin_amdgcn_sched_barrier(0);
            gu_wload(WA, w0, w1, grp(j + 3), lane);
            gu_xload(XA, x16, xr, grp(j + 3));
            __builtin_amdgcn_sched_barrier(0);
            if (j + 1 < nj) gu_mma<NTT>(WB, XB, acc);
            __builtin_amdgcn_sched_barrier(0);
            gu_wload(WB, w0, w1, grp(j + 4), lane);
            gu_xload(XB, x16, xr, grp(j + 4));
            __builtin_amdgcn_sched_barrier(0);
            if (j + 2 < nj) gu_mma<NTT>(WC, XC, acc);
            __builtin_amdgcn_sched_barrier(0);
            gu_wload(WC, w0, w1, grp(j + 5), lane);
            gu_xload(XC, x16, xr, grp(j + 5));
        }
    }
    // wave w sums row block w over the four waves (fixed order: own, then the others by wave)
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
        if (rb != w)
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int t = 0; t < NTT; ++t) red[rb][w < rb ? w : w - 1][m][t][lane] = acc[m][rb][t];
    __syncthreads();
    const int r0 = blockIdx.x * 64 + 16 * w + 4 * (lane >> 4);
#pragma unroll
    for (int t = 0; t < NTT; ++t) {
        float4_t v[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            float4_t a = w == 0 ? acc[m][0][t] : w == 1 ? acc[m][1][t] : w == 2 ? acc[m][2][t] : acc[m][3][t];
#pragma unroll
            for (int q = 0; q < 3; ++q) a += red[w][q][m][t][lane];
            v[m] = a;
        }
        const int n = 16 * t + (lane & 15);
        if (n < it.count) {
            _Float16* dst = p.hg + (int64_t)(it.pos0 + n) * p.I + r0;
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[i] = (_Float16)(gelu_tanh(v[0][i]) * v[1][i]);
        }
    }
}

// ---- gate/up, more than 32 tokens: x staged in LDS for the whole chunk.
typedef _Float16 GuXs[128][pitch_of<kBigKB>()];

__device__ __forceinline__ void gu_big(const Plan& p, const Item& it, GuXs& xs, int* rows) {
    const int wave = wave_id(), lane = threadIdx.x & 63;
    if ((int)threadIdx.x < it.count)
        rows[threadIdx.x] = it.shared ? it.tok0 + threadIdx.x : p.perm[it.pos0 + threadIdx.x] / p.k;
    __syncthreads();
    float4_t acc[2][8];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int t = 0; t < 8; ++t) acc[m][t] = (float4_t){0.f, 0.f, 0.f, 0.f};
    gg_tile<2, kBigKB>(it.w, it.G, p.x16, p.H, rows, it.count, xs, acc);
    const int r0 = blockIdx.x * 64 + 16 * wave + 4 * (lane >> 4);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const int n = 16 * t + (lane & 15);
        if (n < it.count) {
            _Float16* dst = p.hg + (int64_t)(it.pos0 + n) * p.I + r0;
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[i] = (_Float16)(gelu_tanh(acc[0][t][i]) * acc[1][t][i]);
        }
    }
}

// Gate/up + GeGLU: hg[pos] = gelu(gate x) * (up x) in fp16.
// grid (I / 64, max_tiles), block 256.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_gu(Plan p) {
    constexpr size_t kLds = sizeof(GuXs) > sizeof(GuRed) ? sizeof(GuXs) : sizeof(GuRed);
    __shared__ __attribute__((aligned(16))) char lds[kLds];
    __shared__ int rows[128];
    Item it;
    if (!gg_weights(p, false, blockIdx.x, &it)) return;
    const int w = wave_id(), lane = threadIdx.x & 63;
    if (it.ntt > 2) {
        gg_tokens(p, &it);
        gu_big(p, it, *(GuXs*)lds, rows);
        return;
    }
    // first weights, in flight while the tokens arrive
    GuW WA, WB;
    gu_wload(WA, it.w[0], it.w[1], min(w, it.G - 1), lane);
    gu_wload(WB, it.w[0], it.w[1], min(w + 4, it.G - 1), lane);
    gg_tokens(p, &it);
    if (it.ntt == 1) gu_small_n<1>(p, it, WA, WB, *(GuRed*)lds);
    else gu_small_n<2>(p, it, WA, WB, *(GuRed*)lds);
}

// ---- down, up to 32 tokens: the chunk's GeGLU rows are staged in LDS once;
// the workgroup then runs over its kDnTiles output tiles with no further
// barrier, each wave keeping three batches of four column groups of
// weights in flight.
constexpr int kSmKB = 4;

struct DnLoads {
    uint2 c[kSmKB];
    uint32_t s[kSmKB];
};

__device__ __forceinline__ void dn_load(DnLoads& L, const uint8_t* wb, const uint8_t* sb, int64_t rstride, int q,
                                        int nq, int nb, int G) {
    q = min(q, nq - 1);   // prefetch past the end re-reads the last batch
    const int r = q / nb, g0 = (q - r * nb) * kSmKB;
#pragma unroll
    for (int u = 0; u < kSmKB; ++u) {
        const int g = min(g0 + u, G - 1);
        L.c[u] = *(const uint2*)(wb + r * rstride + (int64_t)g * kBlk4);
        L.s[u] = *(const uint32_t*)(sb + r * rstride + (int64_t)g * kBlk4);
    }
}

// Batch of groups g0 .. g0+kSmKB-1; a group past the end (zero weights)
// reads the staged columns of group G-1, which hold finite values.
template <int NTT>
__device__ __forceinline__ void dn_mma(const DnLoads& L, const _Float16* hs, int pitch, int g0, int G, float4_t* acc,
                                       int lane) {
    const int kb = lane >> 4, n = lane & 15;
#pragma unroll
    for (int u = 0; u < kSmKB; ++u) {
        const int col0 = min(g0 + u, G - 1) * 64;
        half2_t s2, b2;
        sb_half2(g0 + u < G ? L.s[u] : 0u, &s2, &b2);   // groups past the end weigh zero
        const half8_t a0 = dequant8(L.c[u].x, s2, b2);
        const half8_t a1 = dequant8(L.c[u].y, s2, b2);
#pragma unroll
        for (int t = 0; t < NTT; ++t) {
            const _Float16* row = hs + (16 * t + n) * pitch + col0 + 8 * kb;
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, *(const half8_t*)row, acc[t], 0, 0, 0);
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, *(const half8_t*)(row + 32), acc[t], 0, 0, 0);
        }
    }
}

// A, B, C hold batches 0, 1, 2, loaded before the chunk was staged.
template <int NTT>
__device__ __forceinline__ void dn_small_n(const Plan& p, const Item& it, int rt0, int nrt, const _Float16* hs,
                                           int pitch, const float* wrow, const uint8_t* wb, const uint8_t* sb,
                                           DnLoads& A, DnLoads& B, DnLoads& C) {
    const int ms = wave_id(), lane = threadIdx.x & 63;
    const int G = it.G, nb = (G + kSmKB - 1) / kSmKB, nq = nrt * nb;
    float4_t acc[NTT];
#pragma unroll
    for (int t = 0; t < NTT; ++t) acc[t] = (float4_t){0.f, 0.f, 0.f, 0.f};
    auto finish = [&](int q) {   // after batch q: store the tile if it was its last batch
        const int r = q / nb;
        if (q - r * nb != nb - 1) return;
        const int r0 = (rt0 + r) * 64 + 16 * ms + 4 * (lane >> 4);
#pragma unroll
        for (int t = 0; t < NTT; ++t) {
            const int n = 16 * t + (lane & 15);
            if (n < it.count) {
                float* dst = p.ysort + (int64_t)(it.pos0 + n) * p.H + r0;
                const float wt = wrow[n];
#pragma unroll
                for (int i = 0; i < 4; ++i) dst[i] = wt * acc[t][i];
            }
            acc[t] = (float4_t){0.f, 0.f, 0.f, 0.f};
        }
    };
    auto grp0 = [&](int q) { return (q % nb) * kSmKB; };
    // one exit: batches past the end skip their multiply
    for (int q = 0; q < nq; q += 3) {
        __builtin_amdgcn_sched_barrier(0);
        dn_mma<NTT>(A, hs, pitch, grp0(q), G, acc, lane);
        finish(q);
        __builtin_amdgcn_sched_barrier(0);
        dn_load(A, wb, sb, it.rstride, q + 3, nq, nb, G);
        __builtin_amdgcn_sched_barrier(0);
        if (q + 1 < nq) {
            dn_mma<NTT>(B, hs, pitch, grp0(q + 1), G, acc, lane);
            finish(q + 1);
        }
        __builtin_amdgcn_sched_barrier(0);
        dn_load(B, wb, sb, it.rstride, q + 4, nq, nb, G);
        __builtin_amdgcn_sched_barrier(0);
        if (q + 2 < nq) {
            dn_mma<NTT>(C, hs, pitch, grp0(q + 2), G, acc, lane);
            finish(q + 2);
        }
        __builtin_amdgcn_sched_barrier(0);
        dn_load(C, wb, sb, it.rstride, q + 5, nq, nb, G);
    }
}

// ---- down, more than 32 tokens: h staged in LDS kDnKB groups at a time per
// output tile, for the whole chunk.
__device__ __forceinline__ void dn_big(const Plan& p, const Item& it, int rt0, int nrt, _Float16* lds, int* rows,
                                       const float* wrow) {
    const int wave = wave_id(), lane = threadIdx.x & 63;
    auto xs = (_Float16(*)[pitch_of<kDnKB>()])lds;
    for (int r = 0; r < nrt; ++r) {
        float4_t acc[1][8];
#pragma unroll
        for (int t = 0; t < 8; ++t) acc[0][t] = (float4_t){0.f, 0.f, 0.f, 0.f};
        const uint8_t* tiles[1] = {it.w[0] + r * it.rstride};
        gg_tile<1, kDnKB>(tiles, it.G, p.hg, p.I, rows, it.count, xs, acc);
        const int r0 = (rt0 + r) * 64 + 16 * wave + 4 * (lane >> 4);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int n = 16 * t + (lane & 15);
            if (n < it.count) {
                const float wt = wrow[n];
                float* dst = p.ysort + (int64_t)(it.pos0 + n) * p.H + r0;
#pragma unroll
                for (int i = 0; i < 4; ++i) dst[i] = wt * acc[0][t][i];
            }
        }
    }
}

// Down projection: ysort[pos] = w_pair * (W_down . h), weight 1 for the
// shared expert's slices.  grid (ceil(H / 64 / kDnTiles), max_tiles), block
// 256, dynamic LDS dn_lds_bytes(I).
__global__ __launch_bounds__(256) void k_dn(Plan p) {
    extern __shared__ __attribute__((aligned(16))) _Float16 hs[];
    __shared__ float wrow[128];
    __shared__ int rows[128];
    const int rt0 = blockIdx.x * kDnTiles, nrt = min(kDnTiles, p.H / 64 - rt0);
    Item it;
    if (!gg_weights(p, true, rt0, &it)) return;
    auto token_rows = [&]() {
        if ((int)threadIdx.x < it.count) {
            wrow[threadIdx.x] = it.shared ? 1.f : p.wts[p.perm[it.pos0 + threadIdx.x]];
            rows[threadIdx.x] = it.pos0 + threadIdx.x;
        }
    };
    if (it.ntt > 2) {
        gg_tokens(p, &it);
        token_rows();
        __syncthreads();
        dn_big(p, it, rt0, nrt, hs, rows, wrow);
        return;
    }
    const int ms = wave_id(), lane = threadIdx.x & 63;
    const int nb = (it.G + kSmKB - 1) / kSmKB, nq = nrt * nb;
    const uint8_t* wb = it.w[0] + ((ms >> 1) * 64 + lane) * 16 + 8 * (ms & 1);
    const uint8_t* sb = it.w[0] + kCodes4 + (lane & 15) * 16 + 4 * ms;
    // first weights, in flight while the tokens arrive
    DnLoads A, B, C;
    dn_load(A, wb, sb, it.rstride, 0, nq, nb, it.G);
    dn_load(B, wb, sb, it.rstride, 1, nq, nb, it.G);
    dn_load(C, wb, sb, it.rstride, 2, nq, nb, it.G);
    gg_tokens(p, &it);
    token_rows();
    // stage the chunk: rows past it repeat its last row; columns past G
    // groups are never read
    const int pitch = p.I + 8;
    const int per = it.G * 8;   // 16-byte pieces per row
    const int nrow = it.ntt * 16;
    for (int c = threadIdx.x; c < nrow * per; c += 256) {
        const int n = c / per, q = c - n * per;
        const int src = it.pos0 + min(n, it.count - 1);
        *(u32x4_t*)&hs[n * pitch + q * 8] = *(const u32x4_t*)(p.hg + (int64_t)src * p.I + q * 8);
    }
    __syncthreads();
    if (nrow == 16) dn_small_n<1>(p, it, rt0, nrt, hs, pitch, wrow, wb, sb, A, B, C);
    else dn_small_n<2>(p, it, rt0, nrt, hs, pitch, wrow, wb, sb, A, B, C);
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

// Dynamic LDS of k_dn: the larger of the small path's staged chunk and the
// big path's batch.
size_t dn_lds_bytes(int I) {
    const size_t small = (size_t)32 * (I + 8) * 2, big = (size_t)128 * pitch_of<kDnKB>() * 2;
    return small > big ? small : big;
}

// The schedule holds chunk indices below 256 (T <= 255 * 128), and the
// LDS of the front and down kernels must fit a workgroup.
bool grouped_ok(int H, int I, int64_t T) {
    return T <= 255 * 128 && dn_lds_bytes(I) <= 160 * 1024 && (size_t)kFrontTokens * H * 4 + kFrontStatic <= 160 * 1024;
}

mq_status launch_grouped(const Plan& p, hipStream_t s) {
    const size_t dn_lds = dn_lds_bytes(p.I);
    if (dn_lds > 64 * 1024 &&
        hipFuncSetAttribute((const void*)k_dn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)dn_lds) != hipSuccess)
        return MQ_ERR_UNSUPPORTED;
    // one token per front workgroup while that fills the machine, else four
    const bool tg4 = p.T > 512;
    const int tg = tg4 ? kFrontTokens : 1;
    const size_t fr_lds = (size_t)tg * p.H * 4;
    const void* fr = tg4 ? (const void*)k_front<kFrontTokens> : (const void*)k_front<1>;
    if (fr_lds > 64 * 1024 && hipFuncSetAttribute(fr, hipFuncAttributeMaxDynamicSharedMemorySize, (int)fr_lds) != hipSuccess)
        return MQ_ERR_UNSUPPORTED;
    if (tg4)
        hipLaunchKernelGGL(k_front<kFrontTokens>, dim3((p.T + tg - 1) / tg), dim3(1024), fr_lds, s, p);
    else
        hipLaunchKernelGGL(k_front<1>, dim3(p.T), dim3(1024), fr_lds, s, p);
    hipLaunchKernelGGL(k_gu, dim3(p.I / 64, p.max_tiles), dim3(256), 0, s, p);
    hipLaunchKernelGGL(k_dn, dim3((p.H / 64 + kDnTiles - 1) / kDnTiles, p.max_tiles), dim3(256), dn_lds, s, p);
    hipLaunchKernelGGL(k_gg_combine, dim3(p.T, (p.H + 255) / 256), dim3(256), 0, s, p);
    return MQ_OK;
}

}  // namespace mq
