// Grouped path (many tokens per call): token -> expert permutation, grouped
// dequant-GEMMs on the matrix cores, and the combine.
//
// One DEV_V1 word per lane holds the eight 4-bit codes of one row and
// eight consecutive columns, which is exactly a weight fragment of
// v_mfma_f32_16x16x32_f16 for lane (row % 16, column block lane / 16), as
// the A operand (D[row][token]) or as the B operand (D[token][row]).
// Accumulation is fp32 throughout.
#include "device.h"
#include "plan.h"

#include "../../include/moegemv.h"

namespace mq {

__global__ void k_tail_grouped(Plan p);   // tail.hip

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

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
// Front of the grouped path: router scores (k_scores), then top-k, softmax,
// the token -> expert permutation and the work schedule (k_select).
// Units with at most this many tokens take the code-operand path of the
// grouped GEMMs, the others the dequantised-weight path for all their
// chunks: the choice is per unit, so a token's arithmetic does not depend
// on which chunk of its expert it lands in.
constexpr int kSmallTokens = 16;

// Schedule entries: the full chunks of every unit (the experts, then the
// shared expert's virtual experts E .. E+n_vs-1 over all T tokens), then
// the partial last chunks by decreasing number of 16-token tiles.  With
// 128-token chunks the partial chunks of units on the dequantised-weight
// path come first, then those on the code-operand path: a dequantised-weight
// chunk streams its whole weight tiles whatever its token count, so even a
// short one takes as long as a full one.  nsched[0] = entries, nsched[1] =
// entries before the code-operand ones (nsched[0] with 64-token chunks, where
// the order by size alone measured best).  Entry .x = unit << 16 | big << 12 | tiles << 8 | chunk
// (big: the unit has more than kSmallTokens tokens), .y = first sorted row
// of the chunk (in hg / ysort) | its token count << 24.  Items are
// independent, so the order within a class does not matter.
// cnt, off: this thread's expert count and first sorted row (thread u < E);
// every thread calls it.
__device__ __forceinline__ void build_schedule(const Plan& p, int cnt, int off, int* scan) {
    __shared__ int ccount[33], cfill[33];   // by class: 16-token tiles, + 16 on the dequantised-weight path
    const int T = p.T, E = p.E, nu = E + p.n_vs;   // nu <= kMaxExperts + a few <= 1024
    const int u = threadIdx.x;
    const int ucnt = u < E ? cnt : (u < nu ? T : 0);
    const int row0 = u < E ? off : T * p.k + (u - E) * T;
    const int nfull = ucnt / p.ntile, rem = ucnt - nfull * p.ntile;
    const int tiles = rem > 0 ? (rem + 15) / 16 : 0;   // 1 .. ntile / 16
    const int big = (ucnt > kSmallTokens) << 12;
    const int cls = tiles > 0 ? tiles + (big && p.ntile > 64 ? 16 : 0) : 0;
    int foff;
    const int tfull = block_scan_total(scan, nu, nfull, &foff);
    for (int c = 0; c < nfull; ++c)
        p.sched[foff + c] =
            make_int2((u << 16) | big | ((p.ntile / 16) << 8) | c, (row0 + c * p.ntile) | (p.ntile << 24));
    if (threadIdx.x < 33) ccount[threadIdx.x] = cfill[threadIdx.x] = 0;
    __syncthreads();
    if (cls > 0) atomicAdd(&ccount[cls], 1);
    __syncthreads();
    if (cls > 0) {
        int before = 0;   // partial chunks of heavier classes
        for (int q = cls + 1; q <= 32; ++q) before += ccount[q];
        p.sched[tfull + before + atomicAdd(&cfill[cls], 1)] =
            make_int2((u << 16) | big | (tiles << 8) | nfull, (row0 + nfull * p.ntile) | (rem << 24));
    }
    if (threadIdx.x == 0) {
        int nbig = 0, nsmall = 0;
        for (int q = 17; q <= 32; ++q) nbig += ccount[q];
        for (int q = 1; q <= 16; ++q) nsmall += ccount[q];
        p.nsched[0] = tfull + nbig + nsmall;
        p.nsched[1] = p.ntile > 64 ? tfull + nbig : tfull + nbig + nsmall;
    }
}

// ---- router scores on the matrix cores (v_mfma_f32_16x16x4_f32: fp32
// operands, so the scores keep fp32 precision).  The RMS factor of the
// router input is a per-token scalar, so the scores are first taken over
// the unnormalised input a = x * router_scale and scaled afterwards:
//     score[t][e] = c[t] * sum_g (s[e][g] sum_{k in g} q[e][k] a[t][k]
//                                + b[e][g] sum_{k in g} a[t][k]),
//     c[t] = 1 / sqrt(mean(x[t]^2) + eps) / sqrt(H).
// Workgroup (token tile of 16, router row tile of 64 experts, column split
// ks): the staged a[16][batch columns] is the A operand (D[token][expert]),
// wave j takes experts 16 j .. 16 j + 15 of the row tile and the 8-bit codes
// of its DEV_V1 words are the B operand (one byte conversion each); the
// group scale and bias are applied once per output in fp32.  The partial
// scores of each column split go to plog[ks][t][e], the partial sums of x^2
// to the router-sum area; the workgroups of row tile 0 also write x16 and
// xso for their columns.  grid (ceil(T / 16), E_pad / 64, splits), block 256.
constexpr int kScBatch = 4;   // column groups per staged batch

__global__ __launch_bounds__(256) void k_scores(Plan p) {
    __shared__ __attribute__((aligned(16))) float A[16][kScBatch * 64 + 4];
    __shared__ __attribute__((aligned(16))) float asum[kScBatch][16];
    const int tt = blockIdx.x, rt = blockIdx.y, ks = blockIdx.z;
    const int tid = threadIdx.x, j = wave_id(), lane = tid & 63;
    const int gpw = (p.G_H + gridDim.z - 1) / gridDim.z;
    const int g_begin = ks * gpw, g_end = min(p.G_H, g_begin + gpw);
    // staging role: token st of the tile, columns c4 .. c4 + 3 of each group
    const int st = tid >> 4, c4 = (tid & 15) * 4;
    const int t_st = tt * 16 + st, tok = min(t_st, p.T - 1);
    const uint16_t* xrow = p.x + (int64_t)tok * p.x_stride;
    const bool writer = rt == 0 && t_st < p.T;   // x16, xso and the x^2 sums
    const uint8_t* rbase = p.router_w + (int64_t)rt * p.G_H * kBlk8;
    float ss = 0.f;
    float4_t out = {0.f, 0.f, 0.f, 0.f};   // token 4 (lane / 16) + i, expert 16 j + lane % 16
    // the batch's router words (wave j's 16 experts) and activations; groups
    // past the range re-read its last group and are not used.  The next
    // batch's loads go out while the current batch is multiplied.
    u32x4_t cw[kScBatch], ncw[kScBatch];
    uint32_t pr[kScBatch], npr[kScBatch];
    uint2 xv[kScBatch], nxv[kScBatch];
    float4_t rs[kScBatch], nrs[kScBatch];
    auto load_batch = [&](int g0) {
#pragma unroll
        for (int gi = 0; gi < kScBatch; ++gi) {
            const int g = min(g0 + gi, g_end - 1);
            ncw[gi] = *(const u32x4_t*)(rbase + (int64_t)g * kBlk8 + (j * 64 + lane) * 16);
            npr[gi] = *(const uint32_t*)(rbase + (int64_t)g * kBlk8 + kCodes8 + (lane & 15) * 16 + 4 * j);
            nxv[gi] = *(const uint2*)(xrow + g * 64 + c4);
            nrs[gi] = p.router_scale ? *(const float4_t*)(p.router_scale + g * 64 + c4)
                                     : (float4_t){1.f, 1.f, 1.f, 1.f};
        }
    };
    load_batch(g_begin);
    for (int g0 = g_begin; g0 < g_end; g0 += kScBatch) {
        const int nbg = min(kScBatch, g_end - g0);
#pragma unroll
        for (int gi = 0; gi < kScBatch; ++gi) {
            cw[gi] = ncw[gi];
            pr[gi] = npr[gi];
            xv[gi] = nxv[gi];
            rs[gi] = nrs[gi];
        }
        load_batch(g0 + kScBatch);
        __syncthreads();   // the previous batch's operands are read
#pragma unroll
        for (int gi = 0; gi < kScBatch; ++gi) {
            if (gi >= nbg) break;
            const float x0 = bf16_lo(xv[gi].x), x1 = bf16_hi(xv[gi].x), x2 = bf16_lo(xv[gi].y), x3 = bf16_hi(xv[gi].y);
            const float4_t a = {x0 * rs[gi][0], x1 * rs[gi][1], x2 * rs[gi][2], x3 * rs[gi][3]};
            *(float4_t*)&A[st][gi * 64 + c4] = a;
            const float as = sum16((a[0] + a[1]) + (a[2] + a[3]));
            if ((tid & 15) == 0) asum[gi][st] = as;
            ss += (x0 * x0 + x1 * x1) + (x2 * x2 + x3 * x3);
            if (rt == 0) {
                // x16 (columns with c & 2 divided by 16; c4 + 2, c4 + 3 are those) and xso
                const _Float16 h0 = (_Float16)x0, h1 = (_Float16)x1, h2 = (_Float16)x2, h3 = (_Float16)x3;
                const _Float16 s2 = h2 * (_Float16)0.0625f, s3 = h3 * (_Float16)0.0625f;
                flag_error(p.f_err, t_st < p.T && (f16_bad(h0) || f16_bad(h1) || f16_bad(h2) || f16_bad(h3)), kErrRange);
                const float xs = sum16(((float)h0 + (float)h1) + ((float)h2 + (float)h3));
                const float xn = sum16(-1024.0f * (((float)h0 + (float)h1) + ((float)s2 + (float)s3)));
                if (t_st < p.T) {
                    typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
                    *(half4_t*)(p.x16 + (int64_t)t_st * p.H + (g0 + gi) * 64 + c4) = (half4_t){h0, h1, s2, s3};
                    if ((tid & 15) == 0)
                        ((float2*)p.xso)[(int64_t)t_st * p.G_H + g0 + gi] = make_float2(xs, xn);
                }
            }
        }
        __syncthreads();
#pragma unroll
        for (int gi = 0; gi < kScBatch; ++gi) {
            if (gi >= nbg) break;
            float4_t acc[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float4_t av = *(const float4_t*)&A[lane & 15][gi * 64 + 16 * i + 4 * (lane >> 4)];
                acc[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[0], (float)((cw[gi][i] >> 0) & 0xFFu),
                                                              (float4_t){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                acc[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[1], (float)((cw[gi][i] >> 8) & 0xFFu), acc[i],
                                                              0, 0, 0);
                acc[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[2], (float)((cw[gi][i] >> 16) & 0xFFu), acc[i],
                                                              0, 0, 0);
                acc[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[3], (float)((cw[gi][i] >> 24) & 0xFFu), acc[i],
                                                              0, 0, 0);
            }
            const float4_t d = (acc[0] + acc[1]) + (acc[2] + acc[3]);
            const float4_t sm = *(const float4_t*)&asum[gi][4 * (lane >> 4)];
            const float sc = bf16_lo(pr[gi]), bi = bf16_hi(pr[gi]);
#pragma unroll
            for (int i = 0; i < 4; ++i) out[i] = fmaf(sc, d[i], fmaf(bi, sm[i], out[i]));
        }
    }
    const int e = rt * 64 + 16 * j + (lane & 15);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = tt * 16 + 4 * (lane >> 4) + i;
        if (t < p.T) p.plog[((int64_t)ks * p.T + t) * p.E_pad + e] = out[i];
    }
    ss = sum16(ss);
    if (writer && (tid & 15) == 0) p.rsum8[(int64_t)ks * p.T + t_st] = ss;
}

// ---- selection: one wave per token.  The scores are the column splits'
// sum times the RMS factor (plus logit_bias); the k highest are taken by
// k rounds of a wave-wide argmax (equal scores go to the lower expert, a
// NaN score ranks last), then the softmax over them times per_expert_scale.
// grid (ceil(T / 4)), block 256: one wave per SIMD.  KM: 64-expert slices
// per lane (E <= 64 KM).
template <int KM>
__global__ __launch_bounds__(256) void k_select(Plan p) {
    const int lane = threadIdx.x & 63, w = wave_id();
    const int t = blockIdx.x * 4 + w, E = p.E, k = p.k, ns = p.rsplit_used;
    if (t < p.T) {
        // the column splits' partials, summed in split order; the loads of a
        // batch of sixteen splits go out together (clamped, in bounds)
        constexpr int kB = 16, kM = KM;
        float ss = 0.f, sum[kM], bias[kM];
#pragma unroll
        for (int m = 0; m < kM; ++m) bias[m] = p.logit_bias ? p.logit_bias[min(lane + 64 * m, E - 1)] : 0.f;
#pragma unroll
        for (int m = 0; m < kM; ++m) sum[m] = 0.f;
        for (int q0 = 0; q0 < ns; q0 += kB) {
            float ps[kB], pl[kM][kB];
#pragma unroll
            for (int i = 0; i < kB; ++i) {
                const int q = min(q0 + i, ns - 1);
                ps[i] = p.rsum8[(int64_t)q * p.T + t];
#pragma unroll
                for (int m = 0; m < kM; ++m)
                    pl[m][i] = p.plog[((int64_t)q * p.T + t) * p.E_pad + min(lane + 64 * m, p.E_pad - 1)];
            }
#pragma unroll
            for (int i = 0; i < kB; ++i)
                if (q0 + i < ns) {
                    ss += ps[i];
#pragma unroll
                    for (int m = 0; m < kM; ++m) sum[m] += pl[m][i];
                }
        }
        const float c = (1.0f / sqrtf(ss / (float)p.H + p.eps)) * (1.0f / sqrtf((float)p.H));
        float v[kM];
#pragma unroll
        for (int m = 0; m < kM; ++m) {
            const int e = lane + 64 * m;
            float a = -INFINITY;
            if (e < E) {
                a = sum[m] * c;
                if (p.logit_bias) a += bias[m];
                if (p.logits_out) p.logits_out[(int64_t)t * E + e] = a;
                if (!(a == a)) a = -INFINITY;   // a NaN score ranks last; ids stay distinct
            }
            v[m] = a;
        }
        // top-k by keys that order like the scores (a NaN is -inf by now):
        // a bitwise search for the k-th largest key (compare, ballot and a
        // scalar count per bit), then the keys above it and the lowest
        // expert indices among those equal to it; finally each chosen
        // expert's rank among the chosen, equal scores by lower index.
        uint32_t key[kM];
#pragma unroll
        for (int m = 0; m < kM; ++m) {
            const uint32_t b = __float_as_uint(v[m] + 0.0f);   // -0 and +0 compare equal
            key[m] = lane + 64 * m < E ? ((b & 0x80000000u) ? ~b : (b | 0x80000000u)) : 0u;   // any score > 0
        }
        uint32_t thr = 0;
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t cand = thr | (1u << bit);
            int n = 0;
#pragma unroll
            for (int m = 0; m < kM; ++m) n += __popcll(__ballot(key[m] >= cand));
            if (n >= k) thr = cand;
        }
        int need = k;   // chosen: every key above thr, then the lowest-index keys equal to it
#pragma unroll
        for (int m = 0; m < kM; ++m) need -= __popcll(__ballot(key[m] > thr));
        bool sel[kM];
#pragma unroll
        for (int m = 0; m < kM; ++m) {
            const uint64_t eq = __ballot(key[m] == thr);
            const int below = __popcll(eq & ((1ull << lane) - 1ull));
            sel[m] = key[m] > thr || (key[m] == thr && below < need);
            need -= min(need, __popcll(eq));
        }
        int rank[kM];
#pragma unroll
        for (int m = 0; m < kM; ++m) rank[m] = 0;
#pragma unroll
        for (int m2 = 0; m2 < kM; ++m2) {
            uint64_t bits = __ballot(sel[m2]);
            while (bits) {
                const int l2 = __ffsll((unsigned long long)bits) - 1;
                bits &= bits - 1;
                const uint32_t k2 = (uint32_t)__builtin_amdgcn_readlane((int)key[m2], l2);
                const int e2 = l2 + 64 * m2;
#pragma unroll
                for (int m = 0; m < kM; ++m) {
                    const int e = lane + 64 * m;
                    rank[m] += sel[m] && (k2 > key[m] || (k2 == key[m] && e2 < e));
                }
            }
        }
        // lane r (r < k) takes the chosen expert of rank r
        int myid = 0;
        float myv = 0.f, v0 = 0.f;
#pragma unroll
        for (int m = 0; m < kM; ++m) {
            const uint64_t bits = __ballot(sel[m]);
            for (uint64_t b2 = bits; b2;) {
                const int l2 = __ffsll((unsigned long long)b2) - 1;
                b2 &= b2 - 1;
                const int r2 = __builtin_amdgcn_readlane(rank[m], l2);
                const float vv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v[m]), l2));
                if (lane == r2) {
                    myid = l2 + 64 * m;
                    myv = vv;
                }
                if (r2 == 0) v0 = vv;
            }
        }
        float ex = lane < k ? expf(myv - v0) : 0.f;
        const float den = wave_sum(ex);
        if (lane < k) {
            const float wt = ex / den * (p.pes ? p.pes[myid] : 1.0f);
            p.ids[t * k + lane] = myid;
            p.wts[t * k + lane] = wt;
            if (p.ids_out) p.ids_out[t * k + lane] = myid;
            if (p.w_out) p.w_out[t * k + lane] = wt;
        }
    }
}

// Sort every (token, slot) pair by expert and build the schedule: one
// workgroup.  grid 1, block 1024.
__global__ __launch_bounds__(1024) void k_sort(Plan p) {
    __shared__ int scan[16];
    __shared__ int ecount[kMaxExperts], efill[kMaxExperts], eoff[kMaxExperts];
    const int tid = threadIdx.x, E = p.E, k = p.k;
    const int P = p.T * k;
    // count the pairs of every expert (LDS atomics: many pairs of one
    // popular expert contend far less here than on one global address)
    for (int e = tid; e < E; e += 1024) ecount[e] = efill[e] = 0;
    __syncthreads();
    for (int q0 = tid; q0 < P; q0 += 1024 * 8) {
        int ex[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) ex[i] = p.ids[min(q0 + 1024 * i, P - 1)];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (q0 + 1024 * i < P) atomicAdd(&ecount[ex[i]], 1);
    }
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
    // the single GEMM launch's per-entry counts of finished gate/up items
    // and its queue of finished entries
    for (int e = tid; e < p.max_tiles; e += 1024) {
        p.gdone[e] = 0;
        p.gqueue[1 + e] = -1;
    }
    if (tid == 0) p.gqueue[0] = 0;
    __syncthreads();
    // positions within an expert's segment come from LDS atomics; the path
    // of a unit is chosen by its pair count, and every token is computed
    // on its own, so their order changes no result.  Eight pairs per thread
    // in flight at a time (the ids are read again: L2-resident now).
    for (int q0 = tid; q0 < P; q0 += 1024 * 8) {
        int ex[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) ex[i] = p.ids[min(q0 + 1024 * i, P - 1)];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int q = q0 + 1024 * i;
            if (q < P) {
                const int pos = eoff[ex[i]] + atomicAdd(&efill[ex[i]], 1);
                p.perm[pos] = q;
                p.inv[q] = pos;
            }
        }
    }
    build_schedule(p, cnt, off, scan);
}

// ---------------------------------------------------------------------------
// 4-bit codes on the matrix cores.
//
// codes8 turns the eight codes of a DEV_V1 word into eight fp16 operands
// with four AND-ORs under the fp16 exponent of 1024.0 (0x6400): columns
// c = 0, 1, 4, 5 of the eight come out as 1024 + q (the code in the low
// mantissa bits), columns 2, 3, 6, 7 as 1024 + 16 q (the code four bits
// higher).  Every activation operand of this path (x16, hg) holds the
// columns with (c & 2) != 0 divided by 16, an exact power-of-two step, so
// over one group of 64 columns, with a_c the stored activations,
//     sum_c code_c a_c = sum_c q_c x_c + 1024 sum_c a_c.
// The group-64 affine dequantisation w = s q + b then gives
//     sum_c w_c x_c = s (sum_c code_c a_c - 1024 sum_c a_c) + b sum_c x_c.
// Two ways through a work item use this:
//  * up to 32 tokens: the codes themselves are the B operand of the MFMAs
//    (D[token][row]); each group's accumulator starts at -1024 sum_c a_c of
//    its tokens and the group's scale and bias are applied once per output
//    in fp32 (one VALU operation per two weights for the codes instead of
//    five for dequantised fp16 weights);
//  * more tokens: the weights are dequantised to fp16 once per workgroup as
//    s (code - 1024) + b, with 16 b for the scaled columns (16 (s q + b)
//    rounds exactly as s q + b does), and shared by all token tiles.
// Per token and group the front kernel stores (sum_c x_c, -1024 sum_c a_c)
// of the layer input in xso; the gate/up kernel stores the same pair of
// every GeGLU row and 64-column group in hso for the down projection.
// (codes8 is in device.h.)

// fp16 scale and bias of a (scale | bias << 16) bf16 pair, and 16 * bias.
struct Sb16 {
    half2_t s, b, b16;
};
__device__ __forceinline__ Sb16 sb16(uint32_t pr) {
    const _Float16 s = (_Float16)bf16_lo(pr), b = (_Float16)bf16_hi(pr);
    const _Float16 b16 = b * (_Float16)16.0f;
    return {(half2_t){s, s}, (half2_t){b, b}, (half2_t){b16, b16}};
}

// Dequantised fp16 weights of one word, scaled columns times 16.
__device__ __forceinline__ half8_t dequant8s(uint32_t w, const Sb16& k) {
    const half8_t c = codes8(w);
    const half2_t off = {(_Float16)1024.0f, (_Float16)1024.0f};
    half8_t r;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const half2_t q = (half2_t){c[2 * m], c[2 * m + 1]} - off;
        const half2_t d = q * k.s + ((m & 1) ? k.b16 : k.b);
        r[2 * m] = d[0];
        r[2 * m + 1] = d[1];
    }
    return r;
}

// Stored activation and its group-sum pair of one GeGLU value h of column c.
__device__ __forceinline__ _Float16 act_store(_Float16 h, int c) { return (c & 2) ? h * (_Float16)0.0625f : h; }


// Grouped dequant-GEMM.  A work item is (64-row tile of one matrix, chunk
// of up to p.ntile = 128 tokens of one expert); for the down projection a
// workgroup takes kDnTiles consecutive row tiles of the item.  The shared
// expert takes part as n_vs virtual experts of I rows each (its gate/up
// rows, and the matching column slices of its down projection), applied to
// every token with weight 1, so it fills the machine together with the
// routed work.  The schedule puts the heaviest chunks first.
//
// Up to kSmallTokens tokens the loop is bound by load latency: the four
// waves split the column groups (gate/up) or own 16 rows each over an
// operand staged once (down), keep several groups of weights in flight and
// take no workgroup barrier in the loop.  With more tokens the token operand
// and the weights pass through a ring of LDS stages (below), and each
// dequantised weight fragment feeds the MFMAs of all the chunk's 16-token
// tiles (wave ms owns rows 16 ms .. 16 ms + 15 of each weight tile).
constexpr int kDnTiles = 4;                   // 64-row output tiles per down workgroup
// 64-row tiles of gate and of up per big gate/up workgroup: two for chunks
// of 128 tokens (the chunk's tokens are then read once per two row tiles),
// one for chunks of up to 64, whose calls have too few big units to fill
// the machine with half the workgroups
__host__ __device__ constexpr int gu_tiles(int MT) { return MT > 4 ? 2 : 1; }

// ---- units of more than kSmallTokens tokens: a ring of LDS stages (kRing),
// one 64-column group each, filled by direct global -> LDS loads
// (global_load_lds_dwordx4: lane i's 16 bytes land at the wave-uniform base
// in M0 plus 16 i).  A stage holds 2 NTT token fragments of 1 KB (fragment
// 2t + h: lane l's 16 bytes are token 16t + l % 16, columns 32h + 8 (l / 16)
// .. +7 of the group, the B operand of v_mfma_f32_16x16x32_f16 read at 16 l,
// which no two lanes of a pass share a bank for), then the NM weight tiles'
// codes (2 KB each) and their scale|bias words (256 B each, in a 1 KB
// slot).  The compiler does not see these loads, so their waits are
// explicit: stage g + kRing - 1 goes out after the barrier of stage g, and
// before that barrier each wave waits until only its loads of the later
// stages are outstanding (a fixed count per wave and stage; wave 0 also
// loads the scale|bias slot).  No other vector-memory operation is issued
// inside the loop.
// Stages of the ring: three, except for the down items of chunks of up to
// 64 tokens (four output tiles: 17 KB a stage), where two keep the single
// GEMM launch's LDS within three workgroups per CU.
__host__ __device__ constexpr int ring_depth(int MT, int NM) { return MT > 4 || NM <= 2 ? 3 : 2; }

__host__ __device__ constexpr int ring_stage_bytes(int MT, int NM) { return (2 * MT + 2 * NM + 1) * 1024; }

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// One direct load of 16 bytes per lane into LDS at lds_base + 16 lane.  The
// base goes in M0 as an input operand, so the compiler writes M0 itself;
// the load needs one wait state after that write.
__device__ __forceinline__ void lds_dma16(const void* g, uint32_t lds_base) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(g), "{m0}"(__builtin_amdgcn_readfirstlane(lds_base))
                 : "memory");
}

// Wait until at most N vector-memory operations of this wave are
// outstanding (expcnt and lgkmcnt left alone).
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt has six bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wait until the loads of the oldest stage in flight have landed, with
// `ahead` (0 .. kRing - 2) later stages of N loads each still outstanding.
template <int N, int kRing>
__device__ __forceinline__ void wait_stages(int ahead) {
    static_assert(kRing >= 2 && kRing <= 4, "ring of 2 to 4 stages");
    if (kRing > 3 && ahead >= 2)
        wait_vm<(kRing > 3 ? 2 : 0) * N>();
    else if (kRing > 2 && ahead >= 1)
        wait_vm<(kRing > 2 ? 1 : 0) * N>();
    else
        wait_vm<0>();
}

// Token fragment of this wave's i-th fragment load.
template <int NTT>
__device__ __forceinline__ int ring_frag(int wave, int i) { return min(wave + 4 * i, 2 * NTT - 1); }

// Weight tile m: row tile m % RT of matrix m / RT, at base + (m % RT)
// rstride + (m / RT) mstride; row tiles from nrt on repeat row tile nrt - 1
// (their results are dropped).
template <int RT>
__device__ __forceinline__ const uint8_t* ring_wtile(const uint8_t* base, int64_t rstride, int64_t mstride, int nrt,
                                                     int m) {
    return base + min(m % RT, nrt - 1) * rstride + (m / RT) * mstride;
}

// The loads of group g into the stage at LDS address st.  Wave w takes
// token fragments w, w + 4, ... (clamped: a repeated fragment rewrites the
// same bytes with the same values) and code kilobytes w, w + 4, ...
// xsrc[i]: this lane's source of fragment ring_frag(wave, i) in group 0;
// xoff: halves from there to the group's columns.
template <int NM, int NTT, int RT>
__device__ __forceinline__ void ring_issue(const uint8_t* base, int64_t rstride, int64_t mstride, int nrt, int g,
                                           const _Float16* const* xsrc, int64_t xoff, uint32_t st, int wave,
                                           int lane) {
#pragma unroll
    for (int i = 0; i < (NTT + 1) / 2; ++i) lds_dma16(xsrc[i] + xoff, st + ring_frag<NTT>(wave, i) * 1024);
    const uint32_t cw = st + 2 * NTT * 1024;
#pragma unroll
    for (int i = 0; i < NM / 2; ++i) {
        const int q = wave + 4 * i;
        lds_dma16(ring_wtile<RT>(base, rstride, mstride, nrt, q >> 1) + (int64_t)g * kBlk4 + (q & 1) * 1024 + lane * 16,
                  cw + q * 1024);
    }
    if (wave == 0) {
        const int m = min(lane >> 4, NM - 1);
        lds_dma16(ring_wtile<RT>(base, rstride, mstride, nrt, m) + (int64_t)g * kBlk4 + kCodes4 + (lane & 15) * 16,
                  cw + 2 * NM * 1024);
    }
}

// The multiplies of one stage: wave ms's weight rows 16 ms .. +15 of every
// tile (A operands dequantised once, fp16) times all 2 NTT token fragments.
template <int NM, int NTT, int MT>
__device__ __forceinline__ void ring_mma(const char* st, float4_t (*acc)[MT], int ms, int lane) {
    const char* cw = st + 2 * NTT * 1024;
    const char* sbw = cw + 2 * NM * 1024;
    half8_t a0[NM], a1[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        const uint2 c = *(const uint2*)(cw + m * 2048 + ((ms >> 1) * 64 + lane) * 16 + 8 * (ms & 1));
        const Sb16 k = sb16(*(const uint32_t*)(sbw + m * 256 + (lane & 15) * 16 + 4 * ms));
        a0[m] = dequant8s(c.x, k);
        a1[m] = dequant8s(c.y, k);
    }
#pragma unroll
    for (int t = 0; t < NTT; ++t) {
        const half8_t b0 = *(const half8_t*)(st + (2 * t) * 1024 + lane * 16);
        const half8_t b1 = *(const half8_t*)(st + (2 * t + 1) * 1024 + lane * 16);
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            acc[m][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0[m], b0, acc[m][t], 0, 0, 0);
            acc[m][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1[m], b1, acc[m][t], 0, 0, 0);
        }
    }
}

// NM weight tiles (ring_wtile) times the chunk's tokens over G column
// groups: acc[m][t] holds rows 16 ms + 4 (lane / 16) + i of tile m, token
// 16 t + lane % 16.  rows[n]: source row of chunk token n (n < count).
// lds: ring_depth(MT, NM) stages of ring_stage_bytes(MT, NM).  Starts and ends with the
// ring unused (the caller's LDS is free before and after).
template <int NM, int RT, int NTT, int MT>
__device__ __forceinline__ void ring_tile_n(const uint8_t* base, int64_t rstride, int64_t mstride, int nrt, int G,
                                            int ksplit, int64_t kjump, const _Float16* src, int64_t stride,
                                            const int* rows, int count, char* lds, float4_t (*acc)[MT]) {
    constexpr int kSt = ring_stage_bytes(MT, NM), kRing = ring_depth(MT, NM);
    constexpr int kOps = (NTT + 1) / 2 + NM / 2;   // loads per wave and stage (wave 0: one more)
    const int ms = wave_id(), lane = threadIdx.x & 63;
    const uint32_t l0 = lds_addr(lds);
    const _Float16* xsrc[(NTT + 1) / 2];
#pragma unroll
    for (int i = 0; i < (NTT + 1) / 2; ++i) {
        const int f = ring_frag<NTT>(ms, i), t = f >> 1, h = f & 1;
        xsrc[i] = src + (int64_t)rows[min(16 * t + (lane & 15), count - 1)] * stride + 32 * h + 8 * (lane >> 4);
    }
#pragma unroll
    for (int g = 0; g < kRing - 1; ++g)
        if (g < G)
            ring_issue<NM, NTT, RT>(base, rstride, mstride, nrt, g, xsrc, g * 64 + (g / ksplit) * kjump, l0 + g * kSt,
                                    ms, lane);
    for (int g = 0; g < G; ++g) {
        // outstanding: stages g .. g + ahead; wait for stage g alone
        const int ahead = min(kRing - 2, G - 1 - g);
        if (ms == 0)
            wait_stages<kOps + 1, kRing>(ahead);
        else
            wait_stages<kOps, kRing>(ahead);
        __syncthreads();
        if (g + kRing - 1 < G) {
            const int gi = g + kRing - 1;
            ring_issue<NM, NTT, RT>(base, rstride, mstride, nrt, gi, xsrc, gi * 64 + (gi / ksplit) * kjump,
                                    l0 + (gi % kRing) * kSt, ms, lane);
        }
        ring_mma<NM, NTT, MT>(lds + (g % kRing) * kSt, acc, ms, lane);
    }
    __syncthreads();
}

template <int NM, int RT, int MT>
__device__ __forceinline__ void ring_tile(const uint8_t* base, int64_t rstride, int64_t mstride, int nrt, int G,
                                          int ksplit, int64_t kjump, const _Float16* src, int64_t stride,
                                          const int* rows, int count, char* lds, float4_t (*acc)[MT]) {
#define MQ_RING(N) \
    ring_tile_n<NM, RT, N, MT>(base, rstride, mstride, nrt, G, ksplit, kjump, src, stride, rows, count, lds, acc)
    switch ((count + 15) / 16) {
        case 1: MQ_RING(1); break;
        case 2: MQ_RING(2); break;
        case 3: MQ_RING(3); break;
        default:
            if constexpr (MT <= 4) {
                MQ_RING(4);
            } else {
                switch ((count + 15) / 16) {
                    case 4: MQ_RING(4); break;
                    case 5: MQ_RING(5); break;
                    case 6: MQ_RING(6); break;
                    case 7: MQ_RING(7); break;
                    default: MQ_RING(8); break;
                }
            }
    }
#undef MQ_RING
}

// The work item of this workgroup: a schedule entry (chunk) and a row tile
// (gate/up) or a run of kDnTiles row tiles (down).  Experts E .. E+n_vs-1
// are the shared expert's virtual experts.
struct Item {
    int rt;             // row tile (gate/up) or first row tile (down)
    int ntiles;         // 64-row tiles of the item's matrices
    int big;            // the unit takes the dequantised-weight path
    int ntt;            // 16-token tiles of the chunk
    int count;          // tokens of the chunk
    int pos0;           // row of chunk token 0 in hg / ysort
    int shared;         // 1 for a virtual shared expert
    int tok0;           // shared: first token of the chunk
    int G;              // column groups of the operand
    int64_t rstride;    // bytes from one 64-row tile of the matrices to the next
    const uint8_t* w[2];
    int ksplit;         // operand rows jump by kjump halves every ksplit column groups
    int64_t kjump;      //   (the shared expert's down over all its columns), else ksplit = G
    int e;              // schedule entry
    int ngu;            // gate/up workgroups of the entry (row tiles of its gate and up)
};

// Grid position of this workgroup in a grid (nx, ny) with ny a multiple of
// 8.  Workgroups go to the eight XCDs round robin by linear index, so XCD x
// runs linear indices x, x + 8, ...; its j-th one takes chunk
// 8 (j / nx) + x and row position j % nx.  Every row position of a chunk
// then runs on one XCD, whose L2 serves the chunk's token rows to all of
// them, and the chunks keep their heaviest-first order across the XCDs.
// (A bijection whatever the dispatch order: only speed depends on it.)
struct GridPos {
    int rx, chunk;
};
__device__ __forceinline__ GridPos grid_pos_at(int L, int nx) {
    const int j = L >> 3;
    return {j % nx, (j / nx) * 8 + (L & 7)};
}

// Position in a launch of one kind of item: L (linear index) < 0 takes the
// two-dimensional grid of the launch.
__device__ __forceinline__ GridPos grid_pos(int L, int nx) {
    return L < 0 ? grid_pos_at(blockIdx.y * gridDim.x + blockIdx.x, gridDim.x) : grid_pos_at(L, nx);
}

// The matrices of row position rx of schedule entry e and its tokens, from
// the entry alone.  Returns false when the workgroup has nothing to do.
__device__ __forceinline__ bool gg_item_at(const Plan& p, bool down, Item* it, int e, int rx) {
    const int rt = down ? rx * kDnTiles : rx;
    it->rt = rt;
    it->e = e;
    const int2 sc = p.sched[e];
    const int ex = sc.x >> 16, c = sc.x & 0xFF;
    it->big = (sc.x >> 12) & 1;
    it->ntt = (sc.x >> 8) & 0xF;
    it->pos0 = sc.y & 0xFFFFFF;
    it->count = (int)((uint32_t)sc.y >> 24);
    it->tok0 = c * p.ntile;
    it->kjump = 0;
    if (ex < p.E) {
        it->shared = 0;
        it->ngu = p.I / 64;
        const uint8_t* base = p.pool_base + (int64_t)ex * p.expert_stride;
        it->ntiles = down ? p.H / 64 : p.I / 64;
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
        it->ngu = min(p.I, p.Is - j * p.I) / 64;
        it->ntiles = down ? p.H / 64 : min(p.I, p.Is - j * p.I) / 64;
        if (down && p.n_vs_dn == 1 && p.n_vs > 1) {
            // the first virtual expert's item takes all G_s groups: its
            // operand rows continue T rows further on every G_I groups
            if (j > 0) return false;
            it->G = p.G_s;
            it->rstride = (int64_t)p.G_s * kBlk4;
            it->w[0] = it->w[1] = p.sh_down + (int64_t)rt * p.G_s * kBlk4;
            it->ksplit = p.G_I;
            it->kjump = (int64_t)p.T * p.I - p.I;
            return true;
        } else if (down) {
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
    it->ksplit = it->G;
    return true;
}

// The item of this workgroup's grid position (L, nx: see grid_pos).
__device__ __forceinline__ bool gg_item(const Plan& p, bool down, Item* it, int L = -1, int nx = 0) {
    const GridPos gp = grid_pos(L, nx);
    const int ns = p.nsched[0];
    if (gp.chunk >= ns) return false;
    // gate/up takes the entries in order; down takes the code-operand ones
    // first (128-token chunks), whose workgroups stage the chunk and take
    // longer there
    const int nb = p.nsched[1];
    const int e = !down ? gp.chunk : (gp.chunk < ns - nb ? nb + gp.chunk : gp.chunk - (ns - nb));
    return gg_item_at(p, down, it, e, gp.rx);
}

// Token of chunk position n (clamped to the chunk).
__device__ __forceinline__ int item_token(const Plan& p, const Item& it, int n) {
    n = min(n, it.count - 1);
    return it.shared ? it.tok0 + n : p.perm[it.pos0 + n] / p.k;
}

// LDS copies tsum[g][n], tneg[g][n] (pitch 32) of the (sum, -1024 sum)
// pairs src[row][g] (ld pairs per row) of chunk slots n < nslot, for G
// groups; thread tid takes slot tid % 32 and groups tid / 32 + 8 i, with
// the loads of six groups in flight.  No barrier inside.
template <bool AGENT = false>
__device__ __forceinline__ void stage_sums(const float2* src, int ld, int row, int G, int nslot, float* tsum,
                                           float* tneg) {
    const int n = threadIdx.x & 31;
    if (n >= nslot) return;
    constexpr int kB = 6;
    for (int g0 = threadIdx.x >> 5; g0 < G; g0 += 8 * kB) {
        float2 v[kB];
#pragma unroll
        for (int i = 0; i < kB; ++i) {
            const float2* a = src + (int64_t)row * ld + min(g0 + 8 * i, G - 1);
            if constexpr (AGENT)
                v[i] = __builtin_bit_cast(float2, __hip_atomic_load((const uint64_t*)a, __ATOMIC_RELAXED,
                                                                    __HIP_MEMORY_SCOPE_AGENT));
            else
                v[i] = *a;
        }
#pragma unroll
        for (int i = 0; i < kB; ++i)
            if (g0 + 8 * i < G) {
                tsum[(g0 + 8 * i) * 32 + n] = v[i].x;
                tneg[(g0 + 8 * i) * 32 + n] = v[i].y;
            }
    }
}

// GeGLU rows and their group sums.  With ONE (the down items run in the same
// launch, on any XCD) they are stored at agent scope: such a store has
// passed this XCD's L2 once it has completed, and gu_done waits for that.
template <bool ONE>
__device__ __forceinline__ void put_h(_Float16* dst, _Float16 v) {
    if constexpr (ONE)
        __hip_atomic_store((uint16_t*)dst, __builtin_bit_cast(uint16_t, v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
        *dst = v;
}

// Four adjacent GeGLU values (dst 8-byte aligned).
template <bool ONE>
__device__ __forceinline__ void put_h4(_Float16* dst, const _Float16* v) {
    if constexpr (ONE) {
        const uint64_t w = (uint64_t)__builtin_bit_cast(uint16_t, v[0]) |
                           ((uint64_t)__builtin_bit_cast(uint16_t, v[1]) << 16) |
                           ((uint64_t)__builtin_bit_cast(uint16_t, v[2]) << 32) |
                           ((uint64_t)__builtin_bit_cast(uint16_t, v[3]) << 48);
        __hip_atomic_store((uint64_t*)dst, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[i] = v[i];
    }
}

// The (sum, -1024 sum) pair of the chunk's GeGLU rows over the tile's 64
// columns: part[w][n] holds wave w's share for chunk token n.
template <bool ONE>
__device__ __forceinline__ void write_hso(const Plan& p, const Item& it, int rt, const float2 (*part)[128]) {
    const int n = threadIdx.x;
    if (n < it.count) {
        float2 v = part[0][n];
#pragma unroll
        for (int w = 1; w < 4; ++w) {
            v.x += part[w][n].x;
            v.y += part[w][n].y;
        }
        float2* dst = (float2*)p.hso + (int64_t)(it.pos0 + n) * p.G_I + rt;
        if constexpr (ONE)
            __hip_atomic_store((uint64_t*)dst, __builtin_bit_cast(uint64_t, v), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        else
            *dst = v;
    }
}

// One launch: the item's GeGLU rows are written; count it for its entry,
// and the last of the entry's gate/up workgroups appends the entry to the
// queue of finished entries.  Each wave first waits for its own stores
// (they complete in order with its loads), so the count follows every store
// of the workgroup, and the append every store of the entry.
template <bool ONE>
__device__ __forceinline__ void gu_done(const Plan& p, const Item& it) {
    if constexpr (ONE) {
        wait_vm<0>();
        __syncthreads();
        if (threadIdx.x == 0 &&
            __hip_atomic_fetch_add(p.gdone + it.e, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == it.ngu - 1) {
            const int slot = __hip_atomic_fetch_add(p.gqueue, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(p.gqueue + 1 + slot, it.e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// One launch: the down items take the entries in the order their gate/up
// items finish.  Slot q of the queue (grid position q, see grid_pos) waits
// for the q-th finished entry (bounded: a give-up sets kErrWait and the
// workgroup does nothing).
constexpr int kGuSpins = 1 << 16;
__device__ __forceinline__ bool gg_item_ready(const Plan& p, Item* it, int L, int nx) {
    __shared__ int s_entry;
    const GridPos gp = grid_pos_at(L, nx);
    if (gp.chunk >= p.nsched[0]) return false;
    if (threadIdx.x == 0) {
        int e, n = 0;
        while ((e = __hip_atomic_load(p.gqueue + 1 + gp.chunk, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) < 0) {
            if (++n > kGuSpins) {
                atomicOr(p.f_err, kErrWait);
                break;
            }
            __builtin_amdgcn_s_sleep(8);
        }
        s_entry = e;
    }
    __syncthreads();
    const int e = s_entry;
    return e >= 0 && gg_item_at(p, true, it, e, gp.rx);
}

// ---- gate/up, up to 32 tokens: codes as the B operand (D[token][row]); the
// four waves split the column groups (wave w takes groups w, w+4, ...) over
// all 64 rows of the tile, each loading its own token fragments straight
// into registers; the partial sums meet in LDS at the end.
struct GuW {
    u32x4_t c[2][2];     // [matrix][row-block pair]: codes, lane's 16 bytes of each half block
    u32x4_t s[2];        // [matrix]: scale|bias of row lane % 16 in each of the four row blocks
};
template <int NTT>
struct GuX {
    half8_t x[NTT][2];   // A operand: token 16 t + lane % 16, columns 8 (lane / 16) .. +7 and 32 + that
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

// out[m][rb][t][i]: token 16 t + 4 (lane / 16) + i, row 16 rb + lane % 16 of
// matrix m.  tsum / tneg: the chunk's staged group constants.  A group past
// the wave's last (valid false) re-reads group G-1 and weighs zero, which
// keeps the loop body free of branches: a conditional multiply splits the
// live ranges of the prefetch buffers, and the copies the compiler then
// makes wait for every load in flight.
template <int NTT>
__device__ __forceinline__ void gu_mma(const GuW& L, const GuX<NTT>& X, const float* tsum, const float* tneg, int g,
                                       bool valid, float4_t (*out)[4][NTT], int lane) {
    float4_t neg[NTT], sum[NTT];
#pragma unroll
    for (int t = 0; t < NTT; ++t) {
        neg[t] = *(const float4_t*)&tneg[g * 32 + 16 * t + 4 * (lane >> 4)];
        sum[t] = *(const float4_t*)&tsum[g * 32 + 16 * t + 4 * (lane >> 4)];
    }
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
            const uint32_t pr = valid ? L.s[m][rb] : 0u;
            const float s = bf16_lo(pr), b = bf16_hi(pr);
            const half8_t q0 = codes8(L.c[m][rb >> 1][2 * (rb & 1)]);
            const half8_t q1 = codes8(L.c[m][rb >> 1][2 * (rb & 1) + 1]);
#pragma unroll
            for (int t = 0; t < NTT; ++t) {
                float4_t a = __builtin_amdgcn_mfma_f32_16x16x32_f16(X.x[t][0], q0, neg[t], 0, 0, 0);
                a = __builtin_amdgcn_mfma_f32_16x16x32_f16(X.x[t][1], q1, a, 0, 0, 0);
#pragma unroll
                for (int i = 0; i < 4; ++i) out[m][rb][t][i] = fmaf(s, a[i], fmaf(b, sum[t][i], out[m][rb][t][i]));
            }
        }
}

typedef float4_t GuRed[4][3][2][64];   // [row block][other wave][matrix][lane], one token tile

// The wave's groups are w + 4 j, j < nj; WA and WB hold the weights of
// j = 0 and 1, loaded before the token bookkeeping.  sched_barrier pins each
// refill right after the multiply that frees its registers, so the next
// groups stay in flight behind the one in use: two of them for one token
// tile, one for two (register budget).  Prefetch past the end re-reads the
// last group; the loops have one exit, a multiply past the end weighs zero.
// tok0 = item_token(lane % 16), tok_s = item_token(threadIdx.x % 32), looked
// up by the caller before the first weights.
template <int NTT, bool ONE>
__device__ __forceinline__ void gu_small_n(const Plan& p, const Item& it, GuW& WA, GuW& WB, char* lds,
                                           float2 (*hpart)[128], int tok0, int tok_s) {
    const int w = wave_id(), lane = threadIdx.x & 63;
    const _Float16* x16 = p.x16;
    float* tsum = (float*)lds;            // [G][32]
    float* tneg = tsum + it.G * 32;       // [G][32]
    int xr[NTT];
#pragma unroll
    for (int t = 0; t < NTT; ++t)
        xr[t] = (t == 0 ? tok0 : item_token(p, it, 16 * t + (lane & 15))) * p.H + 8 * (lane >> 4);
    const int G = it.G, nj = (G - w + 3) / 4;
    auto grp = [&](int j) { return min(w + 4 * j, G - 1); };
    const uint8_t *w0 = it.w[0], *w1 = it.w[1];
    GuX<NTT> XA, XB;
    gu_xload(XA, x16, xr, grp(0));
    gu_xload(XB, x16, xr, grp(1));
    stage_sums((const float2*)p.xso, p.G_H, tok_s, G, 16 * NTT, tsum, tneg);
    float4_t acc[2][4][NTT];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
            for (int t = 0; t < NTT; ++t) acc[m][rb][t] = (float4_t){0.f, 0.f, 0.f, 0.f};
    __syncthreads();
    if constexpr (NTT >= 2) {
        for (int j = 0; j < nj; j += 2) {
            __builtin_amdgcn_sched_barrier(0);
            gu_mma<NTT>(WA, XA, tsum, tneg, grp(j), true, acc, lane);
            __builtin_amdgcn_sched_barrier(0);
            gu_wload(WA, w0, w1, grp(j + 2), lane);
            gu_xload(XA, x16, xr, grp(j + 2));
            __builtin_amdgcn_sched_barrier(0);
            gu_mma<NTT>(WB, XB, tsum, tneg, grp(j + 1), j + 1 < nj, acc, lane);
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
            gu_mma<NTT>(WA, XA, tsum, tneg, grp(j), true, acc, lane);
            __builtin_amdgcn_sched_barrier(0);
            gu_wload(WA, w0, w1, grp(j + 3), lane);
            gu_xload(XA, x16, xr, grp(j + 3));
            __builtin_amdgcn_sched_barrier(0);
            gu_mma<NTT>(WB, XB, tsum, tneg, grp(j + 1), j + 1 < nj, acc, lane);
            __builtin_amdgcn_sched_barrier(0);
            gu_wload(WB, w0, w1, grp(j + 4), lane);
            gu_xload(XB, x16, xr, grp(j + 4));
            __builtin_amdgcn_sched_barrier(0);
            gu_mma<NTT>(WC, XC, tsum, tneg, grp(j + 2), j + 2 < nj, acc, lane);
            __builtin_amdgcn_sched_barrier(0);
            gu_wload(WC, w0, w1, grp(j + 5), lane);
            gu_xload(XC, x16, xr, grp(j + 5));
        }
    }
    // wave w sums row block w over the four waves (fixed order: own, then
    // the others by wave), one token tile at a time; the buffer takes the
    // place of the staged constants, so the first barrier also waits for
    // every wave's last multiply
    GuRed& red = *(GuRed*)lds;
    const int c = it.rt * 64 + 16 * w + (lane & 15);   // GeGLU column of this lane
#pragma unroll
    for (int t = 0; t < NTT; ++t) {
        __syncthreads();
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
            if (rb != w)
#pragma unroll
                for (int m = 0; m < 2; ++m) red[rb][w < rb ? w : w - 1][m][lane] = acc[m][rb][t];
        __syncthreads();
        float4_t v[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            float4_t a = w == 0 ? acc[m][0][t] : w == 1 ? acc[m][1][t] : w == 2 ? acc[m][2][t] : acc[m][3][t];
#pragma unroll
            for (int q = 0; q < 3; ++q) a += red[w][q][m][lane];
            v[m] = a;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int n = 16 * t + 4 * (lane >> 4) + i;
            const _Float16 h = (_Float16)(gelu_tanh(v[0][i]) * v[1][i]);
            const _Float16 a = act_store(h, c);
            flag_error(p.f_err, n < it.count && f16_bad(h), kErrRange);
            if (n < it.count) put_h<ONE>(p.hg + (int64_t)(it.pos0 + n) * p.I + c, a);
            const float hs = sum16((float)h), hn = sum16(-1024.0f * (float)a);
            if ((lane & 15) == 0) hpart[w][n] = make_float2(hs, hn);
        }
    }
    __syncthreads();
    write_hso<ONE>(p, it, it.rt, hpart);
    gu_done<ONE>(p, it);
}

// ---- gate/up, units of more than kSmallTokens tokens: gu_tiles row tiles of
// gate and of up over the ring, so each staged token fragment feeds
// 4 gu_tiles multiplies.
template <int MT, bool ONE>
__device__ __forceinline__ void gu_big(const Plan& p, const Item& it, char* lds, int* rows, float2 (*hpart)[128]) {
    constexpr int kGuTiles = gu_tiles(MT);
    const int wave = wave_id(), lane = threadIdx.x & 63;
    if ((int)threadIdx.x < it.count) rows[threadIdx.x] = item_token(p, it, threadIdx.x);
    __syncthreads();
    const int nrt = min(kGuTiles, it.ntiles - it.rt);
    float4_t acc[2 * kGuTiles][MT];
#pragma unroll
    for (int m = 0; m < 2 * kGuTiles; ++m)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[m][t] = (float4_t){0.f, 0.f, 0.f, 0.f};
    ring_tile<2 * kGuTiles, kGuTiles, MT>(it.w[0], it.rstride, it.w[1] - it.w[0], nrt, it.G, it.ksplit, it.kjump,
                                          p.x16, p.H, rows, it.count, lds, acc);
#pragma unroll
    for (int u = 0; u < kGuTiles; ++u) {
        if (u >= nrt) break;
        // rows r0 + i of the GeGLU output; (r0 + i) & 2 == i & 2
        const int r0 = (it.rt + u) * 64 + 16 * wave + 4 * (lane >> 4);
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            const int n = 16 * t + (lane & 15);
            _Float16 h[4], a[4];
            float hs = 0.f, hn = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                h[i] = (_Float16)(gelu_tanh(acc[u][t][i]) * acc[kGuTiles + u][t][i]);
                a[i] = act_store(h[i], i);
                hs += (float)h[i];
                hn += -1024.0f * (float)a[i];
            }
            flag_error(p.f_err, n < it.count && (f16_bad(h[0]) || f16_bad(h[1]) || f16_bad(h[2]) || f16_bad(h[3])),
                       kErrRange);
            if (n < it.count) put_h4<ONE>(p.hg + (int64_t)(it.pos0 + n) * p.I + r0, a);
            hs = sum_kb(hs);
            hn = sum_kb(hn);
            if (lane < 16) hpart[wave][n] = make_float2(hs, hn);
        }
        __syncthreads();
        write_hso<ONE>(p, it, it.rt + u, hpart);
        __syncthreads();
    }
    gu_done<ONE>(p, it);
}

// Gate/up + GeGLU: hg[pos] = gelu(gate x) * (up x) in fp16 (scaled
// columns divided by 16), hso[pos][tile] its group sums.  MT: most 16-token
// tiles of a chunk; chunks of up to 64 tokens leave room for three waves per
// SIMD.  grid (I / 64, max_tiles), block 256, dynamic LDS gu_lds_bytes.
// (L, nx: see grid_pos; ONE: see put_h.)
template <int MT, bool ONE>
__device__ __forceinline__ void gu_item(const Plan& p, char* lds, float2 (*hpart)[128], int* rows, int L, int nx) {
    static_assert(!ONE || gu_tiles(MT) == 1, "one launch: every row tile of an entry is a workgroup that counts");
    Item it;
    if (!gg_item(p, false, &it, L, nx)) return;
    const int w = wave_id(), lane = threadIdx.x & 63;
    if (it.big) {
        // gu_tiles row tiles per workgroup: the others of the run have none
        if (it.rt % gu_tiles(MT) == 0) gu_big<MT, ONE>(p, it, lds, rows, hpart);
        return;
    }
    // the chunk's token lookups first, then the first weights, in flight
    // while the token rows arrive: loads complete in issue order, so lookups
    // issued behind the weights would wait for them
    const int tok0 = item_token(p, it, lane & 15), tok_s = item_token(p, it, threadIdx.x & 31);
    __builtin_amdgcn_sched_barrier(0);
    GuW WA, WB;
    gu_wload(WA, it.w[0], it.w[1], min(w, it.G - 1), lane);
    gu_wload(WB, it.w[0], it.w[1], min(w + 4, it.G - 1), lane);
    gu_small_n<1, ONE>(p, it, WA, WB, lds, hpart, tok0, tok_s);
}

template <int MT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(MT <= 4 ? 3 : 2))) void k_gu(Plan p) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    __shared__ float2 hpart[4][128];
    __shared__ int rows[128];
    gu_item<MT, false>(p, lds, hpart, rows, -1, 0);
}

// ---- down, up to 32 tokens: the chunk's GeGLU rows and group constants
// are staged in LDS once; the workgroup then runs over its kDnTiles output
// tiles with no further barrier, each wave keeping three batches of four
// column groups of weights in flight.
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

// Batch of groups g0 .. g0+kSmKB-1; a group past the end (zero scale and
// bias) reads the staged columns and constants of group G-1, which hold
// finite values.  acc[t][i]: token 16 t + 4 (lane / 16) + i, row lane % 16
// of the wave's row block.
template <int NTT>
__device__ __forceinline__ void dn_mma(const DnLoads& L, const _Float16* hs, int pitch, const float* tsum,
                                       const float* tneg, int g0, int G, float4_t* acc, int lane) {
    const int kb = lane >> 4, n = lane & 15;
#pragma unroll
    for (int u = 0; u < kSmKB; ++u) {
        const int g = min(g0 + u, G - 1);
        const uint32_t pr = g0 + u < G ? L.s[u] : 0u;
        const float s = bf16_lo(pr), b = bf16_hi(pr);
        const half8_t q0 = codes8(L.c[u].x), q1 = codes8(L.c[u].y);
#pragma unroll
        for (int t = 0; t < NTT; ++t) {
            const _Float16* row = hs + (16 * t + n) * pitch + g * 64 + 8 * kb;
            const float4_t neg = *(const float4_t*)&tneg[g * 32 + 16 * t + 4 * kb];
            const float4_t sum = *(const float4_t*)&tsum[g * 32 + 16 * t + 4 * kb];
            float4_t a = __builtin_amdgcn_mfma_f32_16x16x32_f16(*(const half8_t*)row, q0, neg, 0, 0, 0);
            a = __builtin_amdgcn_mfma_f32_16x16x32_f16(*(const half8_t*)(row + 32), q1, a, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[t][i] = fmaf(s, a[i], fmaf(b, sum[i], acc[t][i]));
        }
    }
}

// A, B, C hold batches 0, 1, 2, loaded before the chunk was staged.
template <int NTT>
__device__ __forceinline__ void dn_small_n(const Plan& p, const Item& it, int rt0, int nrt, const _Float16* hs,
                                           int pitch, const float* tsum, const float* tneg, const float* wrow,
                                           const uint8_t* wb, const uint8_t* sb, DnLoads& A, DnLoads& B,
                                           DnLoads& C) {
    const int ms = wave_id(), lane = threadIdx.x & 63;
    const int G = it.G, nb = (G + kSmKB - 1) / kSmKB, nq = nrt * nb;
    float4_t acc[NTT];
#pragma unroll
    for (int t = 0; t < NTT; ++t) acc[t] = (float4_t){0.f, 0.f, 0.f, 0.f};
    auto finish = [&](int q) {   // after batch q: store the tile if it was its last batch
        const int r = q / nb;
        if (q - r * nb != nb - 1) return;
        const int row = (rt0 + r) * 64 + 16 * ms + (lane & 15);
#pragma unroll
        for (int t = 0; t < NTT; ++t) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int n = 16 * t + 4 * (lane >> 4) + i;
                if (n < it.count) p.ysort[(int64_t)(it.pos0 + n) * p.H + row] = wrow[n] * acc[t][i];
            }
            acc[t] = (float4_t){0.f, 0.f, 0.f, 0.f};
        }
    };
    auto grp0 = [&](int q) { return (q % nb) * kSmKB; };
    // one exit: batches past the end skip their multiply
    for (int q = 0; q < nq; q += 3) {
        __builtin_amdgcn_sched_barrier(0);
        dn_mma<NTT>(A, hs, pitch, tsum, tneg, grp0(q), G, acc, lane);
        finish(q);
        __builtin_amdgcn_sched_barrier(0);
        dn_load(A, wb, sb, it.rstride, q + 3, nq, nb, G);
        __builtin_amdgcn_sched_barrier(0);
        if (q + 1 < nq) {
            dn_mma<NTT>(B, hs, pitch, tsum, tneg, grp0(q + 1), G, acc, lane);
            finish(q + 1);
        }
        __builtin_amdgcn_sched_barrier(0);
        dn_load(B, wb, sb, it.rstride, q + 4, nq, nb, G);
        __builtin_amdgcn_sched_barrier(0);
        if (q + 2 < nq) {
            dn_mma<NTT>(C, hs, pitch, tsum, tneg, grp0(q + 2), G, acc, lane);
            finish(q + 2);
        }
        __builtin_amdgcn_sched_barrier(0);
        dn_load(C, wb, sb, it.rstride, q + 5, nq, nb, G);
    }
}

// ---- down, more than kSmallTokens tokens: the kDnTiles output tiles of the
// workgroup at once over the ring, so each staged token fragment feeds
// 2 kDnTiles multiplies.
template <int MT>
__device__ __forceinline__ void dn_big(const Plan& p, const Item& it, int rt0, int nrt, char* lds, int* rows,
                                       const float* wrow) {
    const int wave = wave_id(), lane = threadIdx.x & 63;
    float4_t acc[kDnTiles][MT];
#pragma unroll
    for (int m = 0; m < kDnTiles; ++m)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[m][t] = (float4_t){0.f, 0.f, 0.f, 0.f};
    ring_tile<kDnTiles, kDnTiles, MT>(it.w[0], it.rstride, 0, nrt, it.G, it.ksplit, it.kjump, p.hg, p.I, rows,
                                      it.count, lds, acc);
#pragma unroll
    for (int m = 0; m < kDnTiles; ++m) {
        if (m >= nrt) break;
        const int r0 = (rt0 + m) * 64 + 16 * wave + 4 * (lane >> 4);
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            const int n = 16 * t + (lane & 15);
            if (n < it.count) {
                const float wt = wrow[n];
                float* dst = p.ysort + (int64_t)(it.pos0 + n) * p.H + r0;
#pragma unroll
                for (int i = 0; i < 4; ++i) dst[i] = wt * acc[m][t][i];
            }
        }
    }
}

// Dynamic LDS of k_dn: the small path's staged chunk (kSmallTokens rows of
// I + 8 halves, then the group constants) or the big path's batch.
__host__ __device__ constexpr size_t dn_small_hs_bytes(int I) { return (size_t)kSmallTokens * (I + 8) * 2; }
size_t dn_lds_bytes(int I, int MT) {
    const size_t small = dn_small_hs_bytes(I) + (size_t)2 * (I / 64) * 32 * 4;
    const size_t big = (size_t)ring_depth(MT, kDnTiles) * ring_stage_bytes(MT, kDnTiles);
    return small > big ? small : big;
}

// Down projection: ysort[pos] = w_pair * (W_down . h), weight 1 for the
// shared expert's slices.  grid (ceil(H / 64 / kDnTiles), max_tiles), block
// 256, dynamic LDS dn_lds_bytes(I, MT).
template <int MT, bool ONE>
__device__ __forceinline__ void dn_item(const Plan& p, _Float16* hs, float* wrow, int* rows, int L, int nx) {
    Item it;
    if constexpr (ONE) {
        if (!gg_item_ready(p, &it, L, nx)) return;
    } else if (!gg_item(p, true, &it, L, nx)) {
        return;
    }
    const int rt0 = it.rt, nrt = min(kDnTiles, p.H / 64 - rt0);
    auto token_rows = [&]() {
        if ((int)threadIdx.x < it.count) {
            wrow[threadIdx.x] = it.shared ? 1.f : p.wts[p.perm[it.pos0 + threadIdx.x]];
            rows[threadIdx.x] = it.pos0 + threadIdx.x;
        }
    };
    if (it.big) {
        token_rows();
        __syncthreads();
        dn_big<MT>(p, it, rt0, nrt, (char*)hs, rows, wrow);
        return;
    }
    const int ms = wave_id(), lane = threadIdx.x & 63;
    const int nb = (it.G + kSmKB - 1) / kSmKB, nq = nrt * nb;
    const uint8_t* wb = it.w[0] + ((ms >> 1) * 64 + lane) * 16 + 8 * (ms & 1);
    const uint8_t* sb = it.w[0] + kCodes4 + (lane & 15) * 16 + 4 * ms;
    // stage the chunk: rows past it repeat its last row; columns past G
    // groups are never read.  The group constants and the first batch of
    // the chunk go out before the first weights, so that waiting for them
    // does not wait for the weights too (loads complete in issue order);
    // six pieces per thread at a time.
    const int pitch = p.I + 8;
    const int per = it.G * 8;   // 16-byte pieces per row
    const int nrow = it.ntt * 16;
    constexpr int kSt = 6;
    const int total = nrow * per;
    float* tsum = (float*)((char*)hs + dn_small_hs_bytes(p.I));
    float* tneg = tsum + it.G * 32;
    stage_sums<ONE>((const float2*)p.hso, p.G_I, it.pos0 + min((int)(threadIdx.x & 31), it.count - 1), it.G, nrow,
                    tsum, tneg);
    auto stage_load = [&](u32x4_t* v, int c0) {
#pragma unroll
        for (int i = 0; i < kSt; ++i) {
            const int c = min(c0 + 256 * i, total - 1), n = c / per, q = c - n * per;
            v[i] = *(const u32x4_t*)(p.hg + (int64_t)(it.pos0 + min(n, it.count - 1)) * p.I + q * 8);
        }
    };
    auto stage_store = [&](const u32x4_t* v, int c0) {
#pragma unroll
        for (int i = 0; i < kSt; ++i) {
            const int c = c0 + 256 * i, n = c / per, q = c - n * per;
            if (c < total) *(u32x4_t*)&hs[n * pitch + q * 8] = v[i];
        }
    };
    // the first batch (every thread loads, clamped), then the first weights
    // (every thread), then the stores and any further batches
    DnLoads A, B, C;
    {
        u32x4_t v[kSt];
        stage_load(v, threadIdx.x);
        dn_load(A, wb, sb, it.rstride, 0, nq, nb, it.G);
        dn_load(B, wb, sb, it.rstride, 1, nq, nb, it.G);
        dn_load(C, wb, sb, it.rstride, 2, nq, nb, it.G);
        stage_store(v, threadIdx.x);
    }
    for (int c0 = threadIdx.x + 256 * kSt; c0 < total; c0 += 256 * kSt) {
        u32x4_t v[kSt];
        stage_load(v, c0);
        stage_store(v, c0);
    }
    token_rows();
    __syncthreads();
    dn_small_n<1>(p, it, rt0, nrt, hs, pitch, tsum, tneg, wrow, wb, sb, A, B, C);
}

template <int MT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(MT <= 4 ? 3 : 2))) void k_dn(Plan p) {
    extern __shared__ __attribute__((aligned(16))) _Float16 hs[];
    __shared__ float wrow[128];
    __shared__ int rows[128];
    dn_item<MT, false>(p, hs, wrow, rows, -1, 0);
}

// Gate/up and down items in one launch (chunks of up to 64 tokens): the
// first nxg ns8 linear indices run the gate/up items of the ns schedule
// entries (ns8: ns rounded up to 8; grid position over nxg row positions),
// the next nxd ny the down items (nxd), which take the entries in the order
// their gate/up items finish (gu_done, gg_item_ready), and the rest (the
// gate/up positions of entries the schedule did not fill) have nothing to
// do: they come last, so that workgroups with work start first.
// Workgroups go to the XCDs round robin by index and each XCD starts its
// own in index order, so once a down workgroup runs, every gate/up
// workgroup on its XCD has started, and on any other XCD either all have
// started or only gate/up workgroups, which wait for nothing, hold its
// slots: every entry finishes and every wait ends (the wait is bounded
// besides).  The down items thus fill the compute units that the last
// gate/up items leave idle.  grid ngu + nxd * ny, block 256.
template <int MT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void k_gd(Plan p, int ny, int nxg, int nxd) {
    static_assert(MT <= 4, "one launch for chunks of up to 64 tokens");
    extern __shared__ __attribute__((aligned(16))) char lds[];
    __shared__ float2 hpart[4][128];
    __shared__ int rows[128];
    __shared__ float wrow[128];
    const int L = blockIdx.x, ngu = nxg * ((p.nsched[0] + 7) & ~7);
    if (L < ngu)
        gu_item<MT, true>(p, lds, hpart, rows, L, nxg);
    else if (L < ngu + nxd * ny)
        dn_item<MT, true>(p, (_Float16*)lds, wrow, rows, L - ngu, nxd);
}

// out[t] = sum_j ysort[inv[t][j]] (slot order) + the shared expert's
// slices, rounded once.  grid (T, ceil(H/1024)), block 256: each thread
// sums four adjacent columns with 16-byte loads, and the loads of a batch of
// rows go out together before any is added (the sum keeps the row order).
__global__ __launch_bounds__(256) void k_gg_combine(Plan p) {
    constexpr int kRb = 8;   // rows per batch of loads
    const int t = blockIdx.x, i = (blockIdx.y * 256 + threadIdx.x) * 4;
    if (i >= p.H) return;    // H % 64 == 0: columns i .. i + 3 all exist
    const int nr = p.k + p.n_vs_dn;
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
    for (int j0 = 0; j0 < nr; j0 += kRb) {
        float4 v[kRb];
#pragma unroll
        for (int u = 0; u < kRb; ++u) {
            const int j = min(j0 + u, nr - 1);   // clamped: in bounds, skipped below
            const int64_t row = j < p.k ? (int64_t)p.inv[t * p.k + j]
                                        : (int64_t)p.T * p.k + (int64_t)(j - p.k) * p.T + t;
            v[u] = *(const float4*)(p.ysort + row * p.H + i);
        }
#pragma unroll
        for (int u = 0; u < kRb; ++u)
            if (j0 + u < nr) {
                a0 += v[u].x;
                a1 += v[u].y;
                a2 += v[u].z;
                a3 += v[u].w;
            }
    }
    if (*p.f_err & kErrWait) {
        // a down item of the single GEMM launch gave up waiting: its rows may
        // be stale, so the output reads NaN rather than a plausible row
        a0 = a1 = a2 = a3 = __builtin_nanf("");
    }
    const int64_t o = (int64_t)t * p.out_stride + i;
    if (p.out_f32) {
        float* out = (float*)p.out + o;
        out[0] = a0;
        out[1] = a1;
        out[2] = a2;
        out[3] = a3;
    } else {
        uint16_t* out = (uint16_t*)p.out + o;
        out[0] = f32_to_bf16(a0);
        out[1] = f32_to_bf16(a1);
        out[2] = f32_to_bf16(a2);
        out[3] = f32_to_bf16(a3);
    }
}

// Dynamic LDS of k_gu: the big path's staged batch, the small path's
// group constants and its reduction buffer, which reuses their space.
size_t gu_lds_bytes(int G_H, int MT) {
    const size_t big = (size_t)ring_depth(MT, 2 * gu_tiles(MT)) * ring_stage_bytes(MT, 2 * gu_tiles(MT)),
                 red = sizeof(GuRed);
    const size_t c = (size_t)2 * G_H * 32 * 4;
    return big > red ? (big > c ? big : c) : (red > c ? red : c);
}

// The schedule holds chunk indices below 256 (T <= 255 * 128) and sorted
// rows below 2^24, and the LDS of the gate/up and down kernels must fit a
// workgroup.
// Shared rows per token of ysort after the down projection.  With chunks of
// 128 tokens (many chunks per call) one item of each shared chunk runs the
// down projection over all the shared columns, which saves the other
// virtual experts' rows of ysort and their reads in the combine; smaller
// calls keep one item per virtual expert, which shortens their longest item.
int grouped_shared_rows(int ntile, int n_vs) { return ntile > 64 && n_vs > 1 ? 1 : n_vs; }

bool grouped_ok(int H, int I, int64_t T, int rows_per_token) {
    return T <= 255 * 128 && T * rows_per_token < (1 << 24) && dn_lds_bytes(I, 8) <= 160 * 1024 &&
           gu_lds_bytes(H / 64, 8) + 5 * 1024 <= 160 * 1024;
}

// The two GEMM launches for chunks of up to 16 MT tokens.
template <int MT>
mq_status launch_gemms(const Plan& p, hipStream_t s) {
    const size_t gu_lds = gu_lds_bytes(p.G_H, MT), dn_lds = dn_lds_bytes(p.I, MT);
    const int ny = (p.max_tiles + 7) / 8 * 8;   // grid_pos needs a multiple of 8
    const int nxg = p.I / 64, nxd = (p.H / 64 + kDnTiles - 1) / kDnTiles;
    if constexpr (MT <= 4) {
        // a down item waits for its own entry only: no item may span the
        // shared expert's virtual experts (merged only at 128-token chunks)
        if (p.n_vs_dn != p.n_vs) return MQ_ERR_UNSUPPORTED;
        const size_t lds = gu_lds > dn_lds ? gu_lds : dn_lds;
        if (lds > 64 * 1024 &&
            hipFuncSetAttribute((const void*)k_gd<MT>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) !=
                hipSuccess)
            return MQ_ERR_UNSUPPORTED;
        hipLaunchKernelGGL(k_gd<MT>, dim3((nxg + nxd) * ny), dim3(256), lds, s, p, ny, nxg, nxd);
    } else {
        if (gu_lds > 64 * 1024 && hipFuncSetAttribute((const void*)k_gu<MT>,
                                                      hipFuncAttributeMaxDynamicSharedMemorySize,
                                                      (int)gu_lds) != hipSuccess)
            return MQ_ERR_UNSUPPORTED;
        if (dn_lds > 64 * 1024 && hipFuncSetAttribute((const void*)k_dn<MT>,
                                                      hipFuncAttributeMaxDynamicSharedMemorySize,
                                                      (int)dn_lds) != hipSuccess)
            return MQ_ERR_UNSUPPORTED;
        hipLaunchKernelGGL(k_gu<MT>, dim3(nxg, ny), dim3(256), gu_lds, s, p);
        hipLaunchKernelGGL(k_dn<MT>, dim3(nxd, ny), dim3(256), dn_lds, s, p);
    }
    return MQ_OK;
}

mq_status launch_grouped(const Plan& p, hipStream_t s) {
    hipLaunchKernelGGL(k_scores, dim3((p.T + 15) / 16, p.E_pad / 64, p.rsplit_used), dim3(256), 0, s, p);
    if (p.E <= 128)
        hipLaunchKernelGGL(k_select<2>, dim3((p.T + 3) / 4), dim3(256), 0, s, p);
    else
        hipLaunchKernelGGL(k_select<kMaxExperts / 64>, dim3((p.T + 3) / 4), dim3(256), 0, s, p);
    hipLaunchKernelGGL(k_sort, dim3(1), dim3(1024), 0, s, p);
    const mq_status st = p.ntile <= 64 ? launch_gemms<4>(p, s) : launch_gemms<8>(p, s);
    if (st != MQ_OK) return st;
    if (p.tail)
        hipLaunchKernelGGL(k_tail_grouped, dim3(p.T), dim3(1024), 0, s, p);
    else
        hipLaunchKernelGGL(k_gg_combine, dim3(p.T, (p.H + 1023) / 1024), dim3(256), 0, s, p);
    return MQ_OK;
}

}  // namespace mq
