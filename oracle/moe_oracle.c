/*
 * CPU oracle for the quantized mixture-of-experts FFN layer (fp64).
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the CPU
 * baseline leg of the benchmark, never by the GPU library, with which it
 * shares no code.  The formulas follow TurboFieldfare "System design":
 *   - affine group-64 codes with a BF16 scale and bias per group
 *     ("Why the runtime has this shape", 4th bullet; ".gturbo directory");
 *   - router: scale-free RMS norm, router_scale / sqrt(hidden), 8-bit affine
 *     projection to expert scores, the 8 highest, softmax over them times
 *     per_expert_scale ("Decode", the router listing);
 *   - routed experts are GeGLU FFNs whose outputs are weighted and summed
 *     ("Metal execution": fused affine decode, GeGLU, weighted reduction);
 *   - the dense shared expert is a separate branch added without a weight
 *     ("Why the runtime has this shape", 3rd bullet), combined with the
 *     routed branch ("Prefill", last bullet; "Decode", phase table, cb2).
 * Readings where the pages are silent (nibble order, the affine sign,
 * epsilon, tie-breaks) are stated at each function.
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#define GROUP 64

/* bf16 bit pattern -> double (exact: bf16 is the top half of an fp32). */
double oq_bf16_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* double -> nearest bf16, ties to even, rounding the exact double once.
 * Finite, non-overflowing inputs only (the layer never produces others). */
uint16_t oq_bf16_round(double v) {
    if (v == 0.0) return signbit(v) ? 0x8000u : 0u;
    double a = fabs(v);
    int e;
    frexp(a, &e);                          /* a = m * 2^e, m in [0.5, 1) */
    int ulp_exp = e - 8;                   /* bf16 keeps 8 significant bits */
    if (ulp_exp < -133) ulp_exp = -133;    /* subnormal bf16 spacing 2^-133 */
    double ulp = ldexp(1.0, ulp_exp);
    double q = a / ulp;                    /* exact: power-of-two scaling */
    double fl = floor(q);
    double rem = q - fl;
    if (rem > 0.5 || (rem == 0.5 && fmod(fl, 2.0) != 0.0)) fl += 1.0;
    double r = fl * ulp;                   /* representable in bf16 */
    float f = (float)r;                    /* exact */
    uint32_t u;
    memcpy(&u, &f, 4);
    uint16_t b = (uint16_t)(u >> 16);
    return v < 0 ? (uint16_t)(b | 0x8000u) : b;
}

/* Code q of element (r, c).  Reading: little-endian words, low bits first. */
int32_t oq_code(const oq_tensor* t, int32_t r, int32_t c) {
    int32_t per_word = 32 / t->bits;
    int32_t words_per_row = t->cols / per_word;
    uint32_t word = t->codes[(int64_t)r * words_per_row + c / per_word];
    uint32_t mask = (t->bits == 32) ? 0xFFFFFFFFu : ((1u << t->bits) - 1u);
    return (int32_t)((word >> (t->bits * (c % per_word))) & mask);
}

/* Affine dequantisation: w = scale * q + bias, q unsigned (reading of "affine"),
 * with one scale and bias per `group` consecutive weights of a row (64 in the
 * checkpoint; 0 in the descriptor means 64). */
double oq_weight(const oq_tensor* t, int32_t r, int32_t c) {
    int32_t gs = t->group > 0 ? t->group : GROUP;
    int32_t groups = t->cols / gs;
    int64_t g = (int64_t)r * groups + c / gs;
    return oq_bf16_to_double(t->scales[g]) * (double)oq_code(t, r, c) + oq_bf16_to_double(t->biases[g]);
}

void oq_dequant(const oq_tensor* t, double* w) {
    for (int32_t r = 0; r < t->rows; ++r)
        for (int32_t c = 0; c < t->cols; ++c) w[(int64_t)r * t->cols + c] = oq_weight(t, r, c);
}

/* y[r] = sum_c w[r][c] * x[c]: the matrix acts on the input from the left. */
void oq_matvec(const oq_tensor* t, const double* x, double* y) {
    for (int32_t r = 0; r < t->rows; ++r) {
        double acc = 0.0;
        for (int32_t c = 0; c < t->cols; ++c) acc += oq_weight(t, r, c) * x[c];
        y[r] = acc;
    }
}

/* GELU, tanh form (Hendrycks and Gimpel 2016): 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))). */
double oq_gelu_tanh(double z) {
    const double k = 0.79788456080286535587989211986876;   /* sqrt(2/pi) */
    return 0.5 * z * (1.0 + tanh(k * (z + 0.044715 * z * z * z)));
}

/* Router scores ("Decode", the router listing): the token is divided by its
 * root mean square (no learned weight), multiplied by router_scale and by
 * 1/sqrt(H), and projected by the 8-bit affine router matrix to one score
 * per expert.  Readings: eps is a parameter (1e-6 in the workloads), inside
 * the square root; logit_bias (the synthetic Zipf skew) is added after the
 * projection. */
void oq_router_logits(const oq_router* rt, const uint16_t* x, int32_t H, double* logits) {
    double* r = (double*)malloc(sizeof(double) * (size_t)H);
    double ss = 0.0;
    for (int32_t i = 0; i < H; ++i) {
        double v = oq_bf16_to_double(x[i]);
        ss += v * v;
    }
    double inv = 1.0 / sqrt(ss / (double)H + rt->eps);
    double inv_sqrt_h = 1.0 / sqrt((double)H);
    for (int32_t i = 0; i < H; ++i) {
        double rs = rt->router_scale ? (double)rt->router_scale[i] : 1.0;
        r[i] = oq_bf16_to_double(x[i]) * inv * rs * inv_sqrt_h;
    }
    oq_matvec(&rt->w, r, logits);
    if (rt->logit_bias)
        for (int32_t e = 0; e < rt->w.rows; ++e) logits[e] += (double)rt->logit_bias[e];
    free(r);
}

/* top_k = the k highest logits; weights = softmax over those k logits times
 * per_expert_scale of each chosen expert ("Decode", the router listing).
 * Readings: the selection compares the exact (fp64) logits and equal values
 * go to the lower expert index; ids come out in selection order (highest
 * first); the softmax uses the fp64 logits. */
void oq_topk(const oq_router* rt, const double* logits, int32_t E, int32_t* ids, double* w) {
    int32_t k = rt->top_k;
    char* taken = (char*)calloc((size_t)E, 1);
    for (int32_t j = 0; j < k; ++j) {
        int32_t best = -1;
        double bv = 0.0;
        for (int32_t e = 0; e < E; ++e) {
            if (taken[e]) continue;
            double v = logits[e];
            if (best < 0 || v > bv) { best = e; bv = v; }
        }
        taken[best] = 1;
        ids[j] = best;
    }
    double m = logits[ids[0]];
    for (int32_t j = 1; j < k; ++j) if (logits[ids[j]] > m) m = logits[ids[j]];
    double den = 0.0;
    for (int32_t j = 0; j < k; ++j) den += exp(logits[ids[j]] - m);
    for (int32_t j = 0; j < k; ++j) {
        double pes = rt->per_expert_scale ? (double)rt->per_expert_scale[ids[j]] : 1.0;
        w[j] = exp(logits[ids[j]] - m) / den * pes;
    }
    free(taken);
}

/* One GeGLU expert: y = W_down . (gelu_tanh(W_gate . x) * (W_up . x)).
 * Reading: the GELU goes on the gate branch. */
void oq_expert(const oq_tensor* gate, const oq_tensor* up, const oq_tensor* down,
               const double* x, double* y) {
    int32_t I = gate->rows;
    double* g = (double*)malloc(sizeof(double) * (size_t)I);
    double* u = (double*)malloc(sizeof(double) * (size_t)I);
    oq_matvec(gate, x, g);
    oq_matvec(up, x, u);
    for (int32_t i = 0; i < I; ++i) g[i] = oq_gelu_tanh(g[i]) * u[i];
    oq_matvec(down, g, y);
    free(g);
    free(u);
}

static int32_t check_shapes(int32_t H, const oq_router* rt, const oq_pool* pool, const oq_shared* sh) {
    if (rt->w.cols != H || rt->w.rows != pool->num_experts || rt->top_k < 1 || rt->top_k > rt->w.rows)
        return -1;
    for (int32_t e = 0; e < pool->num_experts; ++e) {
        if (pool->gate[e].cols != H || pool->up[e].cols != H || pool->down[e].rows != H) return -1;
        if (pool->gate[e].rows != pool->up[e].rows || pool->down[e].cols != pool->gate[e].rows) return -1;
    }
    if (sh && (sh->gate.cols != H || sh->up.cols != H || sh->down.rows != H ||
               sh->gate.rows != sh->up.rows || sh->down.cols != sh->gate.rows))
        return -1;
    return 0;
}

/* Post-FFN RMS norm of one branch: v / sqrt(mean(v^2) + eps) times the
 * learned weight w (element-wise). */
static void tail_norm(const double* v, const float* w, int32_t H, double eps, double* out) {
    double ss = 0.0;
    for (int32_t i = 0; i < H; ++i) ss += v[i] * v[i];
    const double inv = 1.0 / sqrt(ss / (double)H + eps);
    for (int32_t i = 0; i < H; ++i) out[i] = v[i] * inv * (double)w[i];
}

/* The layer tail ("Decode", phase table, cb2: post-FFN norms, residual and
 * layer scalar; "Why the runtime has this shape": parallel shared and routed
 * FFNs and a learned layer scalar).  Readings: each branch may have its own
 * post-FFN RMS norm with a learned weight (NULL: none), their sum may have
 * one more, the residual row is added after those norms, and the layer
 * scalar multiplies the whole result:
 *   out = layer_scalar * (residual + N_out(N_s(s) + N_r(r))). */
void oq_layer_tail(const double* s, const double* r, const uint16_t* resid, int32_t H, const oq_tail* tail,
                   double* out) {
    double* a = (double*)malloc(sizeof(double) * (size_t)H);
    double* b = (double*)malloc(sizeof(double) * (size_t)H);
    if (tail->norm_shared) tail_norm(s, tail->norm_shared, H, tail->eps, a);
    else for (int32_t i = 0; i < H; ++i) a[i] = s[i];
    if (tail->norm_routed) tail_norm(r, tail->norm_routed, H, tail->eps, b);
    else for (int32_t i = 0; i < H; ++i) b[i] = r[i];
    for (int32_t i = 0; i < H; ++i) a[i] += b[i];
    if (tail->norm_out) tail_norm(a, tail->norm_out, H, tail->eps, b);
    else for (int32_t i = 0; i < H; ++i) b[i] = a[i];
    for (int32_t i = 0; i < H; ++i) {
        double res = resid ? oq_bf16_to_double(resid[i]) : 0.0;
        out[i] = tail->layer_scalar * (res + b[i]);
    }
    free(a);
    free(b);
}

/* The layer, token by token: route, run the k chosen experts, weight and sum
 * them (routed branch), run the shared expert (shared branch), add the two
 * (or pass them through the layer tail), round once to bf16. */
int32_t oq_moe_forward_ex(const uint16_t* x, int32_t T, int32_t H, const oq_router* rt,
                          const oq_pool* pool, const oq_shared* shared, const oq_tail* tail,
                          const uint16_t* resid, int32_t* ids, double* w, double* logits, double* out64,
                          uint16_t* out_bf16) {
    if (check_shapes(H, rt, pool, shared)) return -1;
    int32_t E = pool->num_experts, k = rt->top_k;
    double* xf = (double*)malloc(sizeof(double) * (size_t)H);
    double* y = (double*)malloc(sizeof(double) * (size_t)H);
    double* sacc = (double*)malloc(sizeof(double) * (size_t)H);
    double* racc = (double*)malloc(sizeof(double) * (size_t)H);
    double* acc = (double*)malloc(sizeof(double) * (size_t)H);
    double* lg = (double*)malloc(sizeof(double) * (size_t)E);
    int32_t* id = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
    double* wt = (double*)malloc(sizeof(double) * (size_t)k);
    for (int32_t t = 0; t < T; ++t) {
        const uint16_t* xt = x + (int64_t)t * H;
        for (int32_t i = 0; i < H; ++i) xf[i] = oq_bf16_to_double(xt[i]);
        oq_router_logits(rt, xt, H, lg);
        oq_topk(rt, lg, E, id, wt);
        for (int32_t i = 0; i < H; ++i) sacc[i] = racc[i] = 0.0;
        if (shared) {
            oq_expert(&shared->gate, &shared->up, &shared->down, xf, y);
            for (int32_t i = 0; i < H; ++i) sacc[i] = y[i];
        }
        for (int32_t j = 0; j < k; ++j) {
            int32_t e = id[j];
            oq_expert(&pool->gate[e], &pool->up[e], &pool->down[e], xf, y);
            for (int32_t i = 0; i < H; ++i) racc[i] += wt[j] * y[i];
        }
        if (tail)
            oq_layer_tail(sacc, racc, resid ? resid + (int64_t)t * H : NULL, H, tail, acc);
        else
            for (int32_t i = 0; i < H; ++i) acc[i] = sacc[i] + racc[i];
        if (ids) memcpy(ids + (int64_t)t * k, id, sizeof(int32_t) * (size_t)k);
        if (w) memcpy(w + (int64_t)t * k, wt, sizeof(double) * (size_t)k);
        if (logits) memcpy(logits + (int64_t)t * E, lg, sizeof(double) * (size_t)E);
        if (out64) memcpy(out64 + (int64_t)t * H, acc, sizeof(double) * (size_t)H);
        if (out_bf16)
            for (int32_t i = 0; i < H; ++i) out_bf16[(int64_t)t * H + i] = oq_bf16_round(acc[i]);
    }
    free(xf); free(y); free(sacc); free(racc); free(acc); free(lg); free(id); free(wt);
    return 0;
}

int32_t oq_moe_forward(const uint16_t* x, int32_t T, int32_t H, const oq_router* rt,
                       const oq_pool* pool, const oq_shared* shared,
                       int32_t* ids, double* w, double* logits, double* out64, uint16_t* out_bf16) {
    return oq_moe_forward_ex(x, T, H, rt, pool, shared, NULL, NULL, ids, w, logits, out64, out_bf16);
}

/* Brute force for small shapes: all E experts are evaluated, and the sum
 * runs over every expert with weight = (routing weight if selected, else 0). */
int32_t oq_moe_dense_masked(const uint16_t* x, int32_t T, int32_t H, const oq_router* rt,
                            const oq_pool* pool, const oq_shared* shared, double* out64) {
    if (check_shapes(H, rt, pool, shared)) return -1;
    int32_t E = pool->num_experts, k = rt->top_k;
    double* xf = (double*)malloc(sizeof(double) * (size_t)H);
    double* ys = (double*)malloc(sizeof(double) * (size_t)H * (size_t)E);
    double* sh = (double*)malloc(sizeof(double) * (size_t)H);
    double* lg = (double*)malloc(sizeof(double) * (size_t)E);
    double* mask = (double*)malloc(sizeof(double) * (size_t)E);
    int32_t* id = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
    double* wt = (double*)malloc(sizeof(double) * (size_t)k);
    for (int32_t t = 0; t < T; ++t) {
        const uint16_t* xt = x + (int64_t)t * H;
        for (int32_t i = 0; i < H; ++i) xf[i] = oq_bf16_to_double(xt[i]);
        for (int32_t e = 0; e < E; ++e)
            oq_expert(&pool->gate[e], &pool->up[e], &pool->down[e], xf, ys + (int64_t)e * H);
        if (shared) oq_expert(&shared->gate, &shared->up, &shared->down, xf, sh);
        oq_router_logits(rt, xt, H, lg);
        oq_topk(rt, lg, E, id, wt);
        for (int32_t e = 0; e < E; ++e) mask[e] = 0.0;
        for (int32_t j = 0; j < k; ++j) mask[id[j]] = wt[j];
        for (int32_t i = 0; i < H; ++i) {
            double a = shared ? sh[i] : 0.0;
            for (int32_t e = 0; e < E; ++e) a += mask[e] * ys[(int64_t)e * H + i];
            out64[(int64_t)t * H + i] = a;
        }
    }
    free(xf); free(ys); free(sh); free(lg); free(mask); free(id); free(wt);
    return 0;
}

/* Between stacked decode layers: y = bf16(x / sqrt(mean(x^2) + eps)), unit weight. */
void oq_rmsnorm_bf16(const uint16_t* in, int32_t T, int32_t H, double eps, uint16_t* out) {
    for (int32_t t = 0; t < T; ++t) {
        double ss = 0.0;
        for (int32_t i = 0; i < H; ++i) {
            double v = oq_bf16_to_double(in[(int64_t)t * H + i]);
            ss += v * v;
        }
        double inv = 1.0 / sqrt(ss / (double)H + eps);
        for (int32_t i = 0; i < H; ++i)
            out[(int64_t)t * H + i] = oq_bf16_round(oq_bf16_to_double(in[(int64_t)t * H + i]) * inv);
    }
}

/* The tied quantized head at the end of decode ("Why the runtime has this
 * shape": embedding and head share quantized weights, final logit softcap
 * 30.0; "Decode": after the last layer the head returns the argmax token
 * directly in the greedy configuration).  For each token row x (bf16 [H]):
 * logit_v = W_v . x, then cap * tanh(logit_v / cap) when cap > 0, and the
 * argmax over v (the exact fp64 values; equal values to the lower index).
 * logits [T][V] and argmax [T] may each be NULL. */
void oq_qgemv_head(const oq_tensor* t, const uint16_t* x, int32_t T, double softcap, double* logits,
                   int32_t* argmax) {
    int32_t V = t->rows, H = t->cols;
    double* xf = (double*)malloc(sizeof(double) * (size_t)H);
    double* y = (double*)malloc(sizeof(double) * (size_t)V);
    for (int32_t tk = 0; tk < T; ++tk) {
        for (int32_t i = 0; i < H; ++i) xf[i] = oq_bf16_to_double(x[(int64_t)tk * H + i]);
        oq_matvec(t, xf, y);
        if (softcap > 0.0)
            for (int32_t v = 0; v < V; ++v) y[v] = softcap * tanh(y[v] / softcap);
        int32_t best = 0;
        for (int32_t v = 1; v < V; ++v)
            if (y[v] > y[best]) best = v;
        if (logits) memcpy(logits + (int64_t)tk * V, y, sizeof(double) * (size_t)V);
        if (argmax) argmax[tk] = best;
    }
    free(xf);
    free(y);
}
