/*
 * CPU oracle for the quantized mixture-of-experts FFN layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark load this library.  It shares no code,
 * header, table or helper with the GPU library, and the GPU library never
 * calls it.
 *
 * Plain, slow, fp64.  Every matrix is read in the canonical MLX-affine
 * layout, one loop nest per step of the method, in the order the method's
 * description gives them (TurboFieldfare "System design", sections
 * "Why the runtime has this shape", "Decode" and "Metal execution").
 *
 * Canonical layout of a [rows][cols] matrix with b-bit codes (b = 4 or 8):
 *   codes  uint32 [rows][cols*b/32]; element c of a row sits in word
 *          c/(32/b) at bit b*(c mod 32/b), low bits first;
 *   scales bf16   [rows][cols/64]   (bit patterns, uint16)
 *   biases bf16   [rows][cols/64]
 * and the weight is  w[r][c] = scale[r][c/64] * q[r][c] + bias[r][c/64].
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    const uint32_t* codes;
    const uint16_t* scales;         /* [rows][cols/group] */
    const uint16_t* biases;         /* [rows][cols/group] */
    int32_t rows, cols, bits;
    int32_t group;                  /* weights per scale/bias; 0 means 64 */
} oq_tensor;

typedef struct {
    oq_tensor w;                    /* [E][H], 8-bit */
    const float* router_scale;      /* [H], NULL means all ones */
    const float* per_expert_scale;  /* [E], NULL means all ones */
    const float* logit_bias;        /* [E], NULL means all zeros */
    int32_t top_k;
    double eps;                     /* RMS-norm epsilon */
} oq_router;

typedef struct {
    const oq_tensor* gate;          /* [E] tensors, each [I][H] */
    const oq_tensor* up;            /* [E] tensors, each [I][H] */
    const oq_tensor* down;          /* [E] tensors, each [H][I] */
    int32_t num_experts;
} oq_pool;

typedef struct {
    oq_tensor gate, up, down;       /* [Is][H], [Is][H], [H][Is] */
} oq_shared;

/* Layer tail: post-FFN RMS norms (learned weights [H], NULL: none) of the
 * shared branch, the routed branch and their sum, then the residual and the
 * layer scalar. */
typedef struct {
    const float* norm_shared;
    const float* norm_routed;
    const float* norm_out;
    double eps;
    double layer_scalar;
} oq_tail;

double   oq_bf16_to_double(uint16_t b);
uint16_t oq_bf16_round(double v);                       /* nearest, ties to even */
int32_t  oq_code(const oq_tensor* t, int32_t r, int32_t c);
double   oq_weight(const oq_tensor* t, int32_t r, int32_t c);
void     oq_dequant(const oq_tensor* t, double* w);     /* w [rows][cols] */
void     oq_matvec(const oq_tensor* t, const double* x, double* y);
double   oq_gelu_tanh(double z);

void oq_router_logits(const oq_router* rt, const uint16_t* x, int32_t H, double* logits);
void oq_topk(const oq_router* rt, const double* logits, int32_t E, int32_t* ids, double* w);
void oq_expert(const oq_tensor* gate, const oq_tensor* up, const oq_tensor* down,
               const double* x, double* y);

/* Whole layer for T tokens.  Any of ids, w, logits, out64, out_bf16 may be NULL.
 * Returns 0, or -1 on inconsistent shapes. */
int32_t oq_moe_forward(const uint16_t* x, int32_t T, int32_t H, const oq_router* rt,
                       const oq_pool* pool, const oq_shared* shared,
                       int32_t* ids, double* w, double* logits, double* out64, uint16_t* out_bf16);

/* The same with the layer tail (tail NULL: none) and an optional residual
 * (bf16 [T][H], NULL: zero). */
int32_t oq_moe_forward_ex(const uint16_t* x, int32_t T, int32_t H, const oq_router* rt,
                          const oq_pool* pool, const oq_shared* shared, const oq_tail* tail,
                          const uint16_t* resid, int32_t* ids, double* w, double* logits, double* out64,
                          uint16_t* out_bf16);

/* out = layer_scalar * (residual + N_out(N_s(s) + N_r(r))) for one row. */
void oq_layer_tail(const double* s, const double* r, const uint16_t* resid, int32_t H, const oq_tail* tail,
                   double* out);

/* Quantized head: logits = W x per token, softcapped when softcap > 0, and
 * the argmax (ties to the lower row).  logits [T][rows], argmax [T]; either may be NULL. */
void oq_qgemv_head(const oq_tensor* t, const uint16_t* x, int32_t T, double softcap, double* logits,
                   int32_t* argmax);

/* Brute force: every expert evaluated densely, masked to the selected ones. */
int32_t oq_moe_dense_masked(const uint16_t* x, int32_t T, int32_t H, const oq_router* rt,
                            const oq_pool* pool, const oq_shared* shared, double* out64);

/* Unit-weight RMS norm of bf16 rows, rounded back to bf16 (between stacked layers). */
void oq_rmsnorm_bf16(const uint16_t* in, int32_t T, int32_t H, double eps, uint16_t* out);

#ifdef __cplusplus
}
#endif
#endif
