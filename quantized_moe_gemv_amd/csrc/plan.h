// One call's resolved arguments and workspace carve-up, passed by value to
// every kernel of the call.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mq {

constexpr int kRouterTokens = 4;    // tokens per router workgroup
constexpr int kMaxTopK = 16;
constexpr int kMaxExperts = 256;
constexpr int kDownSplits = 4;      // split of the down-projection source list (GEMV path)
constexpr int kRouterPieces = 8;   // single-launch decode: column pieces of a 16-expert router slice
constexpr int kCtrStride = 64;      // counters of the single-launch decode sit 256 bytes apart
constexpr int kFusedMaxWG = 1024;   // largest grid of the single launch (compute units)
// Sticky error bits kept in every workspace (read by mq_workspace_errors).
constexpr uint32_t kErrWait = 1u;   // a bounded wait for another workgroup's result gave up
constexpr uint32_t kErrRange = 2u;  // an fp16 activation overflowed (inf) or was NaN

struct Plan {
    // sizes
    int T, H, E, E_pad, k, I, Is;
    int G_H, G_I, G_s;              // groups of 64 along hidden, inter, shared inter
    int rsplit, rgroups;            // router k-splits and groups per split
    int rsplit_used;                // grouped path: column splits of the router scores (<= rsplit)
    int has_shared;

    // inputs
    const uint16_t* x;
    int64_t x_stride;
    const uint8_t* router_w;
    const float* router_scale;
    const float* pes;
    const float* logit_bias;
    float eps;
    float in_eps;                   // > 0: unit-weight RMSNorm of the input row first (single-launch path)
    const uint8_t* pool_base;
    int64_t expert_stride, gate_off, up_off, down_off;
    const uint8_t* sh_gate;
    const uint8_t* sh_up;
    const uint8_t* sh_down;

    // outputs
    void* out;
    int64_t out_stride;
    int out_f32;
    int32_t* ids_out;
    float* w_out;
    float* logits_out;

    // workspace (GEMV path and router)
    float* r;          // [T][H]      router input, scaled
    float* rsum8;      // [T][G_H][4] sums of r over each lane's 16 columns (8-bit blocks)
    float* xsum4;      // [T][G_H][4] sums of x over each lane's 16 columns (4-bit blocks)
    float* plog;       // [rsplit][T][E_pad] partial router scores
    int32_t* ids;      // [T][k]  (given routing: the caller's ids)
    float* wts;        // [T][k]
    uint16_t* hhi;     // [T][k][I]   GeGLU activations, bf16 high part
    uint16_t* hlo;     // [T][k][I]   bf16 low part (h - hi)
    float* hsum;       // [T][k][G_I][4]
    uint16_t* shi;     // [T][Is]
    uint16_t* slo;     // [T][Is]
    float* ssum;       // [T][G_s][4]
    float* dpart;      // [T][kDownSplits][H]

    // workspace (grouped path)
    _Float16* x16;     // [T][H]      fp16 input, columns with (c & 2) != 0 divided by 16
    float* xso;        // [T][G_H][2] per group: sum of x, -1024 * sum of x16
    int32_t* counts;   // [E]
    int32_t* offsets;  // [E + 1]
    int32_t* perm;     // [T*k]  pair p = t*k + j, sorted by expert (any order within one)
    int32_t* inv;      // [T*k]  position of pair p in perm
    int2* sched;       // [max_tiles] (unit << 16 | tiles << 8 | chunk, first row | count << 24)
    int32_t* nsched;   // [2]: schedule entries, and those on the dequantised-weight path (first)
    // rows T*k + j*T + t of hg / ysort belong to token t and the shared
    // expert's virtual expert j (its rows j*I .. j*I + I - 1)
    _Float16* hg;      // [T*k + n_vs*T][I]  GeGLU activations in sorted order (scaled as x16)
    float* hso;        // [T*k + n_vs*T][G_I][2]  their per-group pairs, as xso
    float* ysort;      // [T*k + n_vs*T][H]  weighted expert outputs in sorted order
    // single-launch decode: tagged words and counters that persist across calls
    uint64_t* f_rpart;   // [copies][E/16][8][16] partial router scores, rpart_stride apart
    uint64_t* f_hs;      // [copies][Is]        shared GeGLU activations (fp16 payload), h_stride apart
    uint64_t* f_h;       // [copies][k][I]      routed GeGLU activations, h_stride apart
    int64_t h_stride, rpart_stride;
    uint64_t* f_piece;   // [G_H][n_src][64]    partial outputs per output tile and source
    // a stack of layers in one launch: the layer input as tagged bf16 pairs
    // (layers after the first) and the layer output published the same way
    // for the next layer, one copy per XCD, xw_stride apart
    const uint64_t* x_w;   // non-null: read the input row from here instead of x
    uint64_t* out_w;       // non-null: publish the output row here (out may then be null)
    int64_t xw_stride;
    uint32_t* f_epoch;   // per workgroup of the single launch: the last tag it used (kFusedMaxWG words)
    uint32_t* f_err;     // non-zero once a bounded wait has given up
    int n_router, n_sd, n_sc, n_rh, n_rng, n_src;   // n_rng: tile ranges per routed down slot
    int nwg;           // workgroups of the single launch (one per compute unit)
    int max_tiles;     // upper bound of scheduled (expert, token chunk) pairs
    int ntile;         // tokens per grouped chunk (32 or 128)
    int n_vs;          // virtual experts of the shared expert (0 without one)

    // fields added after the single-launch decode's (its scalar argument
    // loads are laid out around the fields above)
    int ebits;                // code width of the routed and shared experts (4 or 8)
    float* xsum8;             // [T][G_H][4] sums of x over the lane columns of 8-bit blocks (8-bit experts)
    const int32_t* slots;     // [T][k] pool blob each (token, slot) reads; null: the expert id (GEMV path)
    int gu_item0, dn_split0;  // GEMV path launch offsets: first gate/up item and first down split of a launch
    // layer tail (tail != 0): out = t_scalar * (res + N_o(N_s(s) + N_r(r)))
    int tail;
    const float* tn_s;     // [H] or null: no norm of the shared branch
    const float* tn_r;     // [H] or null: routed branch
    const float* tn_o;     // [H] or null: their sum
    const uint16_t* t_res; // residual rows or null (t_res_in: the input rows as given)
    int64_t t_res_stride;
    int t_res_in;          // residual = the layer's input row before the input norm
    float t_eps, t_scalar;
    uint64_t* f_tail;      // single-launch decode: [G_H][8] tagged partial sums of the tail norms
    int n_vs_dn;           // grouped path: shared rows per token of ysort after the down projection (1 when
                           // one item of each chunk covers all of the shared expert's columns, else n_vs)
    int32_t* gdone;        // grouped path, one GEMM launch: gate/up workgroups finished per schedule entry
    int32_t* gqueue;       //   [0] entries finished, [1 + i] the i-th to finish (-1 until then)
};

// Arguments of the quantized GEMV head (head.hip).
constexpr int kHeadTokens = 8;          // tokens per call
constexpr int kHeadLdsBytes = 60 << 10; // the call's token rows (bf16) and their lane sums staged in LDS

// Dynamic LDS of the head kernel for T token rows of `cols` columns.
inline size_t head_lds_bytes(int T, int cols) { return (size_t)T * cols * 2 + (size_t)T * (cols / 64) * 16; }

struct HeadArgs {
    const uint8_t* w;      // DEV_V1 [rows][cols]
    int rows, cols, bits, T;
    const uint16_t* x;     // bf16 [T][cols], x_stride apart
    int64_t x_stride;
    void* y;               // optional [T][rows] (y_stride apart), f32 or bf16
    int64_t y_stride;
    int y_f32;
    float cap;             // > 0: softcap
    float2* part;          // optional [T][workgroups] best (value, row as int bits) per workgroup
};

// Fields of one layer of a single-launch stack (everything else is shared).
struct StackLayer {
    const uint16_t* x;
    const uint64_t* x_w;
    void* out;
    uint64_t* out_w;
    const uint8_t* router_w;
    const float* router_scale;
    const float* pes;
    const float* logit_bias;
    const uint8_t* pool_base;
    const uint8_t* sh_gate;
    const uint8_t* sh_up;
    const uint8_t* sh_down;
    int32_t* ids_out;
    float* w_out;
    float* logits_out;
    int64_t expert_stride, gate_off, up_off, down_off;
    float eps, in_eps;
    // layer tail
    int tail, t_res_in;
    const float* tn_s;
    const float* tn_r;
    const float* tn_o;
    const uint16_t* t_res;
    int64_t t_res_stride;
    float t_eps, t_scalar;
};

constexpr int kStackChunk = 12;  // layers per argument-writing launch (kernel arguments stay under 4 KiB)

struct StackChunk {
    int n;
    StackLayer l[kStackChunk];
};

}  // namespace mq
