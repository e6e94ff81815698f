/*
 * moegemv: one mixture-of-experts FFN layer over group-64 affine-quantized
 * weights, on one AMD Instinct MI355X (gfx950).
 *
 * The layer (TurboFieldfare "System design"):
 *   - weights are MLX-affine: packed 4-bit (experts) or 8-bit (router) codes
 *     with one BF16 scale and one BF16 bias per group of 64 weights,
 *     w = scale * q + bias  ("Why the runtime has this shape", 4th bullet);
 *   - the router normalises x without a learned scale, multiplies by
 *     router_scale / sqrt(hidden), projects to one score per expert, keeps
 *     the 8 highest and weights them by a softmax over those 8 times
 *     per_expert_scale ("Decode", router listing);
 *   - each selected expert is a GeGLU FFN, down(gelu_tanh(gate x) * up x),
 *     and the selected outputs are weighted and summed ("Metal execution");
 *   - a dense shared expert is added without a weight ("Why the runtime has
 *     this shape", 3rd bullet; "Prefill", last bullet).
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless the comment says HOST.
 *   - The caller owns every buffer.  The library borrows them until the work
 *     it enqueued on `stream` has finished ("Correctness and safety
 *     invariants": a queued consumer owns its scratch until completion) and
 *     allocates no device memory.
 *   - `stream` is a hipStream_t passed as void*; NULL is the default stream.
 *     Calls return once the work is enqueued.
 *   - All arguments are checked on the host before anything is enqueued.  On
 *     an error nothing is enqueued and nothing is written; the return value
 *     is a negative mq_status.  A failed launch returns MQ_ERR_HIP.  Faults
 *     inside kernels surface at the caller's next synchronisation.
 *   - Nothing throws across this interface and there is no global mutable
 *     state: calls on different streams with different workspaces are
 *     independent.
 */
#ifndef MOEGEMV_H
#define MOEGEMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MQ_OK = 0,
    MQ_ERR_NULL = -1,         /* a required pointer is NULL */
    MQ_ERR_SHAPE = -2,        /* inconsistent or unsupported sizes */
    MQ_ERR_ALIGN = -3,        /* a pointer, offset or stride is misaligned */
    MQ_ERR_UNSUPPORTED = -4,  /* bits, group, layout, dtype, path or size not supported */
    MQ_ERR_WORKSPACE = -5,    /* workspace missing or smaller than mq_workspace_bytes */
    MQ_ERR_HIP = -6,          /* a HIP runtime call failed */
    MQ_ERR_BUFFER = -7,       /* a HOST output buffer is too small */
    MQ_ERR_TOO_LARGE = -8     /* the call needs more than the fixed static scratch (moe_layer_forward_noalloc) */
} mq_status;

enum { MQ_LAYOUT_CANONICAL = 0, MQ_LAYOUT_DEV_V1 = 1 };
enum { MQ_DTYPE_BF16 = 0, MQ_DTYPE_F32 = 1 };
/* Kernel schedule.  AUTO: FUSED for one token, GEMV up to 4 tokens, GROUPED
 * above.  FUSED (one token only): one launch for the whole layer.  GEMV:
 * per-(token, expert) dot-product kernels.  GROUPED: tokens sorted by
 * expert, dequantised weights on the matrix cores; it takes at most 32640
 * tokens per call and an expert intermediate size of at most 2496
 * (MQ_ERR_UNSUPPORTED otherwise, before any work is queued). */
enum { MQ_PATH_AUTO = 0, MQ_PATH_GEMV = 1, MQ_PATH_GROUPED = 2, MQ_PATH_FUSED = 3 };

/*
 * A group-64 affine-quantized matrix W [rows][cols], codes of `bits` bits.
 *
 * MQ_LAYOUT_CANONICAL (host side only, the MLX checkpoint form):
 *   codes  uint32 [rows][cols*bits/32], little-endian; element c of a row is
 *          in word c/(32/bits) at bit bits*(c % (32/bits)), low bits first;
 *   scales bf16   [rows][cols/64];  biases bf16 [rows][cols/64].
 *
 * MQ_LAYOUT_DEV_V1 (what the kernels read): `codes` points at one packed
 * region of mq_packed_bytes() bytes, `scales` and `biases` are NULL.  Rows
 * are padded to a multiple of 64 (padding rows have zero codes, scale and
 * bias).  The region is a sequence of blocks, row-tile major: block (t, g)
 * holds rows 64t..64t+63 of group g (columns 64g..64g+63) and sits at byte
 * (t * cols/64 + g) * BLK:
 *   bits 4: BLK = 2304 = 2048 B of codes + 256 B of (scale, bias) pairs
 *   bits 8: BLK = 4352 = 4096 B of codes + 256 B of (scale, bias) pairs
 * The codes are uint32 words at [j][lane 0..63][i 0..3] (j < 2 for 4-bit,
 * j < 4 for 8-bit); with a = 4j + i, word (j, lane, i) holds
 *   4-bit: row 16*(a>>1) + lane%16, columns 32*(a&1) + 8*(lane/16) + 0..7;
 *          column e of the eight sits at bit 4*(e/2) + 16*(e%2);
 *   8-bit: row 16*(a>>2) + lane%16, columns 16*(a&3) + 4*(lane/16) + 0..3;
 *          column e of the four sits at bit 8*e.
 * The pair area is uint32 [r 0..15][m 0..3] = scale | bias << 16 of row
 * 16*m + r.  Packing copies every code, scale and bias unchanged; only
 * their positions move ("Source weights and bounded repack": the repack
 * changes the layout, never the values).
 */
typedef struct {
    const void* codes;
    const void* scales;
    const void* biases;
    int32_t rows, cols, bits, group, layout;
} mq_qtensor;

/* Router: 8-bit DEV_V1 matrix [E][H] plus optional per-feature and
 * per-expert factors (device float arrays; NULL means 1, 1 and 0). */
typedef struct {
    mq_qtensor w;
    const float* router_scale;      /* [H], 16-byte aligned */
    const float* per_expert_scale;  /* [E] */
    const float* logit_bias;        /* [E]: added to the scores before selection */
    int32_t top_k;                  /* 1 <= top_k <= min(E, 16) */
    float eps;                      /* RMS-norm epsilon */
} mq_router;

/* The routed-expert pool: num_experts equally spaced blobs ("The .gturbo
 * directory": fixed-stride expert blobs whose sub-tensors have their own
 * offsets; kernels bind sub-regions of one buffer).  Expert e's gate
 * matrix is DEV_V1 data at base + e*expert_stride + gate_offset, and so on.
 * gate and up are [inter][hidden], down is [hidden][inter], 4-bit.
 * expert_stride and the offsets are multiples of 256. */
typedef struct {
    const void* base;
    int64_t expert_stride;
    int64_t gate_offset, up_offset, down_offset;
    int32_t num_experts, hidden, inter, bits, group, layout;
} mq_expert_pool;

/* The dense shared expert: gate, up [shared_inter][hidden], down
 * [hidden][shared_inter], 4-bit DEV_V1.  Pass NULL for a layer without one. */
typedef struct {
    mq_qtensor gate, up, down;
} mq_shared;

/* Activations [tokens][hidden]; row_stride in elements (>= hidden). */
typedef struct {
    void* data;
    int32_t tokens, hidden, dtype;
    int64_t row_stride;
} mq_act;

/* The layer tail ("Decode", phase table cb2: after the routed branch is
 * reduced and combined with the shared branch, the post-FFN norms, the
 * residual and the layer scalar are applied; "Why the runtime has this
 * shape": parallel shared and routed FFNs, a learned layer scalar).  With s
 * the shared branch and r the weighted routed sum of a token:
 *   out = layer_scalar * (residual + N_out(N_s(s) + N_r(r))),
 *   N(v) = v / sqrt(mean(v^2) + eps) * w   (element-wise learned weight w),
 * where a NULL weight leaves that norm out (N(v) = v).  All in fp32 and
 * rounded once at the end, like the plain layer.  Readings where the pages
 * say only "post-FFN norms": one norm per branch and one on their sum, each
 * optional; the weight multiplies the normalised value directly (a
 * checkpoint that stores 1 + w passes 1 + w); the scalar multiplies the
 * residual too. */
typedef struct {
    const float* norm_shared;   /* [H] or NULL */
    const float* norm_routed;   /* [H] or NULL */
    const float* norm_out;      /* [H] or NULL */
    const void* residual;       /* bf16 [T][H] rows, residual_stride apart; NULL: none (zero) */
    int64_t residual_stride;    /* elements, >= H when residual is given */
    int32_t residual_is_input;  /* 1: the residual rows are x itself, as given (before
                                   input_rmsnorm_eps normalises it); residual is then ignored */
    float eps;                  /* >= 0, finite */
    float layer_scalar;         /* finite */
} mq_tail;

typedef struct {
    int32_t path;           /* MQ_PATH_*: AUTO picks by token count */
    int32_t* topk_ids;      /* optional [T][top_k]: selected experts, highest score first */
    float* topk_w;          /* optional [T][top_k]: their routing weights */
    float* logits;          /* optional [T][E]: router scores (incl. logit_bias) */
    void* workspace;        /* device scratch of workspace_bytes, 256-B aligned */
    size_t workspace_bytes;
    /* > 0: each input row is first replaced by bf16(x / sqrt(mean(x^2) + eps))
     * with this eps (a unit-weight RMSNorm in fp32, as mq_rmsnorm computes;
     * the norm between the layers of a stack), inside the call: the
     * single-launch path normalises while it stages the token, the other
     * paths normalise into the workspace first.  x itself is not written.
     * 0: off.  Negative or not finite: MQ_ERR_UNSUPPORTED. */
    float input_rmsnorm_eps;
    /* NULL: out = s + r.  Otherwise the layer tail above is applied to every
     * token (H <= 16384; weights 4-byte aligned).  moe_stack_forward takes a
     * HOST array of n_layers tails here; in a stack only layer 0 may name an
     * explicit residual, later layers use residual_is_input (their input is
     * the previous layer's output). */
    const mq_tail* tail;
    /* Given routing (GEMV path; AUTO runs it there, FUSED and GROUPED refuse
     * it): the router does not run and the experts come from these device
     * arrays.  route_ids int32 [T][top_k], route_w float [T][top_k]; both or
     * neither.  route_slots (optional, int32 [T][top_k]): the blob of the
     * pool that each (token, j) reads, for a pool of expert slots (a cache of
     * a larger pool held elsewhere); NULL reads blob route_ids[t][j].  Values
     * are not checked: each must name a blob of the pool.  topk_ids, topk_w
     * and logits are not written. */
    const int32_t* route_ids;
    const float* route_w;
    const int32_t* route_slots;
    /* hipEvent_t or NULL (GEMV path): the kernels of the routed experts are
     * enqueued after the stream waits for this event, those of the shared
     * expert before it, so the shared expert runs while the event's work
     * (e.g. copies that fill expert slots) is still in flight ("Decode",
     * phase table: the shared branch overlaps the expert reads). */
    void* experts_ready;
} mq_opts;

/* Device scratch one call needs for up to max_tokens tokens (the library's
 * own exchange buffers between its kernels and workgroups; the pages define
 * no such buffer).  The workspace must be zero-filled once before its first
 * use (the kernels leave their counters at zero when they finish).  Returns
 * 0 for invalid arguments. */
size_t mq_workspace_bytes(const mq_router* router, const mq_expert_pool* pool,
                          const mq_shared* shared, int32_t max_tokens);

/* out = shared(x) + sum_j w_j * expert_{id_j}(x) for every token of x
 * ("Decode": router listing, phase table cb2; "Prefill": routed work grouped
 * by expert, combined with the shared branch; "Metal execution": affine
 * decode, GeGLU and the weighted expert reduction in the expert kernels).
 * x: bf16 [T][H].  out: bf16 (rounded once, to nearest even) or f32 (the
 * same sums before that rounding), [T][H].  T = 0 is valid and does nothing.
 *
 * Preconditions that the host cannot check (they depend on values):
 *   - Range.  The GROUPED and FUSED paths carry x (GROUPED) and the GeGLU
 *     activations gelu(W_gate x) * (W_up x) (both) as fp16, as the pages'
 *     prefill stages FP16 operands ("Prefill").  Magnitudes must stay below
 *     65504; activations below 2^-14 lose relative precision (fp16
 *     subnormals).  Unit-RMS inputs, such as rows after an RMS norm
 *     (input_rmsnorm_eps > 0), meet this with a wide margin for weight
 *     scales up to 0.05.  An overflow sets bit 1 of mq_workspace_errors and
 *     the affected outputs are not finite.  The GEMV path keeps activations
 *     as bf16 high/low pairs (fp32 range) and has no such limit.
 *   - Co-residency (FUSED, and moe_stack_forward).  The single launch runs
 *     one workgroup per compute unit and its workgroups wait for each other's
 *     partial results, so all of them must be resident at once: do not run
 *     it beside other work that occupies whole compute units.  Every wait is
 *     bounded; a wait that gives up sets bit 0 of mq_workspace_errors and the
 *     output rows of that call read NaN.
 *   - Start order (GROUPED with chunks of up to 64 tokens, T <= 1024).  The
 *     gate/up and down projections run in one launch whose down workgroups
 *     wait for gate/up workgroups of lower index; that every wait ends rests
 *     on each XCD starting the workgroups it is given in index order, as the
 *     hardware dispatcher does.  The waits are bounded all the same; a give-up
 *     sets bit 0 and the output rows read NaN. */
mq_status moe_layer_forward(const mq_act* x, const mq_router* router, const mq_expert_pool* pool,
                            const mq_shared* shared, mq_act* out, const mq_opts* opts, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * call as moe_layer_forward, with the same kernels and results, but its
 * scratch is a fixed array in device memory owned by the library instead of
 * a caller workspace (opts->workspace and opts->workspace_bytes are
 * ignored).  It allocates nothing: no hipMalloc, hipFree or allocating
 * library call.
 *   - Limit: the call's scratch (mq_workspace_bytes for its token count)
 *     must fit mq_noalloc_scratch_bytes() = 40 MiB, every call of up to 128
 *     tokens of the Gemma-shaped layer; larger calls return
 *     MQ_ERR_TOO_LARGE before anything is enqueued.
 *   - Each device holds its own copy of the array from the library's first
 *     call on it until the process ends.  The first call on a device clears
 *     it on `stream` and must not be under stream capture
 *     (MQ_ERR_UNSUPPORTED); later calls may be captured.
 *   - Every call on one device shares that device's array, which keeps the
 *     last call's state: calls that may overlap on one device (other streams,
 *     other threads) race and give wrong results; serialise them.
 *   - Errors: as moe_layer_forward; the error bits of mq_workspace_errors
 *     are not reachable for this scratch. */
mq_status moe_layer_forward_noalloc(const mq_act* x, const mq_router* router, const mq_expert_pool* pool,
                                    const mq_shared* shared, mq_act* out, const mq_opts* opts, void* stream);

/* Bytes of the static scratch behind moe_layer_forward_noalloc. */
size_t mq_noalloc_scratch_bytes(void);

/* Device scratch of one moe_stack_forward call over these n_layers layers
 * (HOST arrays of n_layers descriptors; shared NULL or n_layers entries).
 * Zero-filled once before first use, as for mq_workspace_bytes.  A stack
 * workspace may also serve moe_layer_forward calls on one token of any of
 * its layers.  Returns 0 for invalid arguments. */
size_t mq_stack_workspace_bytes(const mq_router* routers, const mq_expert_pool* pools,
                                const mq_shared* shared, int32_t n_layers);

/* One decode token through a stack of n_layers layers in one launch (the
 * runtime decodes a token through every layer in turn, 30 of them for this
 * model: "Why the runtime has this shape"; "Decode").  Layer l computes as
 * moe_layer_forward on its input; layer 0's input is x, normalised first
 * when opts->input_rmsnorm_eps > 0; layer l > 0 takes the previous layer's
 * output rounded to bf16, normalised first when between_eps > 0 (the
 * unit-weight RMS norm of mq_rmsnorm).  out receives the last layer's output.
 * routers, pools, shared: HOST arrays of n_layers descriptors (shared NULL
 * when no layer has a shared expert), every layer with the sizes of the
 * first.  x and out: one token.  opts->path AUTO or FUSED (the single-launch
 * path must fit the device: MQ_ERR_UNSUPPORTED otherwise); opts->topk_ids,
 * topk_w [n_layers][k] and logits [n_layers][E] are optional per-layer
 * reports; the workspace must hold mq_stack_workspace_bytes.  The result is
 * bit for bit that of n_layers FUSED moe_layer_forward calls chained the
 * same way.  Errors as moe_layer_forward; n_layers < 1 or layers of
 * different sizes: MQ_ERR_SHAPE. */
mq_status moe_stack_forward(const mq_act* x, int32_t n_layers, const mq_router* routers,
                            const mq_expert_pool* pools, const mq_shared* shared, float between_eps,
                            mq_act* out, const mq_opts* opts, void* stream);

/* HOST result: the sticky error bits that the kernels keep in a workspace
 * ("Correctness and safety invariants": a queued consumer owns its scratch
 * until completion, so the bits are read after the stream has finished).
 *   Bit 0 (FUSED, GROUPED, stack): a bounded wait for another workgroup's
 *         result gave up, so the calls since the bits were last clear may
 *         have wrong results; their outputs read NaN (it happens only if the
 *         workgroups of a launch are not all resident at once, or, GROUPED,
 *         not started in index order).
 *   Bit 1 (FUSED, GROUPED, stack): an fp16 activation overflowed or was NaN
 *         (see the range precondition of moe_layer_forward).
 * Copies the bits into *errors after the work queued on `stream` has
 * finished (the call synchronises the stream).  The bits stay set until the
 * workspace is zero-filled again.  workspace_bytes >= 1024. */
mq_status mq_workspace_errors(const void* workspace, size_t workspace_bytes, uint32_t* errors, void* stream);

/* Unit-weight RMS norm between stacked layers: out = bf16(x / sqrt(mean(x^2) + eps))
 * (the scale-free RMS norm of the "Decode" router listing, applied to the
 * layer input as the stack harness does between layers; eps inside the
 * root).  x and out bf16 [T][H]; they may alias.  MQ_ERR_* on invalid
 * arguments, nothing written then. */
mq_status mq_rmsnorm(const mq_act* x, mq_act* out, float eps, void* stream);

/* Bytes of a matrix in `layout` (0 for unsupported arguments): codes plus
 * one BF16 scale and bias per group ("Why the runtime has this shape", 4th
 * bullet; per-expert blob sizes as in "Resource split"). */
size_t mq_packed_bytes(int32_t rows, int32_t cols, int32_t bits, int32_t group, int32_t layout);

/* HOST: fill *pool's offsets and stride for experts packed back to back as
 * gate, up, down, each blob rounded up to page_bytes (a power of two >= 256)
 * ("The .gturbo directory": fixed-stride page-aligned expert blobs;
 * "Resource split": the page-rounded blob size).
 * base is left as given.  Returns the stride, 0 on invalid arguments. */
int64_t mq_pool_layout(int32_t hidden, int32_t inter, int32_t bits, int32_t group,
                       int64_t page_bytes, mq_expert_pool* pool);

/* HOST: canonical (MLX affine: packed codes, one BF16 scale and bias per
 * group, "Why the runtime has this shape") -> DEV_V1, the same values in the
 * matrix-core fragment order described above.  src describes HOST canonical arrays; dst is a
 * HOST buffer of dst_bytes >= mq_packed_bytes(.., MQ_LAYOUT_DEV_V1).  On
 * success *dst_desc (may be NULL) describes dst as a DEV_V1 tensor. */
mq_status mq_pack(const mq_qtensor* src, void* dst, size_t dst_bytes, mq_qtensor* dst_desc);

/* HOST: DEV_V1 -> canonical; the exact inverse of mq_pack.  src->codes is a
 * HOST copy of the packed region; codes/scales/biases are HOST buffers of
 * the canonical sizes. */
mq_status mq_unpack(const mq_qtensor* src, uint32_t* codes, uint16_t* scales, uint16_t* biases);

/* Parity hooks (test infrastructure, not a pages operation): the GPU's
 * reading of a DEV_V1 tensor, w = scale * q + bias as in "Why the runtime
 * has this shape".  codes_out uint8
 * [rows][cols] receives every code; w_out float [rows][cols] receives
 * scale * q + bias in fp32 (exact when the fp32 product is, e.g. for the
 * synthetic bias = -2^(bits-1) * scale). */
mq_status mq_debug_unpack_codes(const mq_qtensor* t, uint8_t* codes_out, void* stream);
mq_status mq_debug_dequant(const mq_qtensor* t, float* w_out, void* stream);

/* Routing only: the router input, projection, top-k and softmax weights of
 * moe_layer_forward for every token of x ("Decode": the first phase ends
 * when the top-8 ids are ready for the CPU to read, before it plans the
 * expert reads).  ids int32 [T][top_k] and w float [T][top_k] (device,
 * required), logits float [T][E] (optional).  The workspace holds
 * mq_route_workspace_bytes(router, T) bytes (256-byte aligned, no clearing).
 * Errors as moe_layer_forward. */
size_t mq_route_workspace_bytes(const mq_router* router, int32_t max_tokens);
mq_status mq_route(const mq_act* x, const mq_router* router, int32_t* ids, float* w, float* logits,
                   void* workspace, size_t workspace_bytes, void* stream);

/* HOST: the expert slot cache of a pool kept in host memory ("Load and
 * ownership": a fixed group of slots per layer, the cache records which
 * expert occupies each slot, least-frequently-used eviction with recency
 * as the tie-breaker, a hit reuses its slot, a miss takes an evictable slot
 * and starts a read, no two reads into one slot).  The state is a caller
 * buffer of mq_lfu_state_bytes (8-byte aligned) set up by mq_lfu_init.
 * mq_lfu_plan takes the n expert ids one layer call will use (repeats
 * allowed) and, for each, the slot that holds it after the plan
 * (slot_of_id [n]); every distinct expert counts one use; missing experts
 * get slots that no expert of this call holds, empty slots first, then the
 * resident expert with the fewest uses, ties to the one used longest ago,
 * then the lower slot; the misses to fill are (miss_expert, miss_slot)
 * [*n_miss] (arrays of n entries).  More distinct experts than slots, or an
 * id outside [0, num_experts): MQ_ERR_SHAPE with the state unchanged.  The
 * caller keeps slot reads ordered after the device work that last used the
 * slot ("Correctness and safety invariants": a queued consumer owns its
 * slot until completion). */
size_t mq_lfu_state_bytes(int32_t num_experts, int32_t num_slots);
mq_status mq_lfu_init(void* state, size_t state_bytes, int32_t num_experts, int32_t num_slots);
mq_status mq_lfu_plan(void* state, size_t state_bytes, const int32_t* ids, int32_t n, int32_t* slot_of_id,
                      int32_t* miss_expert, int32_t* miss_slot, int32_t* n_miss);

/* The same affine dequant-GEMV at other shapes: the tied 4-bit head at the
 * end of decode ("Why the runtime has this shape": embedding and head share
 * one quantized matrix, final logit softcap 30.0; "Decode": after the last
 * layer the head returns the argmax token directly in the greedy
 * configuration) or any other projection.
 *   w: DEV_V1 [rows][cols], 4- or 8-bit, group 64 (16-byte aligned).
 *   x: bf16 [T][cols] token rows, T <= 8 and T * cols * 2.25 <= 60 KiB
 *      (the rows and their partial sums are staged on chip).
 *   y: optional ([T][rows], bf16 or f32): y = W x in fp32, then
 *      softcap * tanh(y / softcap) when softcap > 0 (0: none).
 *   argmax: optional int32 [T], the row of the largest (softcapped) value,
 *      equal values to the lower row, NaN ranking last; it needs a workspace
 *      of mq_qgemv_workspace_bytes(rows, T) (16-byte aligned; no clearing).
 * At least one of y and argmax.  Errors as moe_layer_forward. */
size_t mq_qgemv_workspace_bytes(int32_t rows, int32_t tokens);
mq_status mq_qgemv(const mq_qtensor* w, const mq_act* x, mq_act* y, float softcap, int32_t* argmax,
                   void* workspace, size_t workspace_bytes, void* stream);

/* Measurement: reads bytes of buf once with 16-byte streaming loads, the
 * access the expert kernels use, over `workgroups` workgroups of 256
 * threads, and writes one fold of the words per workgroup to sink
 * [workgroups].  It gives the HBM read rate the device reaches, which the
 * benchmark reports beside the vendor peak ("Correctness and safety
 * invariants": throughput evidence comes from production-mode runs, not slow
 * profiling modes).  buf 16-byte aligned, bytes a multiple of 16. */
mq_status mq_stream_read(const void* buf, size_t bytes, uint32_t* sink, int32_t workgroups, void* stream);

const char* mq_status_str(mq_status s);

#ifdef __cplusplus
}
#endif
#endif
