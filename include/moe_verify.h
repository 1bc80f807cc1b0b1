/*
 * moe_verify.h -- C ABI of the MI355X (gfx950) block-verify MoE layer.
 *
 * What it computes.  One mixture-of-experts FFN layer of a target model that
 * verifies K draft rows in one pass (speculative block verify).  Per layer:
 *   1. router GEMV:  logits[r][e] = sum_h x[r][h] * Wr[e][h]   (bf16 in,
 *      fp32 accumulate; routers stay bf16 -- mlxfast README, "Why this
 *      challenge exists");
 *   2. selection: top-k experts per row by key, ties to the lower expert
 *      index; key = logit (softmax scoring) or fp32 sigmoid(logit) + bias
 *      (the router tail of PR #844 section 4, item 3); mixture weights are
 *      the softmax renormalised over the selected set, or the sigmoids
 *      (renormalised when norm_topk) -- the bias only selects;
 *   3. cross-row dedup: the distinct experts of all K*k slots, ascending,
 *      with a CSR of their slots (PR #844 section 8 notes the stock gather
 *      reads a repeated expert once per slot; here each is streamed once);
 *   4. NVFP4 dequantisation inside the GEMM loops: W = e2m1(q) * e4m3(s) * ts
 *      (README: expert projections are NVFP4 4-bit group-16);
 *   5. gate/up GEMM + SwiGLU: h = silu(x Wg^T) * (x Wu^T), fp32;
 *   6. down GEMM: o = h Wd^T, fp32;
 *   7. shared expert: the same FFN on every row with weight 1 (ungated);
 *   8. combine, in the order of PR #844 section 4 item 4 / section 5:
 *        y[r] = routed_scale * sum_j w[r][j] * o[r][j]  + shared[r]
 *               (+ residual[r])
 *      summed over j in rank order (deterministic; no atomics).
 *   9. stack glue: layer l+1 consumes bf16(gamma_l * RMSNorm(y_l)), eps =
 *      rms_eps, gamma_l = layer l's norm_w (ones when NULL); optionally the
 *      decoder's residual stream (PR #844 section 4 item 4): layer 0 adds
 *      the caller's residual, layer l >= 1 adds bf16(y_{l-1}); the stack
 *      returns the last layer's y.
 *
 * Activation range.  bf16 activations of any finite magnitude are accepted.
 * On the matrix cores (gate/up) each row enters as fp16 of x * 2^-sig, sig
 * = ilogb(max_row |x|) - 14: values within 2^-28 of the row's largest
 * magnitude are exact, smaller ones keep an absolute precision of
 * 2^-24 * 2^sig (below 2^-38 of the row maximum), nothing overflows; the
 * sums are multiplied by 2^sig.  Intermediates are fp32: outputs whose true
 * value exceeds the fp32 range (SwiGLU is quadratic in x, so |x| beyond
 * about 1e17 at the benchmark's weight scale) come out infinite, as in any
 * fp32 evaluation.
 *
 * Conventions for every entry point.
 *  - All array pointers are DEVICE pointers owned by the caller; the structs
 *    themselves (moe_cfg, moe_layer_weights, moe_route_out, moe_debug) live
 *    in host memory.  Arrays must be 16-byte aligned.
 *  - bf16 values are passed as uint16_t bit patterns.
 *  - NVFP4 matrix of `rows x cols` per expert (moe_nvfp4):
 *      q  uint8 [E][rows][cols/2]  two E2M1 codes per byte; the even column
 *                                  in the low nibble, the odd column in the
 *                                  high nibble (sign = bit 3 of a nibble);
 *      s  uint8 [E][rows][cols/16] OCP E4M3FN scale per 16 consecutive
 *                                  columns of a row;
 *      ts fp32  [E]                one tensor scale per expert matrix.
 *    gate/up: rows = inter, cols = hidden;  down: rows = hidden, cols = inter.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *    and the call returns without synchronising.  Nothing is allocated on the
 *    device: scratch lives in the caller's workspace.
 *  - Return codes: MOE_OK, or a negative MOE_ERR_*; the thread-local text of
 *    the last error is available from moe_verify_last_error().  There is no
 *    silent fallback: an unsupported configuration is an error.
 */
#ifndef MOE_VERIFY_H
#define MOE_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define MOE_API __attribute__((visibility("default")))
#else
#define MOE_API
#endif

#define MOE_OK 0
#define MOE_ERR_INVALID (-1)      /* null/misaligned pointer, K out of range, bad enum */
#define MOE_ERR_UNSUPPORTED (-2)  /* a shape this library does not implement */
#define MOE_ERR_HIP (-3)          /* a HIP runtime call failed (text has hipGetErrorString) */
#define MOE_ERR_WORKSPACE (-4)    /* workspace smaller than moe_verify_workspace_bytes() */

#define MOE_SCORE_SOFTMAX 0       /* select on logits; weights = softmax over the selection */
#define MOE_SCORE_SIGMOID_BIAS 1  /* select on fp32 sigmoid(logit) + bias; weights = sigmoid */

/* Shape regime (moe_cfg.regime): the same computation by two kernel families.
 * AUTO runs the verify-width kernels below 8 rows and the grouped kernels
 * from 8 rows (when the shape meets the grouped limits; always above 16);
 * VERIFY forces the verify-width kernels (K <= 16, MOE_ERR_UNSUPPORTED
 * above); GROUPED forces the grouped kernels at any K (their limits apply).
 * VERIFY_ONE_LAUNCH is VERIFY with a layer of at most 2 rows run as one
 * launch when its down tasks fit the launch (same results bit for bit; the
 * two-launch layer is faster on MI355X, so AUTO and VERIFY use it). */
#define MOE_REGIME_AUTO 0
#define MOE_REGIME_VERIFY 1
#define MOE_REGIME_GROUPED 2
#define MOE_REGIME_VERIFY_ONE_LAUNCH 3

typedef struct moe_nvfp4 {
    const uint8_t* q;
    const uint8_t* s;
    const float* ts;
} moe_nvfp4;

typedef struct moe_cfg {
    int32_t hidden;        /* H */
    int32_t n_experts;     /* E routed experts */
    int32_t top_k;         /* k */
    int32_t inter;         /* I, routed expert intermediate */
    int32_t shared_inter;  /* I_s of the one shared expert; 0 = none */
    int32_t score_fn;      /* MOE_SCORE_* */
    int32_t norm_topk;     /* 1 = divide the selected weights by their sum
                              (required with MOE_SCORE_SOFTMAX) */
    float routed_scale;    /* multiplies the weighted routed sum (2.5 on the
                              pages' checkpoint, 1.0 for plain softmax MoE) */
    float rms_eps;         /* RMSNorm epsilon between stacked layers */
    int32_t max_rows;      /* largest K a workspace of this cfg serves
                              (1..1024; above 16 the cfg must also meet the
                              grouped-regime limits below) */
    int32_t regime;        /* MOE_REGIME_*: which kernels serve K rows */
} moe_cfg;

typedef struct moe_layer_weights {
    const uint16_t* router_w;  /* bf16 [E][H] */
    const float* router_bias;  /* fp32 [E]; required iff score_fn == SIGMOID_BIAS,
                                  must be NULL otherwise */
    moe_nvfp4 gate, up, down;  /* E experts */
    moe_nvfp4 sh_gate, sh_up, sh_down;  /* one expert; all NULL iff shared_inter == 0 */
    const uint16_t* norm_w;    /* stack only: bf16 [H] RMSNorm weight applied to this
                                  layer's output to form the next layer's input;
                                  NULL = ones.  Ignored for the last layer of a
                                  stack and by the single-layer entry points. */
} moe_layer_weights;

/* Outputs of the selection step (device arrays, K = rows of the call):
 *   ids [K][k] int32 selected experts in rank order; w [K][k] fp32 mixture
 *   weights (routed_scale not folded in); n_unique [1]; uniq [K*k] distinct
 *   experts ascending (first n_unique valid); off [K*k+1] CSR offsets
 *   (first n_unique+1 valid); asg [K*k] flat slots r*k+j grouped by expert,
 *   ascending within an expert; inv [K*k] position of each slot in asg. */
typedef struct moe_route_out {
    int32_t* ids;
    float* w;
    int32_t* n_unique;
    int32_t* uniq;
    int32_t* off;
    int32_t* asg;
    int32_t* inv;
} moe_route_out;

/* Optional per-layer copies of intermediates (device arrays, any may be
 * NULL).  For a stack of L layers each array holds L consecutive per-layer
 * blocks of the sizes in moe_route_out (logits: [K][E] fp32), plus
 * x_in [K][H] bf16 (the layer's input), y32 [K][H] fp32 (its output) and
 * res_in [K][H] bf16 (the residual it added; written only when the call has
 * a residual). */
typedef struct moe_debug {
    float* logits;
    int32_t* ids;
    float* w;
    int32_t* n_unique;
    int32_t* uniq;
    int32_t* off;
    int32_t* asg;
    int32_t* inv;
    uint16_t* x_in;
    float* y32;
    uint16_t* res_in;
    int32_t* status;    /* [1] per layer: 0, or nonzero when an in-kernel hand-off
                           wait gave up (the layer's results are then invalid) */
} moe_debug;

/* Bytes of device workspace that layer/stack/route calls with this cfg need
 * (K <= cfg->max_rows).  0 if cfg is invalid (see moe_verify_last_error). */
MOE_API size_t moe_verify_workspace_bytes(const moe_cfg* cfg);

/* One layer (steps 1-8) on bf16 rows x [K][H].  residual (bf16 [K][H]) may be
 * NULL.  Writes y bf16 [K][H] (round to nearest even of y32) and, if y32 is
 * not NULL, the fp32 result.  dbg may be NULL.
 *
 * Two shape regimes of the same computation, picked by K and cfg->regime
 * (MOE_REGIME_*; AUTO: verify width below 8 rows, grouped from 8 rows when
 * the shape meets the grouped limits, grouped above 16 rows):
 *  - verify width (K <= 16): every unique expert is streamed once by
 *    skinny kernels: router + selection + gate/up in one launch, whose
 *    gate/up workgroups wait for the router workgroups of the same launch
 *    through a bounded in-kernel hand-off, then down + combine (with
 *    MOE_REGIME_VERIFY_ONE_LAUNCH at K <= 2 the down workgroups are part of
 *    the same launch, holding their down weights while gate/up runs and
 *    waiting, bounded, for every gate/up workgroup's h);
 *  - grouped (prefill, e.g. the 512-row seed prefill of the mlxfast README,
 *    "Why this challenge exists", and wide verify blocks): the T*k slots are
 *    grouped by expert into tiles of up to 32 tokens and the expert GEMMs
 *    run on the matrix cores (six launches).  Limits: inter and shared_inter
 *    multiples of 64 and at most 1024 (MOE_ERR_UNSUPPORTED when the grouped
 *    kernels are required).  h enters the down GEMM as a pair of fp16 values
 *    (hi + lo) of h scaled by a per-token power of two, about 22 significant
 *    bits. */
MOE_API int moe_verify_layer(const moe_cfg* cfg, const moe_layer_weights* w, const uint16_t* x, int32_t K,
                     const uint16_t* residual, uint16_t* y, float* y32, void* workspace,
                     size_t workspace_bytes, void* stream, const moe_debug* dbg);

/* moe_verify_layer with the grouped (prefill) kernels at any K <= max_rows,
 * including K <= 16: the same arguments, outputs and errors, plus the
 * grouped-regime limits.  For tests and for callers that batch prefill rows
 * in small groups. */
MOE_API int moe_verify_layer_grouped(const moe_cfg* cfg, const moe_layer_weights* w, const uint16_t* x,
                                     int32_t K, const uint16_t* residual, uint16_t* y, float* y32,
                                     void* workspace, size_t workspace_bytes, void* stream,
                                     const moe_debug* dbg);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * moe_verify_layer with the same arguments, outputs and errors, but no
 * workspace argument -- its scratch is a fixed device array inside the
 * library, moe_verify_noalloc_scratch_bytes() bytes (5 MiB: the full-size
 * layer up to 40 rows), one per GPU, held until the process ends.  A cfg
 * whose workspace (moe_verify_workspace_bytes) exceeds it returns
 * MOE_ERR_UNSUPPORTED before any device work.  The call allocates nothing:
 * the array's device address is looked up once per device (with that
 * device current) on the first call there.  Every call on a GPU shares that
 * GPU's array and nothing in it needs to start at zero; calls that overlap
 * on one GPU (two streams, two threads) race on it and must be serialised
 * by the caller. */
MOE_API int moe_verify_layer_noalloc(const moe_cfg* cfg, const moe_layer_weights* w, const uint16_t* x, int32_t K,
                                     const uint16_t* residual, uint16_t* y, float* y32, void* stream,
                                     const moe_debug* dbg);
MOE_API size_t moe_verify_noalloc_scratch_bytes(void);

/* n_layers layers (steps 1-9).  layers is a HOST array of n_layers weight
 * structs.  x bf16 [K][H] is layer 0's input.  residual (bf16 [K][H]) NULL:
 * no residual anywhere; given: the residual stream -- layer 0 adds
 * `residual`, layer l >= 1 adds layer l-1's bf16 output (the decoder
 * residual of PR #844 section 4 item 4 carried through the stack).  Layer
 * l+1's input is bf16(norm_w_l * RMSNorm(y_l)).  Writes the last layer's
 * output to y (bf16) and y32 (fp32, may be NULL).  dbg may be NULL.  K and
 * cfg->regime pick the kernels as in moe_verify_layer. */
MOE_API int moe_verify_stack(const moe_cfg* cfg, const moe_layer_weights* layers, int32_t n_layers,
                     const uint16_t* x, const uint16_t* residual, int32_t K, uint16_t* y, float* y32,
                     void* workspace, size_t workspace_bytes, void* stream, const moe_debug* dbg);

/* Profiling aid: the work of moe_verify_stack (no debug copies), with each
 * kernel launched so that a start/stop event pair carries that kernel's own
 * dispatch timestamps.  Synchronises `stream`, then writes the durations in
 * milliseconds to the HOST array kernel_ms[n_layers][2] (router + selection
 * + gate/up + SwiGLU, down + combine; a one-launch layer reports the whole
 * launch first and 0 second), and returns MOE_ERR_HIP if an
 * in-kernel hand-off wait gave up.  Verify-width kernels only
 * (MOE_ERR_UNSUPPORTED when K and cfg->regime pick the grouped ones). */
MOE_API int moe_verify_stack_timed(const moe_cfg* cfg, const moe_layer_weights* layers, int32_t n_layers,
                                   const uint16_t* x, const uint16_t* residual, int32_t K, uint16_t* y,
                                   float* y32, void* workspace, size_t workspace_bytes, void* stream,
                                   float* kernel_ms);

/* Measurement aid: read `bytes` (a positive multiple of 16) of device memory
 * at src (16-byte aligned) once, as a plain streaming read: each workgroup
 * reads its own contiguous range with non-temporal 16-byte loads, several per
 * thread in flight (the fastest of the read patterns measured on MI355X).
 * A thread whose XOR of the data it read equals a fixed constant stores it
 * to the device word *sink, so the reads cannot be dropped; *sink carries no
 * other meaning.  Timed by the caller: the read ceiling the layer's
 * bandwidth figures are compared with.  Asynchronous on `stream`. */
MOE_API int moe_verify_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

/* Selection only (steps 2-3) from given fp32 logits [K][E] (device), with
 * the same selection code the layer uses.  bias as in moe_layer_weights.
 * For K > 16 the grouped regime's selection kernel runs, then a grouping
 * kernel that builds the same CSR the layer's gate/up workgroups rebuild for
 * themselves, and the workspace (sized by moe_verify_workspace_bytes) is
 * required; for K <= 16 workspace may be NULL. */
MOE_API int moe_verify_route(const moe_cfg* cfg, const float* logits, const float* bias, int32_t K,
                     const moe_route_out* out, void* workspace, size_t workspace_bytes, void* stream);

/* Step 4 alone: dequantise n_experts expert matrices of rows x cols into
 * fp32 out [E][rows][cols]: e2m1(code) * e4m3(scale), then one fp32 multiply
 * by ts.  The product is formed by each decode the GEMM kernels use -- the
 * fp32 convert and multiply of the down kernels, the bf16 convert, and the
 * fp16 operand decode of the gate/up matrix-core tiles (fp16 convert, then a
 * packed fp16 multiply by the scale) -- and is NaN where they disagree.
 * (In the GEMMs the tensor scale, and in the verify-width down kernel also
 * the block scale, multiply partial sums rather than each weight.) */
MOE_API int moe_verify_dequant_nvfp4(const moe_nvfp4* m, int32_t n_experts, int32_t rows, int32_t cols,
                             float* out, void* stream);

/* A captured stack launch (hipGraph) of moe_verify_stack.  It bakes in cfg,
 * the weight pointers, K, x, residual, y, y32 and the workspace; re-create
 * it when any of them changes.  A handle must not be launched from two
 * threads at once. */
typedef struct moe_stack_graph moe_stack_graph;
MOE_API int moe_stack_graph_create(const moe_cfg* cfg, const moe_layer_weights* layers, int32_t n_layers,
                           const uint16_t* x, const uint16_t* residual, int32_t K, uint16_t* y, float* y32,
                           void* workspace, size_t workspace_bytes, void* stream, moe_stack_graph** out);
MOE_API int moe_stack_graph_launch(moe_stack_graph* g, void* stream);
MOE_API void moe_stack_graph_destroy(moe_stack_graph* g);

/* ------------------------------------------------------------------------
 * The step after the MoE stack: the verify rows' lm_head and greedy block
 * acceptance.  logits[r][v] = sum_h x[r][h] * W[v][h] for EVERY verify row
 * (PR #844 section 5, trap 1: the verifier needs one greedy token per verify
 * row; section 2: W is bf16 [100352][2048], 0.41 GB), bf16 inputs with fp32
 * accumulation; row r's greedy token is its argmax (ties to the lower token
 * id).  Row r >= 1's input token is the draft token draft[r-1], so draft[j]
 * is accepted when it equals row j's greedy token or its logit ties row j's
 * maximum within tie_tol (mlxfast README, "Correctness fixtures": an exact
 * match, or a top-logit tie within 1e-6; 0 = plain greedy); a step keeps the
 * longest accepted prefix plus the greedy token of the first row it does not
 * cover.  A draft token outside [0, vocab) is never accepted.
 * ------------------------------------------------------------------------ */
typedef struct moe_greedy_out {
    int32_t* target;        /* [K] greedy token of each row */
    float* target_logit;    /* [K] its logit */
    int32_t* n_accepted;    /* [1] accepted draft tokens a (0 .. K-1) */
    int32_t* emitted;       /* [K] the a accepted draft tokens, then row a's greedy token (first a + 1 valid) */
    int32_t* n_emitted;     /* [1] a + 1 */
} moe_greedy_out;

/* Device workspace of moe_verify_lm_head_greedy (0 when the arguments are
 * invalid). */
MOE_API size_t moe_verify_lm_head_workspace_bytes(int32_t vocab, int32_t K);

/* x bf16 [K][hidden] device rows (K in [1, 16]; hidden 256, 512, 1024 or
 * 2048), w bf16 [vocab][hidden] device, draft int32 [K-1] device (NULL
 * allowed when K == 1), logits fp32 [K][vocab] device or NULL (then only the
 * greedy results are written), out: device arrays (struct in host memory).
 * Asynchronous on `stream`; errors as elsewhere (MOE_ERR_WORKSPACE when
 * workspace_bytes is short). */
MOE_API int moe_verify_lm_head_greedy(const uint16_t* x, int32_t K, const uint16_t* w, int32_t vocab, int32_t hidden,
                                      const int32_t* draft, float tie_tol, float* logits, const moe_greedy_out* out,
                                      void* workspace, size_t workspace_bytes, void* stream);

/* Algorithmic HBM bytes of one layer step: the router (if with_router), each
 * of n_unique routed experts once, the shared expert (if with_shared and
 * cfg->shared_inter > 0), x in and y out (bf16, K rows).  NVFP4 matrices
 * count codes + scales + the fp32 tensor scale. */
MOE_API size_t moe_verify_weight_bytes(const moe_cfg* cfg, int32_t n_unique, int32_t K, int32_t with_shared,
                               int32_t with_router);

/* Text of the last error on this thread ("" if none). */
/* ------------------------------------------------------------------------
 * The target's dense first layer and the prefill stack (mlxfast README, "Why
 * this challenge exists": layer 0 carries a dense SwiGLU MLP of intermediate
 * 8192 ahead of the MoE layers; PR #844 section 3: the 512-row seed prefill
 * runs through the same layers).  y[t] = W_down (silu(W_gate x_t) .*
 * (W_up x_t)) (+ residual[t]): bf16 weights and rows, fp32 sums of exact
 * bf16 products on the matrix cores; h enters the down GEMM as two bf16
 * values (hi + lo: 16 significant bits, any magnitude).
 * ------------------------------------------------------------------------ */
typedef struct moe_dense_weights {
    const uint16_t* gate;    /* bf16 [inter][hidden] */
    const uint16_t* up;      /* bf16 [inter][hidden] */
    const uint16_t* down;    /* bf16 [hidden][inter] */
    const uint16_t* norm_w;  /* bf16 [hidden] RMSNorm weight applied to this layer's
                                output to form the next input; NULL = ones */
} moe_dense_weights;

/* Device workspace of moe_dense_mlp for up to max_rows rows; 0 (see
 * moe_verify_last_error) when the shape is unsupported: hidden a multiple of
 * 64 in [64, 2048], inter a multiple of 256, max_rows >= 1. */
MOE_API size_t moe_dense_workspace_bytes(int32_t hidden, int32_t inter, int32_t max_rows);

/* The dense layer on bf16 rows x [T][hidden] (T >= 1; all arrays device,
 * 16-byte aligned).  residual (bf16 [T][hidden]) may be NULL.  Writes y bf16
 * [T][hidden] (RNE of y32), y32 fp32 [T][hidden] (required) and, when x_next
 * is not NULL, the next stacked layer's input bf16(norm_w * y32 /
 * sqrt(mean(y32^2) + eps)) with fp32 arithmetic.  The workspace holds at
 * least moe_dense_workspace_bytes(hidden, inter, T).  Asynchronous on
 * `stream`; errors as elsewhere. */
MOE_API int moe_dense_mlp(const uint16_t* x, int32_t T, int32_t hidden, int32_t inter, const moe_dense_weights* w,
                          const uint16_t* residual, float eps, uint16_t* y, float* y32, uint16_t* x_next,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Device workspace of moe_prefill_stack: the MoE layers' workspace for cfg,
 * then the dense layer's for cfg->max_rows rows and its output buffers; 0
 * when cfg or the dense shape is invalid. */
MOE_API size_t moe_prefill_workspace_bytes(const moe_cfg* cfg, int32_t dense_inter);

/* The prefill stack: the dense layer on x (T rows), then n_layers >= 1 MoE
 * layers exactly as moe_verify_stack runs them on the dense layer's
 * normalised output (the kernels cfg->regime picks for T rows).  The glue
 * between the dense layer and the first MoE layer is the stack's (the dense
 * weights' norm_w, cfg->rms_eps); with a residual, the dense layer adds it
 * and the first MoE layer adds bf16 of the dense output (the residual
 * stream).  y/y32 as moe_verify_stack.  dense_y32 (nullable, fp32
 * [T][hidden]) receives the dense layer's output; dbg (nullable) covers the
 * MoE layers as moe_verify_stack's does. */
MOE_API int moe_prefill_stack(const moe_cfg* cfg, const moe_dense_weights* dense, int32_t dense_inter,
                              const moe_layer_weights* layers, int32_t n_layers, const uint16_t* x,
                              const uint16_t* residual, int32_t T, uint16_t* y, float* y32, float* dense_y32,
                              void* workspace, size_t workspace_bytes, void* stream, const moe_debug* dbg);

/* ------------------------------------------------------------------------
 * The verify step's sliding-window KV cache (PR #844 section 8 items 1-2,
 * section 10: at K >= 2 rows the sliding layers rebuilt their keys and
 * values by concatenation every step, about 0.126 GB of copies per step
 * (section 2), and a wrapped rotating cache could not drop rejected rows,
 * so a rejecting round replayed the forward; mlxfast README, "Why this
 * challenge exists": 512-token sliding windows, 8 KV heads of head_dim 128).
 *
 * A ring of `capacity` slots per layer and KV head holds position q in slot
 * q % capacity.  A verify block of K rows writes its rows in place at the
 * positions len .. len+K-1 (len: a device counter, read by the kernels);
 * the commit keeps row 0 and the block's accepted drafts by advancing len
 * by 1 + n_accepted (read on the device, e.g. moe_greedy_out.n_accepted),
 * which drops the rejected rows without moving data.  capacity must be at
 * least window + K - 1 (moe_kv_ring_capacity), so no position that a row of
 * the block, or of the next block after any rollback, can see is ever
 * overwritten.  No host round trip: a step is graph-capturable.
 *
 * Ownership: the caller allocates k, v and len (moe_kv_ring_bytes each for
 * k and v) and keeps them alive while work on the ring is queued; the
 * library holds no pointer after a call returns.  A ring's calls are
 * ordered by the stream they are queued on: calls on different streams that
 * overlap race on its length and slots.
 * ------------------------------------------------------------------------ */
typedef struct moe_kv_ring {
    uint16_t* k;       /* bf16 [n_layers][n_kv][capacity][head_dim], device */
    uint16_t* v;       /* the same layout for values */
    int32_t* len;      /* device int32 [1]: committed length */
    int32_t n_layers, n_kv, head_dim, window, capacity;
} moe_kv_ring;

/* Slots per ring for blocks of up to max_rows rows: window + max_rows - 1
 * (0 when window < 1 or max_rows < 1). */
MOE_API int32_t moe_kv_ring_capacity(int32_t window, int32_t max_rows);

/* Bytes of one of the ring's two arrays (keys or values). */
MOE_API size_t moe_kv_ring_bytes(int32_t n_layers, int32_t n_kv, int32_t head_dim, int32_t capacity);

/* Sets the committed length to len (>= 0) on `stream`. */
MOE_API int moe_kv_ring_reset(const moe_kv_ring* ring, int32_t len, void* stream);

/* Writes a block's rows: k_new, v_new bf16 [n_layers][K][n_kv][head_dim]
 * device, row r at position len + r.  Errors: MOE_ERR_INVALID for NULL or
 * misaligned pointers, head_dim not a positive multiple of 8, K < 1 or
 * capacity < window + K - 1. */
MOE_API int moe_kv_ring_write(const moe_kv_ring* ring, const uint16_t* k_new, const uint16_t* v_new, int32_t K,
                              void* stream);

/* Writes one layer's rows of a block: k_new, v_new bf16 [K][n_kv][head_dim]
 * device, row r at position len + r of `layer` (a forward writes each sliding
 * layer's new keys and values just before that layer's attention reads its
 * window).  Errors as moe_kv_ring_write, and MOE_ERR_INVALID for a layer
 * outside [0, n_layers). */
MOE_API int moe_kv_ring_write_layer(const moe_kv_ring* ring, int32_t layer, const uint16_t* k_new,
                                    const uint16_t* v_new, int32_t K, void* stream);

/* Commits the last written block of K rows: len += 1 + n_accepted, the
 * device count clamped to [0, K - 1]. */
MOE_API int moe_kv_ring_commit(const moe_kv_ring* ring, const int32_t* n_accepted, int32_t K, void* stream);

/* What the last written block's row r sees of `layer`, for r < K: k_out,
 * v_out bf16 [K][n_kv][window][head_dim] device, positions
 * len + r - window + 1 .. len + r oldest first, zeros before position 0.
 * Call between the block's write and its commit. */
MOE_API int moe_kv_ring_window(const moe_kv_ring* ring, int32_t layer, int32_t K, uint16_t* k_out, uint16_t* v_out,
                               void* stream);

MOE_API const char* moe_verify_last_error(void);

/* ABI version (major * 100 + minor). */
MOE_API int moe_verify_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_VERIFY_H */
