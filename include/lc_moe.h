/*
 * lc_moe -- forward pass of a mixture-of-experts layer with zero-computation experts,
 * for AMD Instinct MI355X (gfx950).
 *
 * The layer (LongCat-Flash article, itouyu.top; Italian kqgmpj.cn; French dhxrcw.cn;
 * section "Zero-computation experts"): the expert pool holds N FFN experts and Z
 * zero-computation experts that return their input unchanged.  A softmax router R
 * scores token x_t over all N+Z experts, p_t = softmax(W_r x_t).  An expert-specific bias
 * b_i, adjusted from recent expert usage and decoupled from the training loss (same
 * section, bias paragraph), is added to the scores only to choose the K experts of each
 * token; the chosen experts are combined with the unbiased scores as gates:
 *
 *   S_t  = K largest p_t,i + b_i  (equal values: lower index first)
 *   y_t  = sum_{i in S_t, i <  N} p_t,i * W_down,i (silu(W_gate,i x_t) * (W_up,i x_t))
 *        + sum_{i in S_t, i >= N} p_t,i * x_t
 *
 * so a token runs between 0 and K FFN experts.  The FFN experts are SwiGLU blocks
 * without biases, silu(a) = a / (1 + exp(-a)).  Experts 0..N-1 are FFN experts,
 * N..N+Z-1 are zero-computation experts.
 *
 * Conventions shared by every entry point
 *   - All array arguments are DEVICE pointers, row-major and contiguous, aligned to 16
 *     bytes; the caller owns them and keeps them alive until the stream work completes.
 *     The library allocates no device memory, never synchronises the stream and keeps no
 *     pointer after return.  Its only mutable global state is that of
 *     lc_moe_forward_noalloc: one static workspace array per GPU and a cache of its
 *     device addresses.
 *   - dtype LC_MOE_BF16: x, the three expert weight tensors and y are bf16;
 *     LC_MOE_F32: they are fp32.  The router weight W_r, the bias b and the gates are
 *     always fp32; arithmetic accumulates in fp32 (the router logits exactly as an fp32
 *     dot product of x with W_r).
 *   - Host-side checks (LC_MOE_E_NULLPTR, _SHAPE, _DTYPE, _ALIGN, _WORKSPACE) run before
 *     anything is enqueued: on those statuses nothing is enqueued and every output is left
 *     untouched.  LC_MOE_E_DEVICE reports a launch error from the HIP runtime; kernels of
 *     the same call launched before it may already be enqueued, so the outputs are then
 *     undefined.  Device faults surface at the caller's next synchronisation.  NaN or Inf
 *     inputs are outside the contract.
 *   - Results are deterministic: two calls with the same inputs give bitwise equal
 *     outputs (no floating-point atomics anywhere).
 *   - The header is C (C99 and later) and C++.  It takes hipStream_t from
 *     <hip/hip_runtime_api.h>, which needs __HIP_PLATFORM_AMD__ defined (hipcc defines it;
 *     a plain C or C++ compiler takes -D__HIP_PLATFORM_AMD__ -I<ROCm>/include).
 *   - Limits: T, d, N, K, I >= 1; Z >= 0; K <= N+Z; N+Z <= 4096; N <= 2048;
 *     d and I multiples of 8 for bf16 (4 for fp32); and every kernel launch of the shape
 *     within the device's grid (at most 2^32 - 1 work-items along x): this needs
 *     T*K < 2^24, and for layers with many experts' worth of tiles somewhat less.  A shape
 *     outside these limits gives LC_MOE_E_SHAPE (lc_moe_workspace_size returns 0).
 */
#ifndef LC_MOE_H
#define LC_MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LC_MOE_OK = 0,
  LC_MOE_E_NULLPTR = 1,   /* a required pointer is NULL                                */
  LC_MOE_E_SHAPE = 2,     /* a size is out of range (see the limits above)             */
  LC_MOE_E_DTYPE = 3,     /* dtype is neither LC_MOE_F32 nor LC_MOE_BF16              */
  LC_MOE_E_ALIGN = 4,     /* a pointer is not 16-byte aligned                          */
  LC_MOE_E_WORKSPACE = 5, /* workspace smaller than lc_moe_workspace_size()            */
  LC_MOE_E_DEVICE = 6     /* a HIP call or kernel launch reported an error             */
} lc_moe_status;

typedef enum { LC_MOE_F32 = 0, LC_MOE_BF16 = 1 } lc_moe_dtype;

/* Layer shape (host struct).  T tokens of width d; N FFN experts with SwiGLU
 * intermediate width I; Z zero-computation experts; K experts chosen per token. */
typedef struct {
  int32_t T, d, N, Z, K, I;
  int32_t dtype; /* lc_moe_dtype */
} lc_moe_shape;

/* Layer weights (host struct holding device pointers). */
typedef struct {
  const float* w_router; /* [N+Z][d] fp32: router R                                      */
  const float* bias;     /* [N+Z]    fp32: expert bias b, used for selection only         */
  const void* w_gate;    /* [N][I][d] dtype: SwiGLU gate projection of each FFN expert    */
  const void* w_up;      /* [N][I][d] dtype: SwiGLU up projection                        */
  const void* w_down;    /* [N][d][I] dtype: SwiGLU down projection                      */
  const void* fp8;       /* NULL, or the block-FP8 expert weights made by
                            lc_moe_quantize_weights; then the FFN uses them and w_gate,
                            w_up, w_down are not read (they may be NULL)                 */
  const void* packed;    /* NULL, or the bf16 expert weights re-laid by
                            lc_moe_pack_weights; then the FFN reads them instead of
                            w_gate, w_up, w_down (which may be NULL).  At most one of fp8
                            and packed may be set (else LC_MOE_E_DTYPE)                  */
  int32_t fp8_act;       /* 0, or nonzero with fp8 set: the FFN also quantizes its
                            activations (x, and H = silu(G) U) to block FP8 in 1 x 128
                            blocks and multiplies FP8 by FP8 on the matrix cores (see
                            lc_moe_quantize_activations).  Needs fp8 (else
                            LC_MOE_E_DTYPE) and d, I multiples of 64 with
                            T * K * I < 2^31 (else LC_MOE_E_SHAPE)                       */
} lc_moe_weights;

/* Stages of lc_moe_forward, in launch order (names from lc_moe_stage_name). */
#define LC_MOE_NUM_STAGES 5 /* route, permute, gate_up, down, combine */

/* Bytes of device workspace every entry point below needs for this shape (0 if the
 * shape is invalid).  The same workspace may be reused by consecutive calls on one
 * stream; calls that overlap in time need separate workspaces.  Pure host arithmetic. */
size_t lc_moe_workspace_size(const lc_moe_shape* shape);

/* Router and biased top-K (section "Zero-computation experts": softmax router R over
 * the whole N+Z pool, bias added for the choice only).
 *   x          [T][d] dtype        tokens
 *   w_router   [N+Z][d] fp32       router weights
 *   bias       [N+Z] fp32          expert bias
 *   topk_idx   [T][K] int32 (out)  chosen experts of each token, ordered by
 *                                  (p + b descending, expert index ascending)
 *   topk_gate  [T][K] fp32 (out)   their unbiased softmax probabilities p
 * p is computed in fp32: logits as fp32 dot products, max-subtracted exp, sum, divide;
 * the selection compares fp32 p + b. */
lc_moe_status lc_moe_route(const lc_moe_shape* shape, const void* x, const float* w_router,
                           const float* bias, int32_t* topk_idx, float* topk_gate,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Expert usage counts, the statistic a bias controller consumes (bias paragraph of the
 * same section: the bias follows recent expert usage).
 *   topk_idx       [T][K] int32       picks (values in 0..N+Z-1; a token may repeat an
 *                                     expert, each pick counts)
 *   load           [N+Z] int32 (out)  number of picks of each expert; sums to T*K
 *   ffn_per_token  [T] int32 (out)    number of FFN experts (index < N) among each
 *                                     token's picks, 0..K; may be NULL */
lc_moe_status lc_moe_expert_load(const lc_moe_shape* shape, const int32_t* topk_idx,
                                 int32_t* load, int32_t* ffn_per_token, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream);

/* Token permutation into expert-contiguous rows.  Zero-computation picks get no row:
 * they need no compute (section "Zero-computation experts").
 *   x            [T][d] dtype
 *   topk_idx     [T][K] int32        values in 0..N+Z-1; a token may pick an expert more
 *                                    than once, and every such pick gets its own row
 *                                    (the router's picks are always distinct; repeated
 *                                    ones take a slower, serial ranking of their block)
 *   ffn_offsets  [N+1] int32 (out)   exclusive prefix sum of the FFN experts' loads;
 *                                    ffn_offsets[N] = nnz, the number of FFN picks
 *   perm_token   [T*K] int32 (out)   token of each row; rows of expert e are
 *                                    ffn_offsets[e]..ffn_offsets[e+1]-1, in (token,
 *                                    pick) order; entries from nnz on are untouched
 *   slot_row     [T][K] int32 (out)  row of pick (t,k), -1 for a zero-computation pick
 *   x_perm       [T*K][d] dtype (out) x_perm[r] = x[perm_token[r]] for r < nnz; may be NULL
 *   load         [N+Z] int32 (out)   as lc_moe_expert_load; may be NULL */
lc_moe_status lc_moe_permute(const lc_moe_shape* shape, const void* x, const int32_t* topk_idx,
                             int32_t* ffn_offsets, int32_t* perm_token, int32_t* slot_row,
                             void* x_perm, int32_t* load, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);

/* Whole layer: route -> permute -> grouped SwiGLU FFN over the FFN picks only ->
 * combine.  For each token the combine accumulates in fp32, starting from zero: first
 * g * (expert output) of each FFN pick, in pick order (one fused multiply-add per
 * element and pick); then, if the token has zero-computation picks, gz * x_t, where gz
 * is the fp32 sum of their gates taken in pick order; y is rounded once to dtype
 * (nearest even).  So the result equals the layer's sum with the identity experts'
 * terms grouped as (sum of their gates) * x_t.  Intermediates (gated activations H,
 * expert outputs) are stored in dtype (nearest even).  One stream, no host
 * synchronisation, capturable into a HIP graph.
 *   x          [T][d] dtype
 *   weights    host struct of device pointers (see lc_moe_weights)
 *   y          [T][d] dtype (out)
 *   topk_idx   [T][K] int32 (out, may be NULL)
 *   topk_gate  [T][K] fp32 (out, may be NULL)
 *   load       [N+Z] int32 (out, may be NULL) */
lc_moe_status lc_moe_forward(const lc_moe_shape* shape, const void* x,
                             const lc_moe_weights* weights, void* y, int32_t* topk_idx,
                             float* topk_gate, int32_t* load, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);

/* lc_moe_forward with instrumentation: when stage_events is not NULL it holds
 * LC_MOE_NUM_STAGES + 1 events created by the caller; event 0 is recorded on the stream
 * before the first stage and event i+1 after stage i.  Same results as lc_moe_forward.
 * A layer of at most 256 tokens runs the top-K and the permutation as one kernel; it is
 * counted in the route stage and the permute stage's span is empty. */
lc_moe_status lc_moe_forward_staged(const lc_moe_shape* shape, const void* x,
                                    const lc_moe_weights* weights, void* y, int32_t* topk_idx,
                                    float* topk_gate, int32_t* load, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream,
                                    hipEvent_t* stage_events);

/* lc_moe_forward for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same arguments as
 * lc_moe_forward without the workspace, same kernels, so the same results bit for bit.
 * The workspace is a file-scope device array of LC_MOE_STATIC_WORKSPACE_BYTES, one per
 * GPU, held from the library's load until the process ends; this entry point takes its
 * address (hipGetSymbolAddress) on its first call on each device and calls no allocating
 * routine.  Shapes whose lc_moe_workspace_size exceeds the array give LC_MOE_E_WORKSPACE
 * with nothing enqueued (every decode-sized layer fits: the 768-expert, d=6144, I=2048
 * layer needs 97 MB at T=256).  Nothing in the array needs to start at zero: every region
 * a kernel reads was written earlier in the same call.  All calls on one GPU share the
 * array, and it keeps the last call's contents: calls that overlap in time on one GPU (on
 * different streams, or from different host threads) race and give undefined results;
 * the caller must order them. */
#define LC_MOE_STATIC_WORKSPACE_BYTES ((size_t)128 << 20)
lc_moe_status lc_moe_forward_noalloc(const lc_moe_shape* shape, const void* x,
                                     const lc_moe_weights* weights, void* y, int32_t* topk_idx,
                                     float* topk_gate, int32_t* load, hipStream_t stream);

/* Block-FP8 expert weights.  The pages quantize with the fine-grained block scheme of
 * DeepSeek-V3 (LongCat-Flash article, section "System-level optimisation", quantization
 * paragraph) without fixing its details; this library takes: OCP FP8 E4M3 codes; one
 * scale per block of 128 rows x 128 reduction columns of every expert matrix (partial
 * blocks at the edges); the scale is a power of two, 2^k with k the smallest integer such
 * that the block's largest |w| <= 448 * 2^k; each w / 2^k is rounded to the nearest E4M3
 * value, ties to the even code.  By itself (fp8_act = 0) weights only: activations, H and
 * Y stay bf16, and the layer computed is the bf16 layer with every expert weight replaced
 * by code * 2^k (exact in bf16); with fp8_act the activations are quantized too (see
 * lc_moe_quantize_activations).  Blocks whose scale would fall below 2^-126 (max |w| < 448 * 2^-126) are
 * outside the contract.
 *
 * lc_moe_fp8_weights_size: bytes of the packed form for this shape; 0 when the shape
 * has none (fp32 layers, d or I not a multiple of 32, or d or I above 16384).
 * lc_moe_quantize_weights: writes the packed form (an opaque tile layout the FFN streams
 * plus the fp32 scales) of the bf16 W_gate, W_up [N][I][d] and W_down [N][d][I] into
 * fp8_weights (fp8_weights_bytes >= lc_moe_fp8_weights_size, 16-byte aligned).  Pass it
 * as lc_moe_weights.fp8.  Needs dtype LC_MOE_BF16 (else LC_MOE_E_DTYPE) and a shape
 * with a packed form (else LC_MOE_E_SHAPE). */
size_t lc_moe_fp8_weights_size(const lc_moe_shape* shape);
lc_moe_status lc_moe_quantize_weights(const lc_moe_shape* shape, const void* w_gate,
                                      const void* w_up, const void* w_down, void* fp8_weights,
                                      size_t fp8_weights_bytes, hipStream_t stream);

/* Block-FP8 activations (the same section and reading as the weights above, with blocks of
 * 1 row x 128 columns): the quantizer of lc_moe_weights.fp8_act, which applies it to x and,
 * inside the FFN, to H.  Each block of 128 consecutive columns of a row (the last one
 * partial) gets the scale 2^k, k the smallest integer with the block's max |v| <= 448 * 2^k
 * (k = 0 for an all-zero block), stored as the E8M0 byte k + 127; each v / 2^k rounds to
 * the nearest E4M3 code, ties to the even code.  The layer computed with fp8_act is then
 *   G = Q(x) Q(W_gate)^T, U = Q(x) Q(W_up)^T (exact products of dequantized values, summed
 *   by the FP8 matrix cores: about 12 bits below the largest addend per 64-element step,
 *   so G and U may be off by about 2^-13 (|G| + rss of the products), not fp32-exact),
 *   H = silu(G) U (fp32), Y = Q(H) Q(W_down)^T rounded to bf16,
 * combined as the bf16 layer's Y is.  Blocks whose max |v| is nonzero but below
 * 448 * 2^-127 are outside the contract.
 *   x       [rows][cols] bf16
 *   codes   [rows][cols] uint8 (out): E4M3 codes
 *   scales  [rows][ceil(cols / 128)] uint8 (out): E8M0 exponents k + 127
 * cols a multiple of 64 in [64, 16384], 0 <= rows < 2^24 (else LC_MOE_E_SHAPE); pointers
 * 16-byte aligned (LC_MOE_E_ALIGN) and non-NULL unless rows = 0 (LC_MOE_E_NULLPTR).
 * Enqueued on `stream`. */
lc_moe_status lc_moe_quantize_activations(const void* x, int32_t rows, int32_t cols, void* codes,
                                          void* scales, hipStream_t stream);

/* Packed bf16 expert weights: the same values as W_gate, W_up [N][I][d] and W_down
 * [N][d][I], re-laid so that every (expert, 128 gate/up or 256 down output columns, 32-wide
 * K step) tile is one contiguous 16 KB block in the order the FFN kernel stages it.  A
 * one-time copy, made when the weights are loaded, for callers that do this once at load
 * time: reading contiguous blocks streams the weights faster (about 5% for a layer of
 * many tokens, a few % at decode).  With more than 256 tokens the layer computed with it
 * is the same to the bit as with the row-major weights (one kernel, another address per
 * weight); with fewer, row-major weights take a kernel that adds the K steps in another
 * order, and the two agree to rounding.
 * lc_moe_packed_weights_size: bytes of the packed form for this shape (about the size of
 * the three expert matrices); 0 when the shape has none (fp32 layers, d or I not a
 * multiple of 32).
 * lc_moe_pack_weights: writes it into packed_weights (packed_weights_bytes >=
 * lc_moe_packed_weights_size, 16-byte aligned); pass that as lc_moe_weights.packed.  Needs
 * dtype LC_MOE_BF16 (else LC_MOE_E_DTYPE) and a shape with a packed form (else
 * LC_MOE_E_SHAPE); a short buffer gives LC_MOE_E_WORKSPACE.  Enqueued on `stream`; the
 * source weights must stay valid until it has run. */
size_t lc_moe_packed_weights_size(const lc_moe_shape* shape);
lc_moe_status lc_moe_pack_weights(const lc_moe_shape* shape, const void* w_gate,
                                  const void* w_up, const void* w_down, void* packed_weights,
                                  size_t packed_weights_bytes, hipStream_t stream);

/* Backward of the grouped SwiGLU FFN, for training.  The pages describe the model's
 * training (LongCat-Flash article, section "Model scaling and multi-stage training") but no
 * backward pass; this is the plain gradient of the layer's sum (section "Zero-computation
 * experts") with the routing held fixed: given the forward's picks topk_idx and gates
 * topk_gate and the gradient dy of the layer output y, it computes the gradients of
 * L = sum_t <dy_t, y_t> with respect to x and the three matrices of every FFN expert.  For
 * an FFN pick (t, i) with gate g, with G = W_gate x_t, U = W_up x_t, s = sigmoid(G),
 * a = G s, H = a U:
 *   dH = g W_down^T dy_t;  dG = dH U (s + a (1 - s));  dU = dH a
 *   dW_down += g dy_t H^T;  dW_gate += dG x_t^T;  dW_up += dU x_t^T
 *   dx_t += W_gate^T dG + W_up^T dU
 * and a zero-computation pick adds g dy_t to dx_t.  The router's gradient (through the
 * gates and the softmax) is not part of it.  bf16 layers with d and I multiples of 32
 * (else LC_MOE_E_DTYPE / LC_MOE_E_SHAPE); row-major weights (weights->w_gate, w_up,
 * w_down; the router, bias, fp8 and packed fields are not read).  Arithmetic: bf16
 * operands, fp32 accumulation; the row intermediates g*H, dG, dU and dX are rounded to
 * bf16, dH is kept in fp32; each token's dx adds its FFN picks' rows in pick order, then
 * its zero picks' gate sum times dy_t, in fp32, and is rounded once.  Deterministic.
 *   x          [T][d] bf16            the forward's input
 *   topk_idx   [T][K] int32, topk_gate [T][K] fp32   the forward's picks and gates
 *   dy         [T][d] bf16            gradient of y
 *   dx         [T][d] bf16 (out)
 *   dw_gate, dw_up [N][I][d], dw_down [N][d][I] bf16 (out); an expert without rows gets zeros
 * The workspace (lc_moe_backward_workspace_size; 0 for shapes without a backward) holds the
 * permutation of the picks, the x and dy rows gathered in FFN-row order and the row
 * intermediates: about (T*K) * (10*I + 6*d) bytes. */
size_t lc_moe_backward_workspace_size(const lc_moe_shape* shape);
lc_moe_status lc_moe_ffn_backward(const lc_moe_shape* shape, const void* x,
                                  const lc_moe_weights* weights, const int32_t* topk_idx,
                                  const float* topk_gate, const void* dy, void* dx, void* dw_gate,
                                  void* dw_up, void* dw_down, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream);

/* PID gains of the expert-bias controller (host struct). */
typedef struct {
  float kp, ki, kd;
} lc_moe_pid;

/* Expert-bias controller: one update of the selection bias from the last step's loads.
 * The pages say only that the bias follows recent expert usage and that its update rule
 * is a PID controller adjusting it in real time, which keeps the activated parameters
 * per token within a band (LongCat-Flash article, section "Zero-computation experts",
 * bias paragraph).  Error signal and gains are not given; this library takes, for every
 * expert i of the pool (FFN and zero-computation alike), in fp32:
 *   e_i        = target_i - load_i / (T*K)           (load_i and T*K converted to fp32,
 *                                                     IEEE division)
 *   integral_i = integral_i + e_i
 *   bias_i     = bias_i + (kp*e_i + ki*integral_i + kd*(e_i - prev_err_i))
 *   prev_err_i = e_i
 * so an expert picked less often than its target share gains bias.  Targets on the
 * zero-computation experts set the zero share of the picks, hence the mean number of FFN
 * experts per token.
 *   gains      host struct {kp, ki, kd}
 *   load       [N+Z] int32            picks per expert (lc_moe_expert_load / lc_moe_forward)
 *   target     [N+Z] fp32             target share of the T*K picks per expert (the
 *                                     caller's choice; normally summing to 1)
 *   bias       [N+Z] fp32 (in/out)
 *   integral   [N+Z] fp32 (in/out)    running sum of the errors; zero before the first call
 *   prev_err   [N+Z] fp32 (in/out)    previous error; zero before the first call, so the
 *                                     first derivative term is kd*e_i
 * Reads T, K, N, Z of shape (which must pass the usual checks).  bias, integral and
 * prev_err may not alias each other or load/target. */
lc_moe_status lc_moe_bias_update(const lc_moe_shape* shape, const lc_moe_pid* gains,
                                 const int32_t* load, const float* target, float* bias,
                                 float* integral, float* prev_err, hipStream_t stream);

/* Static strings; never NULL. */
const char* lc_moe_status_str(lc_moe_status status);
const char* lc_moe_stage_name(int stage);

#ifdef __cplusplus
}
#endif
#endif /* LC_MOE_H */
