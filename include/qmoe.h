/*
 * qmoe.h -- C ABI of libqmoe.so, the MI355X (gfx950) quantized
 * Mixture-of-Experts (QMoE) FFN layer.
 *
 * The layer: top-k routing from router logits, expert grouping into sorted
 * offsets and a tile work-list, a grouped fc1 projection over block-wise
 * int2/int3/int4 packed weights dequantized in registers, a SwiGLU or GeGLU
 * gated activation, a grouped fc2 projection, and a routing-weighted combine.
 *
 * Sources (page title, then the named function or paragraph):
 *   [qmoe.rs]   docs.rs source page of onnx-runtime-ep-cuda, src/kernels/qmoe.rs
 *   [PR 32198]  onnxruntime pull request 32198, "[CUDA] QMoE: fused int2
 *               mixed-input GEMM + GeGLU activation + fractional zero-point"
 *   [PR 33569]  onnxruntime pull request 33569, "[CUDA] Add fast INT3 QMoE
 *               kernels and offline SM80 INT2/INT4 prepack support"
 *   [gemm_quant_moe.rs]  metrale_model_layers layers/ops/gemm_quant_moe.rs
 *
 * Conventions shared by every entry point
 *   - Every pointer argument except `stream` is a DEVICE pointer, owned by the
 *     caller; the library allocates nothing and frees nothing.  Tensors are
 *     dense row-major with no padding.
 *   - `stream` is a hipStream_t passed as void*; NULL is the legacy default
 *     stream.  Every call only enqueues work on `stream` and returns; nothing
 *     synchronizes the host.  Results are valid once the stream reaches them.
 *   - Return value: QMOE_OK (0) or a negative QMOE_ERR_* code.  All argument
 *     checks run before any launch, so on an error nothing was enqueued and no
 *     output was written.  qmoe_last_error() then returns a message (thread
 *     local, valid until the next call on the same thread).
 *   - Calls that overlap in time and share output or workspace buffers race;
 *     the library holds no state between calls except the optional kernel
 *     timer below.
 *   - Route r = t*top_k + s is slot s of token t.
 */
#ifndef QMOE_H
#define QMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define QMOE_OK 0
#define QMOE_ERR_INVALID_ARG (-1) /* bad shape, null pointer, alignment, value     */
#define QMOE_ERR_UNSUPPORTED (-2) /* valid op, but no kernel for this combination */
#define QMOE_ERR_WORKSPACE (-3)   /* workspace or work-list capacity too small     */
#define QMOE_ERR_HIP (-4)         /* a HIP runtime call or launch failed           */

/* activation dtypes (hidden states, scales, output) */
#define QMOE_DTYPE_F16 1
#define QMOE_DTYPE_BF16 2

/* gated activations on interleaved fc1 rows (row 2j = gate, 2j+1 = up)
 * [qmoe.rs, qmoe_activate with swiglu_fusion = 1; PR 32198, GeGLU uses the same
 * interleaved fc1 rows as SwiGLU with a tanh-GELU gate] */
#define QMOE_ACT_SWIGLU 0 /* silu(g) * u                                            */
#define QMOE_ACT_GEGLU 1  /* 0.5 g (1 + tanh(0.7978845608028654 (g + 0.044715 g^3))) * u */

/* Expanded-row count R = T*top_k at or below which qmoe_forward takes the
 * decode path (each selected expert's weights streamed once for all of its
 * rows); above it, the prefill grouped GEMM.  [PR 33569: GEMV dispatch for
 * up to 80 expanded rows] */
#define QMOE_DECODE_MAX_ROUTES 80

/*
 * One quantized projection of all E experts: N output rows of K inputs.
 *   codes        uint8 [E, N, K*bits/8].  2- and 4-bit codes fill each byte
 *                from the least significant bits up (code kk of a row sits in
 *                byte kk/(8/bits) at bit (kk%(8/bits))*bits) [qmoe.rs,
 *                decode_affine_weight].  3-bit codes come in 3-byte groups of
 *                8: code kk is bits [3(kk%8), 3(kk%8)+3) of the little-endian
 *                24-bit word of group kk/8 [PR 33569, 24-bit 8-code INT3
 *                unpacking].  16-byte aligned.
 *   scales       fp16/bf16 (the layer's dtype) [E, N, K/block_size]; block
 *                b covers inputs [b*block_size, (b+1)*block_size).  2-byte
 *                aligned (16-byte alignment lets the decode kernels stage a
 *                row's scales with 16-byte loads).
 *   zero_points  NULL, or uint8 [E, N, Z]: bits-wide values packed like the
 *                2/4-bit codes with Z = ceil((K/block_size)/(8/bits)), or one
 *                byte per block for bits = 3 (Z = K/block_size).
 *   bits         1, 2, 3, 4 or 8 (1 and 8 as [qmoe.rs, QMoEFactory::create]
 *                accepts them: codes packed LSB-first like 2/4 bits, centre
 *                2^(bits-1)).
 * Dequantized weight: W[e,n,kk] = (code - zp) * scale[e,n,kk/block_size]
 * where zp is the zero_points entry if the tensor is given, else the layer's
 * zero_point_offset if it is not NaN, else the symmetric centre 2^(bits-1)
 * [qmoe.rs, decode_affine_weight; PR 32198, zero_point_offset].
 */
typedef struct qmoe_proj {
    const uint8_t* codes;
    const void* scales;
    const uint8_t* zero_points;
    int32_t bits;
} qmoe_proj;

/* Message describing the last error returned on this thread ("" if none). */
const char* qmoe_last_error(void);

/*
 * Top-k routing [qmoe.rs, total_order_key, route_value_is_better, qmoe_route].
 *   logits        float32 [T, E]
 *   topk_ids      int32 [T, top_k] out: the top_k experts of each token in
 *                 descending order of the route key, equal keys to the lower
 *                 index.  The key orders float32 bit patterns totally (-0
 *                 below +0, +NaN above +inf, -NaN below -inf).
 *   topk_weights  float32 [T, top_k] out: exp(l - m) / D with m the largest
 *                 non-NaN logit of the token; D sums exp(l - m) over the
 *                 selected experts if normalize, else over all E experts.
 * Requires T >= 0, 1 <= E <= 1024, 1 <= top_k <= E, normalize in {0, 1}.
 */
int qmoe_route(const float* logits, int64_t T, int32_t E, int32_t top_k, int32_t normalize,
               int32_t* topk_ids, float* topk_weights, void* stream);

/*
 * Router projection fused with top-k routing, one launch
 * [gemm_quant_moe.rs, moe_gate_topk_fused: gate logits = input row times the
 * transposed gate weight, then the top-k expert indices and weights of those
 * logits; moe.rs, the router GEMM before routing].
 *   hidden        dtype [T, H] (16-byte aligned)
 *   gate_weight   dtype [E, H] row-major (16-byte aligned): one row per expert
 *   logits_out    NULL or float32 [T, E] out: sum_h hidden[t,h] * gate[e,h],
 *                 products and sums in float32 (the values routed on; they can
 *                 be passed to qmoe_forward as its logits)
 *   topk_ids, topk_weights   as qmoe_route computes them from those logits
 * Requires 1 <= E <= 1024, 1 <= top_k <= E, H a multiple of 32 (else
 * QMOE_ERR_UNSUPPORTED).  T = 0 returns QMOE_OK and enqueues nothing.
 */
int qmoe_router(const void* hidden, const void* gate_weight, int64_t T, int32_t H, int32_t E,
                int32_t dtype, int32_t top_k, int32_t normalize, float* logits_out,
                int32_t* topk_ids, float* topk_weights, void* stream);

/* Work-list capacity (items) that always suffices for qmoe_group with these
 * arguments: (ceil(R/m_tile) + min(E, R)) * ceil(N/n_tile), R = T*top_k
 * [gemm_quant_moe.rs, moe_build_tile_worklist: one item per m-tile and
 * n-tile of every expert that has rows; with at most min(E, R) such experts,
 * each contributes at most one partial m-tile beyond ceil(R/m_tile)].
 * Returns -1 on invalid arguments or overflow. */
int64_t qmoe_worklist_capacity(int64_t T, int32_t top_k, int32_t E, int32_t m_tile,
                               int32_t n_tile, int32_t N);

/*
 * Expert grouping and tile work-list [qmoe.rs, launch_grouping (counts,
 * offsets, grouped routes); gemm_quant_moe.rs, moe_build_tile_worklist].
 *   topk_ids        int32 [T*top_k] expert of each route; entries outside
 *                   [0, E) join no group.
 *   expert_offsets  int32 [E+1] out: exclusive prefix sum of per-expert
 *                   route counts (offsets[E] = number of grouped routes).
 *   sorted_routes   int32 [T*top_k] out: route ids grouped by expert, experts
 *                   ascending, route ids ascending within an expert (stable).
 *                   Entries at and past offsets[E] are left untouched.
 *   worklist        int32 [worklist_capacity, 3] out: one item
 *                   {expert, m_tile_index, n_tile_index} for every m_tile rows
 *                   of an expert with routes times every n_tile columns of N;
 *                   experts ascending, then m, then n.
 *   n_items         int32 [1] out: number of items.
 * Requires 1 <= E <= 1024, m_tile >= 1, n_tile >= 1, N >= 1, T*top_k < 2^31,
 * worklist_capacity >= qmoe_worklist_capacity(...).  One workgroup does all
 * of it; no atomics, so the output is deterministic.
 */
int qmoe_group(const int32_t* topk_ids, int64_t T, int32_t top_k, int32_t E, int32_t m_tile,
               int32_t n_tile, int32_t N, int32_t* expert_offsets, int32_t* sorted_routes,
               int32_t* worklist, int64_t worklist_capacity, int32_t* n_items, void* stream);

/* Workspace bytes qmoe_forward needs for these sizes (0 on invalid sizes)
 * [qmoe.rs, QMoEKernel::execute sizes its scratch pool (route ids and
 * weights, fc1 and activation rows, route outputs, grouping arrays) from the
 * shapes alone; moe.rs, the MoE workspace estimator].  The layout depends on
 * neither the weight widths nor block_size, so unlike those estimators this
 * takes no bits or block_size argument.  It never decreases as T grows (the
 * other sizes fixed), so a workspace sized for the largest batch serves every
 * smaller one. */
size_t qmoe_workspace_size(int64_t T, int32_t H, int32_t I, int32_t E, int32_t top_k,
                           int32_t dtype);

/*
 * The whole layer [qmoe.rs, QMoEKernel::execute; PR 32198; PR 33569].
 *   hidden      dtype [T, H]           input states, 16-byte aligned
 *   logits      float32 [T, E]         router logits
 *   fc1         N = 2*I rows (row 2j gate, 2j+1 up), K = H
 *   fc2         N = H rows, K = I
 *   zero_point_offset   fractional zero point, NaN = none; finite otherwise.
 *               Used for a projection whose zero_points is NULL.
 *   block_size  power of two >= 16 dividing H and I
 *   top_k, normalize    as in qmoe_route
 *   activation  QMOE_ACT_SWIGLU or QMOE_ACT_GEGLU
 *   dtype       QMOE_DTYPE_F16 or QMOE_DTYPE_BF16
 *   out         dtype [T, H] out: sum over slots s (in slot order) of
 *               w[t,s] * fc2_e(act(fc1_e(x_t))), rounded once to dtype
 *   topk_ids_out, topk_w_out  NULL, or int32/float32 [T, top_k] copies of the
 *               routing decision
 *   workspace   >= qmoe_workspace_size(T, H, I, E, top_k, dtype) bytes,
 *               256-byte aligned; contents on entry do not matter.
 * Requires 1 <= E <= 1024, 1 <= top_k <= E, H and I multiples of 128,
 * bits in {1,2,3,4,8} per projection, T*H < 2^32 and T*top_k*I < 2^32 (the
 * projection kernels address their inputs with 32-bit element offsets).
 * T = 0 returns QMOE_OK and enqueues nothing.
 * Launches: prefill (T*top_k > QMOE_DECODE_MAX_ROUTES) route, group, fc1,
 * fc2, combine; streamed decode (see qmoe_timer_start) fc1 with routing and
 * grouping, then fc2 with the combine (its last workgroup per column block
 * sums the slots, in slot order); other decode layers a routing + m-tile plan,
 * fc1, fc2 and the combine.
 * Numerics: products accumulate in float32, the activation is rounded to
 * dtype, fc2 outputs stay float32 until the combine.  The prefill kernels
 * (T*top_k > QMOE_DECODE_MAX_ROUTES) and the decode kernels for block sizes
 * below 128 round each dequantized weight (code - zp) * scale once to dtype
 * (round to nearest even) before the products [PR 33569: dequantized weights
 * rounded to the activation type before accumulation].  The decode kernels
 * for block sizes that are multiples of 128 feed the MFMA the exact codes
 * (biased into dtype values, see qmoe_raw_codes) and apply zero point and
 * scale to the float32 partial sums of each 128-input step, so W is never
 * rounded there.  For many routes, fc2 may split its K range into 2 or 4
 * parts (chosen from the sizes alone); their float32 partial sums are added
 * in part order before the routing weights apply, so results stay
 * deterministic.
 */
int qmoe_forward(const void* hidden, const float* logits, int64_t T, int32_t H, int32_t I,
                 int32_t E, const qmoe_proj* fc1, const qmoe_proj* fc2, float zero_point_offset,
                 int32_t block_size, int32_t top_k, int32_t normalize, int32_t activation,
                 int32_t dtype, void* out, int32_t* topk_ids_out, float* topk_w_out,
                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * The layer with a shared expert [moe.rs: routed experts plus a shared
 * expert whose output is added to the routed output times the sigmoid of a
 * per-token gate logit (shared gate GEMM, gated add)].
 *   fc1, fc2, logits, ... as qmoe_forward (the routed experts)
 *   I_shared     the shared expert's intermediate size (a multiple of 128
 *                and of block_size)
 *   shared_fc1   one expert: N = 2*I_shared interleaved gate/up rows, K = H
 *   shared_fc2   one expert: N = H rows, K = I_shared
 *                (same widths rules, block_size and zero_point_offset as the
 *                routed projections)
 *   shared_gate  dtype [H] (16-byte aligned): the shared gate's weights
 *   out          dtype [T, H] out: RNE(routed + s_t * shared_t) with
 *                s_t = sigmoid(sum_h x[t,h] shared_gate[h]) in float32, the
 *                routed and shared outputs each rounded to dtype first (as the
 *                page's weighted sum and shared output are)
 *   workspace    >= qmoe_shared_workspace_size(...) bytes, 256-byte aligned
 * Runs qmoe_forward for the routed experts, a token-gate kernel, the shared
 * expert as a one-expert qmoe_forward, and a gated add.
 */
size_t qmoe_shared_workspace_size(int64_t T, int32_t H, int32_t I, int32_t E, int32_t top_k,
                                  int32_t I_shared, int32_t dtype);
int qmoe_forward_shared(const void* hidden, const float* logits, int64_t T, int32_t H, int32_t I,
                        int32_t E, const qmoe_proj* fc1, const qmoe_proj* fc2, int32_t I_shared,
                        const qmoe_proj* shared_fc1, const qmoe_proj* shared_fc2,
                        const void* shared_gate, float zero_point_offset, int32_t block_size,
                        int32_t top_k, int32_t normalize, int32_t activation, int32_t dtype,
                        void* out, int32_t* topk_ids_out, float* topk_w_out, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * qmoe_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).  The
 * same arguments and kernels as qmoe_forward without workspace and
 * workspace_bytes: the workspace is a fixed array of
 * QMOE_NOALLOC_SCRATCH_BYTES inside the library, one copy per GPU, held until
 * the process ends.  The call allocates and frees nothing.
 * Sizes whose qmoe_workspace_size exceeds QMOE_NOALLOC_SCRATCH_BYTES return
 * QMOE_ERR_WORKSPACE before any launch (64 MiB holds, e.g., 512 tokens of a
 * hidden = inter = 2048 top-2 layer; use qmoe_forward for larger layers).
 * Every call on one GPU uses that GPU's array: calls that overlap in time on
 * one GPU (other streams, other threads) race.  Nothing in the array needs to
 * start at zero; it keeps the last call's contents.
 */
#define QMOE_NOALLOC_SCRATCH_BYTES (64u << 20)
int qmoe_forward_noalloc(const void* hidden, const float* logits, int64_t T, int32_t H, int32_t I,
                         int32_t E, const qmoe_proj* fc1, const qmoe_proj* fc2,
                         float zero_point_offset, int32_t block_size, int32_t top_k,
                         int32_t normalize, int32_t activation, int32_t dtype, void* out,
                         int32_t* topk_ids_out, float* topk_w_out, void* stream);

/*
 * Operator options beyond the base layer [qmoe.rs, the QMoE operator's
 * optional inputs and attributes].  Zero-initialising the struct is NOT the
 * default: use QMOE_LAYER_OPTS_DEFAULT, or pass NULL to qmoe_forward_ex.
 *   fc1_bias       NULL or float32 [E, rows of fc1] (2*I, or I with a separate
 *                  fc3), added to fc1's float32 outputs before the activation
 *   fc2_bias       NULL or float32 [E, H], added to fc2's outputs
 *   fc3            NULL, or (swiglu_fusion = 0) the up projection [E, I, H]:
 *                  fc1 then holds the I gate rows; fc3 must have fc1's width
 *                  and zero-point mode (else QMOE_ERR_UNSUPPORTED)
 *   fc3_bias       NULL or float32 [E, I] (only with fc3)
 *   router_weights NULL or float32 [T, E]: the logits only select the
 *                  experts; a selected expert's weight is its router_weights
 *                  value, divided by the slot-order sum of the selected values
 *                  when normalize is set (0 when that sum is 0)
 *   swiglu_fusion  QMOE_SWIGLU_INTERLEAVED (fc1 rows 2j gate, 2j+1 up),
 *                  QMOE_SWIGLU_HALVES (gate j, up I + j) or
 *                  QMOE_SWIGLU_SEPARATE (gate in fc1, up in fc3); the last two
 *                  only with QMOE_ACT_SWIGLU [qmoe.rs, swiglu_fusion 1 / 2 / 0]
 *   activation_alpha, activation_beta, swiglu_limit   SwiGLU as
 *                  g' sigmoid(alpha g') (u' + beta), g' = fminf(g, limit),
 *                  u' = u clamped to [-limit, limit] (NaN stays NaN)
 *                  [qmoe.rs, swiglu_value]; GeGLU ignores them
 * Layers with biases, a non-interleaved layout, router_weights or 1/8-bit
 * codes run on the generic kernels (prefill tiles; decode plan + m-tile
 * kernels).
 */
#define QMOE_SWIGLU_SEPARATE 0
#define QMOE_SWIGLU_INTERLEAVED 1
#define QMOE_SWIGLU_HALVES 2
typedef struct qmoe_layer_opts {
    const float* fc1_bias;
    const float* fc2_bias;
    const qmoe_proj* fc3;
    const float* fc3_bias;
    const float* router_weights;
    int32_t swiglu_fusion;
    float activation_alpha;
    float activation_beta;
    float swiglu_limit;
} qmoe_layer_opts;
#define QMOE_LAYER_OPTS_DEFAULT \
    {NULL, NULL, NULL, NULL, NULL, QMOE_SWIGLU_INTERLEAVED, 1.0f, 0.0f, __builtin_inff()}

/* qmoe_forward with operator options (opts NULL = qmoe_forward). */
int qmoe_forward_ex(const void* hidden, const float* logits, int64_t T, int32_t H, int32_t I,
                    int32_t E, const qmoe_proj* fc1, const qmoe_proj* fc2, float zero_point_offset,
                    int32_t block_size, int32_t top_k, int32_t normalize, int32_t activation,
                    int32_t dtype, void* out, int32_t* topk_ids_out, float* topk_w_out,
                    const qmoe_layer_opts* opts, void* workspace, size_t workspace_bytes,
                    void* stream);

/*
 * Test hook: the dequantization of the weight-rounding kernels, written out
 * in full [qmoe.rs, decode_affine_weight: (code - zp) * scale with the code
 * read LSB-first and the zero point from the tensor or the centre; PR 32198,
 * zero_point_offset as the zero point of every block].
 *   p           one projection as above (E experts, N rows, K inputs, K a
 *               multiple of 32 and of block_size)
 *   codes_out   NULL or int32 [E, N, K] out: unpacked codes
 *   w_out       dtype [E, N, K] out: round-to-nearest-even of (code - zp) * scale
 * The prefill kernels and the decode kernels for block sizes below 128 call
 * the same device unpack and dequant routines (the raw-code decode path is
 * covered by qmoe_raw_codes).  Errors: QMOE_ERR_INVALID_ARG for bad sizes,
 * pointers or dtype; QMOE_ERR_UNSUPPORTED for K not a multiple of 32.
 */
int qmoe_dequantize(const qmoe_proj* p, int32_t E, int32_t N, int32_t K, int32_t block_size,
                    float zero_point_offset, int32_t dtype, int32_t* codes_out, void* w_out,
                    void* stream);

/*
 * Test hook: the codes as the decode kernels' raw-code MFMA operands carry
 * them [qmoe.rs, decode_affine_weight, LSB-first code order; PR 33569, 24-bit
 * 8-code INT3 groups].  For block sizes that are multiples of 128 the decode
 * kernels place each code in the mantissa of a dtype value base + code
 * (exact) and take base and zero point out of the float32 sums.  This runs the
 * same device routines on every 32-code span and writes base + code - base,
 * i.e. the code each MFMA input carries, at its input position.
 *   p           one projection (only codes and bits are read)
 *   variant     QMOE_RAW_SINGLE_BASE: one base per dtype (fp16 1024, bf16
 *               128), the m-tile and expert-stationary decode kernels, 2/3/4
 *               bits; QMOE_RAW_MULTI_BASE: a power-of-two base per register,
 *               the streamed decode kernels, 2/4 bits
 *   codes_out   int32 [E, N, K] out
 * Requires K a multiple of 32.  Errors as qmoe_dequantize; 3-bit codes with
 * QMOE_RAW_MULTI_BASE, and 1- and 8-bit codes (no kernel feeds them raw),
 * return QMOE_ERR_UNSUPPORTED.
 */
#define QMOE_RAW_SINGLE_BASE 0
#define QMOE_RAW_MULTI_BASE 1
int qmoe_raw_codes(const qmoe_proj* p, int32_t E, int32_t N, int32_t K, int32_t dtype,
                   int32_t variant, int32_t* codes_out, void* stream);

/*
 * Kernel timer for measurement.  After qmoe_timer_start(stage), every
 * qmoe_forward call attaches a HIP event pair to the dispatch of that
 * stage's kernel (hipExtLaunchKernelGGL start/stop events, at most 4096
 * pairs).  qmoe_timer_stop() waits for the recorded events, stores the summed
 * elapsed milliseconds and the number of launches timed, and disables the
 * timer.  Stages: 0 route (on the decode path: routing, grouping and the
 * m-tile list in one kernel), 1 group (prefill path only), 2 fc1
 * (+ activation), 3 fc2, 4 combine (no launch on the streamed decode path,
 * T <= 16 and T*top_k <= 64 with E <= T*top_k or E <= 32 and widths and
 * blocks the streamed kernels take, whose fc2 launch performs the combine).
 */
#define QMOE_STAGE_ROUTE 0
#define QMOE_STAGE_GROUP 1
#define QMOE_STAGE_FC1 2
#define QMOE_STAGE_FC2 3
#define QMOE_STAGE_COMBINE 4
int qmoe_timer_start(int32_t stage);
int qmoe_timer_stop(double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* QMOE_H */
