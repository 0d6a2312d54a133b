/*
 * decodehp.h -- C ABI of libdecodehp, the MI355X (gfx950) decode hot path:
 * INT4-affine dequantizing GEMV / GEMM, routed-MoE decode, hyper-connection read/inject.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every pointer argument that names tensor data is a DEVICE pointer (HIP device
 *    memory, or memory the device can address) owned by the caller. The library never
 *    allocates, frees or retains caller memory; it holds no pointer past the return.
 *  - Every call is asynchronous on `stream` (a hipStream_t passed as void*, NULL for the
 *    default stream). The library never synchronizes. Results are valid once the caller
 *    has synchronized with `stream`.
 *  - Arguments are validated on the host before any HIP call. A nonzero return means
 *    nothing was launched, except DHP_ERR_LAUNCH, which reports that the HIP runtime
 *    rejected a launch; decodehp_last_error() then holds a message for this thread.
 *  - Calls that overlap on one device share nothing but their arguments: two calls are
 *    independent unless the caller passes them the same output or workspace buffer.
 *  - Deterministic: no floating-point atomics; the same inputs give the same bits.
 *
 * INT4-affine weights (struct dhp_int4)
 * -------------------------------------
 * "src/real_forward.rs" (turbospark-runtime 0.3.0), module doc, memory model: every
 * projection binds the weights, scales and biases of an INT4-affine tensor in place, with
 * nothing staged per dispatch. Element (n, k) of a [rows x cols] tensor is
 *     W[n, k] = q[n, k] * scale[n, k / 64] + bias[n, k / 64],    q in 0..15,
 * with one bf16 scale and one bf16 bias per group of 64 consecutive k.
 *   codes : uint8 [rows][cols/2], row-major; byte j of a row holds k = 2j in bits 0..3
 *           and k = 2j+1 in bits 4..7. 16-byte aligned.
 *   scales: bf16 (uint16 bit patterns) [rows][cols/64], row-major. 2-byte aligned.
 *   biases: bf16 [rows][cols/64], row-major. 2-byte aligned.
 *   cols % 64 == 0, group == 64.
 */
#ifndef DECODEHP_H
#define DECODEHP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define DHP_OK 0
#define DHP_ERR_INVALID (-1)     /* null pointer, non-positive or inconsistent size */
#define DHP_ERR_UNSUPPORTED (-2) /* a shape or option outside what the kernels cover */
#define DHP_ERR_MISALIGNED (-3)  /* a pointer below its required alignment */
#define DHP_ERR_WORKSPACE (-4)   /* workspace missing or smaller than decodehp_workspace_bytes */
#define DHP_ERR_NO_DEVICE (-5)   /* no HIP device, or the current device is not gfx950 */
#define DHP_ERR_LAUNCH (-6)      /* the HIP runtime rejected a launch */

/* Element types. */
#define DHP_F16 0
#define DHP_F32 1
#define DHP_BF16 2
#define DHP_I8 3     /* signed 8-bit codes (the INT8 router) */

/* Workspace queries (decodehp_workspace_bytes `op`). */
#define DHP_OP_GEMV_ARGMAX 1 /* a = rows (N), b = m                       */
#define DHP_OP_MOE_DECODE 2  /* a = n_experts, b = top_k, c = inter (rows of gate) */
#define DHP_OP_HC_READ 3     /* a = C, b = R (low rank)                  */

/* moe_decode flags. */
#define DHP_MOE_FP16_BOUNDARY 1 /* round routed sum and gated shared output to fp16 before the add */

/* Limits. */
#define DHP_GEMV_MAX_M 16
#define DHP_GEMM_MAX_M 128
#define DHP_MOE_MAX_TOP_K 10
#define DHP_MOE_PREFILL_MAX_M 128
#define DHP_HC_MAX_C 16

typedef struct dhp_int4 {
    const void* codes;  /* uint8 [rows][cols/2], 16-byte aligned */
    const void* scales; /* bf16  [rows][cols/64] */
    const void* biases; /* bf16  [rows][cols/64] */
    int32_t rows;
    int32_t cols;
    int32_t group; /* must be 64 */
} dhp_int4;

/* A stack of same-shaped INT4 tensors (one per expert): expert e's codes start at
 * first.codes + e * codes_stride bytes, its scales and biases at first.scales /
 * first.biases + e * scales_stride bytes. The analog of the pages' per-layer expert
 * offset table ("src/real_forward.rs", fields around the routed blob layout). */
typedef struct dhp_int4_experts {
    dhp_int4 first;
    int64_t codes_stride;  /* bytes, multiple of 16 */
    int64_t scales_stride; /* bytes, multiple of 2 */
    int32_t count;
} dhp_int4_experts;

/*
 * decodehp_dequant_gemv -- Y[r, n] = sum_k W[n, k] * X[r, k] for r < m (m <= 16).
 * "src/real_forward.rs": module doc (dequant_int4_gemv_simd against resident INT4-affine
 * weights) and field batched_gemv_prefill (the batched GEMV and the per-row GEMV agree bit for
 * bit). The LM head of "src/families/qwen4/mod.rs" (decoder-layer pseudocode, exit) is this
 * call over the vocabulary, with argmax.
 * Every row r of an m-row call gives exactly the bits (y and argmax) of an m = 1 call on row r
 * alone, for any weights and biases: both run each output as s * (q . x) + b * sum(x) per
 * 64-weight group, with q . x an exact integer sum (the group's activations taken to 21 bits
 * of its largest magnitude; every activation within 2^10 of it exactly) and the groups joined
 * in fp32 in one fixed operation order (see decodehp_dequant_gemv_mc for the fp16
 * matrix-core arm, which does not). The activations must be finite.
 *   w       : weight [N x K].
 *   x       : fp16 [m][K], row-major, 16-byte aligned.
 *   y       : [m][N] row-major, fp16 (y_dtype DHP_F16) or fp32 (DHP_F32); fp32 accumulate.
 *   argmax  : nullable int32 [m]; when set, argmax[r] = lowest n with the largest fp32 value
 *             of row r (computed before any fp16 rounding of y).
 *   ws      : workspace of decodehp_workspace_bytes(DHP_OP_GEMV_ARGMAX, N, m, 0) bytes when
 *             argmax is set (may be NULL otherwise), 16-byte aligned. Scratch only: contents
 *             are undefined after the call; calls sharing one buffer must not overlap.
 * Errors: -1 null/size, -2 K % 64, K > 16384, group != 64, m outside 1..16, y_dtype, -3 alignment,
 *         -4 workspace, -5 device, -6 launch.
 */
int decodehp_dequant_gemv(const dhp_int4* w, const void* x, int32_t m, void* y, int32_t y_dtype,
                          int32_t* argmax, void* ws, size_t ws_bytes, void* stream);

/*
 * decodehp_dequant_gemv_mc -- decodehp_dequant_gemv on the fp16 matrix cores (the pages' separate
 * matrix-instruction variant, "src/real_forward.rs", field batched_gemv_prefill). It is NOT
 * bit-equal to the m = 1 call, and at the LM head's size over 8 rows it is no faster than
 * decodehp_dequant_gemv (about 52 against 49 us per call from HBM). Each weight is
 * dequantized once into an fp16 operand, q*s+b rounded to fp16 (exact when the bias is
 * -8*scale and the scale is a bf16 value in fp16's normal range; otherwise off by up to half
 * an fp16 ulp per weight, which can put outputs near zero past the 1e-3 + 1e-2|y| bar), and
 * the products are summed in the matrix cores' order. Arguments, workspace and errors: as
 * decodehp_dequant_gemv.
 */
int decodehp_dequant_gemv_mc(const dhp_int4* w, const void* x, int32_t m, void* y, int32_t y_dtype,
                             int32_t* argmax, void* ws, size_t ws_bytes, void* stream);

/*
 * decodehp_dequant_gemm_batched -- Y = X W^T for a chunked-prefill block of m <= 128 rows.
 * "src/real_forward.rs", field batched_gemv_prefill: resident GEMVs run as one M-row GEMM;
 * the same field and prefill_steel give the 64-row micro-batched form this replaces.
 * Matrix cores (fp16 operands, fp32 accumulate): each weight is dequantized once into an
 * fp16 operand, q*s+b rounded to fp16 (exact when the bias is -8*scale and the scale is
 * a bf16 value in fp16's normal range; for other biases each weight can be off by half an
 * fp16 ulp, which can put outputs near zero past the 1e-3 + 1e-2|y| bar).
 *   w : weight [N x K], N % 16 == 0.   x : fp16 [m][K], 16-byte aligned.   y : fp16 [m][N].
 * Errors: -1, -2 (K % 64, N % 16, m outside 1..128, K > 32768), -3, -5, -6.
 */
int decodehp_dequant_gemm_batched(const dhp_int4* w, const void* x, int32_t m, void* y,
                                  void* stream);

/*
 * decodehp_moe_decode -- one token through a routed MoE layer with a gated shared expert.
 * "src/families/qwen4/mod.rs", section MoE: top-k on the raw router logits, softmax over
 * the selected set only. "src/families/qwen/state.rs", struct RealQwenState: fp32 router
 * logits, unit router and per-expert scales, the shared expert gated by a scalar logit
 * through a sigmoid. "src/real_forward.rs", module doc: phase 1 = gate/up GEMV and the
 * gated-FFN activation silu(gate)*up, phase 2 = down GEMV and the weighted k-way reduce.
 *     logits = router @ x (fp32); ids = the top_k largest, largest first, lowest expert
 *     index first among equal fp32 logits; weights = softmax over those logits;
 *     out = fp16( sum_j weights[j] * down_ids[j](act_ids[j]) + sigmoid(g) * down_s(act_s) ),
 *     act_e = silu(gate_e x) * (up_e x) kept in fp32, g = shared_gate_row . x.
 * With DHP_MOE_FP16_BOUNDARY the routed sum and the gated shared output are each rounded
 * to fp16 before the add ("src/families/qwen4/mod.rs", section MoE, the fp16 boundary).
 *   x               : fp16 [hidden], 16-byte aligned.
 *   router          : [n_experts][hidden], bf16 (router_dtype DHP_BF16), fp32 (DHP_F32) or
 *                     signed int8 codes (DHP_I8, taken at unit scale here), rows 16-byte
 *                     aligned (int8 rows 8-byte).
 *   shared_gate_row : bf16 [hidden], 16-byte aligned.
 *   gate, up        : experts [inter x hidden];  down : experts [hidden x inter]; same count.
 *   shared_*        : one expert of the same shapes.
 *   top_k           : 1..DHP_MOE_MAX_TOP_K (10), <= n_experts.
 *   out             : fp16 [hidden].  ids : int32 [top_k].  weights : fp32 [top_k].
 *   ws              : decodehp_workspace_bytes(DHP_OP_MOE_DECODE, n_experts, top_k, inter).
 * Errors: -1, -2 (hidden % 512, hidden > 4096, inter % 64, inter > 1024, top_k,
 *         n_experts > 1024, router_dtype, flags), -3, -4, -5, -6.
 */
int decodehp_moe_decode(const void* x, const void* router, int32_t router_dtype,
                        const void* shared_gate_row, const dhp_int4_experts* gate,
                        const dhp_int4_experts* up, const dhp_int4_experts* down,
                        const dhp_int4* shared_gate, const dhp_int4* shared_up,
                        const dhp_int4* shared_down, int32_t top_k, int32_t flags, void* out,
                        int32_t* ids, float* weights, void* ws, size_t ws_bytes, void* stream);

/*
 * decodehp_moe_decode_noalloc -- decodehp_moe_decode without a workspace argument, for callers
 * that cannot allocate device memory (code recorded under graph capture, tight serving loops,
 * harnesses that forbid allocation). The call allocates nothing: its scratch (router logits,
 * gate logit, fp32 activations) lives in a fixed array inside the library, one per GPU,
 * DHP_NOALLOC_SCRATCH_BYTES (48 KiB) long and held until the process ends.
 *   Arguments, results and the kernels run: as decodehp_moe_decode, minus ws and ws_bytes.
 *   Limit: decodehp_workspace_bytes(DHP_OP_MOE_DECODE, n_experts, top_k, inter), about
 *   4 * (n_experts + (top_k + 1) * inter) + 9216 bytes, must not exceed DHP_NOALLOC_SCRATCH_BYTES: every
 *   top_k <= 10 fits up to n_experts 1024 with inter 640 (the 256-expert top-8 layer with inter
 *   512 takes 28,928 bytes); larger layers get -4 and must use decodehp_moe_decode.
 *   Concurrency: every call on one GPU uses the same array, so calls that overlap in time on
 *   one GPU (different streams, or different threads' streams) race; calls on one stream are
 *   ordered and safe. Nothing in the array has to start at zero: each call writes what it reads.
 * Errors: as decodehp_moe_decode (-4: the layer needs more than the fixed scratch; -6 also when
 *         the scratch's device address cannot be obtained).
 */
#define DHP_NOALLOC_SCRATCH_BYTES 49152
int decodehp_moe_decode_noalloc(const void* x, const void* router, int32_t router_dtype,
                                const void* shared_gate_row, const dhp_int4_experts* gate,
                                const dhp_int4_experts* up, const dhp_int4_experts* down,
                                const dhp_int4* shared_gate, const dhp_int4* shared_up,
                                const dhp_int4* shared_down, int32_t top_k, int32_t flags, void* out,
                                int32_t* ids, float* weights, void* stream);

/*
 * decodehp_moe_prefill -- a chunk of m tokens through the same MoE layer in one pass.
 * "src/real_forward.rs", the forward state's switch that runs a chunked-prefill layer's
 * routed half as one batched dispatch over a route list, byte-identical to running the
 * tokens one at a time. Row i of out, ids and weights is bit-identical to what
 * decodehp_moe_decode returns for row i of x (same weights, top_k and flags); each expert's
 * weights are streamed once per call for all the tokens routed to it.
 *   x               : fp16 [m][hidden], 16-byte aligned.   m : 1..DHP_MOE_PREFILL_MAX_M.
 *   router, shared_gate_row, gate, up, down, shared_*, top_k, flags : as decodehp_moe_decode.
 *   out             : fp16 [m][hidden].  ids : int32 [m][top_k].  weights : fp32 [m][top_k].
 *   ws              : decodehp_moe_prefill_workspace_bytes(m, n_experts, top_k, inter, hidden)
 *                     bytes, 16-byte aligned.
 * Errors: as decodehp_moe_decode, and -2 for m outside 1..DHP_MOE_PREFILL_MAX_M.
 */
int decodehp_moe_prefill(const void* x, int32_t m, const void* router, int32_t router_dtype,
                         const void* shared_gate_row, const dhp_int4_experts* gate,
                         const dhp_int4_experts* up, const dhp_int4_experts* down,
                         const dhp_int4* shared_gate, const dhp_int4* shared_up,
                         const dhp_int4* shared_down, int32_t top_k, int32_t flags, void* out,
                         int32_t* ids, float* weights, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes decodehp_moe_prefill needs (0 for arguments out of range). */
size_t decodehp_moe_prefill_workspace_bytes(int32_t m, int32_t n_experts, int32_t top_k,
                                            int32_t inter, int32_t hidden);

/*
 * The router variants ("src/families/qwen/state.rs", struct RealQwenState, fields router_ones and
 * per_expert_ones): an INT8 router whose kernel multiplies x[n] by an effective scale per
 * element, and a per-expert scale on each selected expert's routing weight. Both are ones for
 * this family (the plain entry points above); the _ex entry points take them:
 *     logits[e]  = sum_n R[e][n] * (elem_scale[n] * x[n])        (elem_scale NULL: ones)
 *     weights[j] = softmax over the selected logits, then * expert_scale[ids[j]]   (NULL: ones)
 * R is bf16, fp32 or signed int8 codes (DHP_I8; the scale of an INT8 router lives in elem_scale).
 * With both NULL and a bf16/fp32 router the results equal the plain entry points' bit for bit.
 */
typedef struct dhp_router {
    const void* weights;         /* [n_experts][hidden], rows 16-byte aligned (int8 rows 8-byte) */
    int32_t dtype;               /* DHP_BF16, DHP_F32 or DHP_I8 */
    const void* elem_scale;      /* bf16 [hidden], 16-byte aligned, or NULL */
    const float* expert_scale;   /* fp32 [n_experts], or NULL */
} dhp_router;

int decodehp_moe_decode_ex(const void* x, const dhp_router* router, const void* shared_gate_row,
                           const dhp_int4_experts* gate, const dhp_int4_experts* up,
                           const dhp_int4_experts* down, const dhp_int4* shared_gate,
                           const dhp_int4* shared_up, const dhp_int4* shared_down, int32_t top_k,
                           int32_t flags, void* out, int32_t* ids, float* weights, void* ws,
                           size_t ws_bytes, void* stream);
int decodehp_moe_prefill_ex(const void* x, int32_t m, const dhp_router* router, const void* shared_gate_row,
                            const dhp_int4_experts* gate, const dhp_int4_experts* up,
                            const dhp_int4_experts* down, const dhp_int4* shared_gate,
                            const dhp_int4* shared_up, const dhp_int4* shared_down, int32_t top_k,
                            int32_t flags, void* out, int32_t* ids, float* weights, void* ws,
                            size_t ws_bytes, void* stream);

/*
 * decodehp_hc_read -- one hyper-connection read (attn_hc / mlp_hc / the final mixer).
 * "src/families/qwen4/mod.rs", section Hyper-connections, and "src/families/qwen4/hc.rs",
 * encode_hyper_connection. Element (c, h) of the C streams of width H sits at c*H + h. With
 * rho[c] the RMS of stream c (eps inside the root), n[c,h] = raw[c,h] / rho[c] * hc_norm[c,h]
 * (the stored weight multiplies as is), lo[r] = silu(sum_j down[r][j] n[j] / C),
 * mixed[h] = (1/C) sum_c sigmoid(sum_r up[c*H+h][r] lo[r]) * n[c,h] (fp16 [H]) and
 * inject_w[c] = 2 sigmoid(sum_j inject[c][j] n[j] / C) (fp32 [C]).
 * `raw` is read and never written (hc.rs doc); the caller injects separately.
 *   raw     : fp16 [C*H], 16-byte aligned.   hc_norm : bf16 [C*H], 16-byte aligned.
 *   down    : [R x C*H].   up : [C*H x R].   inject : [C x C*H] or NULL (final mixer).
 *   mixed   : fp16 [H].    inject_w : fp32 [C], NULL exactly when inject is NULL.
 *   ws      : decodehp_workspace_bytes(DHP_OP_HC_READ, C, R, 0) bytes.
 * Errors: -1, -2 (C not a power of two in 1..16, H % 64, C*H not a multiple of 2048 or
 *         above 32768, R % 64, R > 1024),
 *         -3, -4, -5, -6.
 */
int decodehp_hc_read(const void* raw, const void* hc_norm, int32_t C, int32_t H, float eps,
                     const dhp_int4* down, const dhp_int4* up, const dhp_int4* inject,
                     void* mixed, float* inject_w, void* ws, size_t ws_bytes, void* stream);

/*
 * decodehp_hc_inject -- wide[c*H + h] = fp16(wide[c*H + h] + out[h] * inject_w[c]), in place.
 * "src/families/qwen4/mod.rs", the decoder-layer pseudocode and THE INJECTION TRAP: the
 * sublayer output is added, scaled per stream, to the UN-normalized residual `raw`.
 *   wide : fp16 [C*H] (raw in, hidden out), 16-byte aligned.   out : fp16 [H], 16-byte aligned.
 *   inject_w : fp32 [C].
 * Errors: -1, -2 (C outside 1..16, H % 8), -3, -5, -6.
 */
int decodehp_hc_inject(void* wide, const void* out, const float* inject_w, int32_t C, int32_t H,
                       void* stream);

/*
 * decodehp_hc_inject_read -- a sublayer's inject followed by the next hyper-connection read, in
 * one call: the step pair the decoder-layer pseudocode runs between two sublayers
 * ("src/families/qwen4/mod.rs", decoder-layer pseudocode; "src/families/qwen4/hc.rs",
 * encode_hyper_connection). First
 *     hidden[c*H + h] = fp16(prev[c*H + h] + out[h] * inject_w[c])
 * (the same bits decodehp_hc_inject stores), then decodehp_hc_read of hidden. The inject's add
 * is formed inside the read's first kernel, which also stores hidden, so the call saves the
 * separate inject's launch.
 *   prev     : fp16 [C*H], the residual before the inject, 16-byte aligned (not written).
 *   out      : fp16 [H], the sublayer output, 16-byte aligned.   inject_w : fp32 [C] (its gates).
 *   hidden   : fp16 [C*H], 16-byte aligned, the residual after the inject. Must not overlap prev
 *              or out (the read's blocks are still reading them while one block stores hidden).
 *   hc_norm, C, H, eps, down, up, inject, mixed, ws : as decodehp_hc_read (of hidden).
 *   inject_w_next : fp32 [C], the new read's inject weights; must not overlap inject_w.
 * Errors: those of decodehp_hc_read and decodehp_hc_inject; -1 when hidden overlaps prev or
 *         out, or inject_w_next overlaps inject_w.
 */
int decodehp_hc_inject_read(const void* prev, const void* out, const float* inject_w, void* hidden,
                            const void* hc_norm, int32_t C, int32_t H, float eps, const dhp_int4* down,
                            const dhp_int4* up, const dhp_int4* inject, void* mixed, float* inject_w_next,
                            void* ws, size_t ws_bytes, void* stream);

/*
 * decodehp_hc_read_batched / decodehp_hc_inject_batched -- the read and the inject for the m
 * tokens of a chunked-prefill micro-batch ("src/families/qwen4/hc.rs", encode_hyper_connection:
 * inside a micro-batch every token's inject gate has a row of its own). Row t of each output is
 * the per-token call's on row t of the inputs, within the tolerance (the low-rank projections
 * run as matrix-core GEMMs over the m rows, with normed and lo rounded to fp16 as their
 * operands).
 *   raw, wide : fp16 [m][C*H], 16-byte aligned.   mixed, out : fp16 [m][H], 16-byte aligned.
 *   inject_w  : fp32 [m][C] (NULL exactly when inject is NULL).   m : 1..DHP_GEMM_MAX_M.
 *   C, H, eps, hc_norm, down, up, inject : as decodehp_hc_read.
 *   ws        : decodehp_hc_read_batched_workspace_bytes(m, C, H, R) bytes, 16-byte aligned.
 * Errors: as decodehp_hc_read / decodehp_hc_inject, and -2 for m outside 1..128.
 */
size_t decodehp_hc_read_batched_workspace_bytes(int32_t m, int32_t C, int32_t H, int32_t R);
int decodehp_hc_read_batched(const void* raw, int32_t m, const void* hc_norm, int32_t C, int32_t H, float eps,
                             const dhp_int4* down, const dhp_int4* up, const dhp_int4* inject, void* mixed,
                             float* inject_w, void* ws, size_t ws_bytes, void* stream);
int decodehp_hc_inject_batched(void* wide, int32_t m, const void* out, const float* inject_w, int32_t C,
                               int32_t H, void* stream);

/*
 * Whole decoder layers for one token, and their capture as one HIP graph.
 * "src/families/qwen4/mod.rs", module doc, "The decoder layer, as pseudocode": the token's
 * hidden vector is replicated over the C streams at entry; each layer runs
 *     attn_hc read -> sublayer -> inject -> mlp_hc read -> moe -> inject
 * with the inject adding the sublayer output, scaled per stream, to the un-normalized residual;
 * at exit the hyper_connection_mixer (a read with no inject projection) gives the H-wide output.
 * The attention sublayer is not part of this library: `sublayer` is an INT4 [H x H] linear map
 * standing in for it (out = sublayer . mixed). The graph form is the counterpart of the pages'
 * one command buffer per token: the whole sequence replays with one launch.
 */
typedef struct dhp_hc_block {
    const void* hc_norm;     /* bf16 [C*H], 16-byte aligned */
    const dhp_int4* down;    /* [R x C*H] */
    const dhp_int4* up;      /* [C*H x R] */
    const dhp_int4* inject;  /* [C x C*H]; NULL exactly for the final mixer */
} dhp_hc_block;

typedef struct dhp_decode_layer {
    dhp_hc_block attn_hc;
    const dhp_int4* sublayer;               /* [H x H], the attention stand-in */
    dhp_hc_block mlp_hc;
    const void* router;                     /* as decodehp_moe_decode */
    int32_t router_dtype;
    const void* shared_gate_row;
    const dhp_int4_experts* gate;
    const dhp_int4_experts* up;
    const dhp_int4_experts* down;
    const dhp_int4* shared_gate;
    const dhp_int4* shared_up;
    const dhp_int4* shared_down;
    int32_t top_k;
    int32_t moe_flags;
} dhp_decode_layer;

/* Workspace bytes decodehp_decode_layers needs (0 for invalid arguments). */
size_t decodehp_decode_layers_workspace_bytes(int32_t C, int32_t H, const dhp_decode_layer* layers,
                                              int32_t n_layers, const dhp_hc_block* mixer);

/*
 * decodehp_decode_layers -- one token through n_layers layers and the final mixer, on `stream`.
 *   x         : fp16 [H], 16-byte aligned (read once, at entry).
 *   layers    : n_layers >= 0 descriptors (read during the call only).
 *   mixer     : the final mixer (inject must be NULL).
 *   hidden    : fp16 [C*H], 16-byte aligned: the residual, replicated from x at entry; holds
 *               the residual after the last layer's inject on return. Between the steps the
 *               residual alternates between hidden and a buffer in ws (an inject writes a new
 *               copy instead of updating in place); the count of injects is even, so the last
 *               one lands in hidden.
 *   mixed_out : fp16 [H], the mixer's output.
 *   ws        : decodehp_decode_layers_workspace_bytes(...) bytes, 16-byte aligned.
 * Each step is an entry point of its own with its checks and errors: the first read is
 * decodehp_hc_read; every later read, the mixer's included, is decodehp_hc_inject_read (the
 * previous sublayer's inject fused in front); the sublayers are decodehp_dequant_gemv (the
 * stand-in) and decodehp_moe_decode. On an error the sequence stops there and hidden and
 * mixed_out are unspecified.
 */
int decodehp_decode_layers(const void* x, int32_t C, int32_t H, float eps, const dhp_decode_layer* layers,
                           int32_t n_layers, const dhp_hc_block* mixer, void* hidden, void* mixed_out,
                           void* ws, size_t ws_bytes, void* stream);

/*
 * A captured decodehp_decode_layers sequence. Capture first waits for all work on the device
 * (hipDeviceSynchronize: inputs written by asynchronous work on any stream are complete), runs
 * the sequence once on a private stream (it writes hidden and mixed_out), then records it and
 * waits for the private stream again before returning; every launch replays it on the
 * given stream with the same buffers (write the next token into x before a launch). The
 * descriptors may be freed after capture; the weights and buffers must outlive the graph.
 * Errors: those of decodehp_decode_layers, and -6 when capture or instantiation fails.
 */
typedef struct dhp_graph dhp_graph;
int decodehp_graph_capture_decode_layers(const void* x, int32_t C, int32_t H, float eps,
                                         const dhp_decode_layer* layers, int32_t n_layers,
                                         const dhp_hc_block* mixer, void* hidden, void* mixed_out,
                                         void* ws, size_t ws_bytes, dhp_graph** graph);
int decodehp_graph_launch(const dhp_graph* graph, void* stream);
void decodehp_graph_destroy(dhp_graph* graph);

/*
 * Measurement probes (not steps of the decode path): the launch floor, the cost of a grid-wide
 * barrier and the HBM read ceiling the decode kernels are measured against.
 *
 * decodehp_probe_empty -- launches `count` (1..100000) kernels that do nothing, back to back
 * on the stream. Errors: -2 count, -5, -6.
 *
 * decodehp_probe_read -- reads `bytes` of `buf` once with 16-byte nontemporal loads:
 * blocks_per_cu * (compute units) blocks of 256 threads in a grid stride, loads_in_flight
 * (1, 2, 4 or 8) loads per lane issued together. Block b writes the XOR of the words its
 * lanes read to sink[b] (so that no load can be dropped); the value means nothing else.
 *   buf : device memory, 16-byte aligned, bytes a multiple of 16.   sink : uint32 [sink_words],
 *   at least blocks_per_cu * compute units words.
 * Errors: -1 null buf/sink or zero bytes, -2 blocks_per_cu outside 1..16 or loads_in_flight,
 *         -3 alignment, -4 sink too small, -5, -6.
 *
 * decodehp_probe_grid_barrier -- one launch of `blocks` (1..compute units) blocks of 256 threads
 * that pass n (0..10000) grid-wide barriers: the cost of joining all blocks inside a launch, to
 * set against a kernel boundary. ordered != 0: each arrival is a device-scope release and each
 * wait ends with an acquire (the caches are written back and invalidated, as a barrier that
 * hands data between blocks needs); 0: relaxed atomics only. Every wait is bounded (2^18 polls);
 * one that runs out sets state[2] and ends the launch.
 *   state : uint32 [4] device memory, zero before the first call (left with state[0] = 0).
 *   sink  : uint32 [blocks]; block b writes 1 if all its waits ended normally.
 * Errors: -1 null state/sink, -2 blocks or n out of range, -5, -6.
 */
int decodehp_probe_empty(int32_t count, void* stream);
int decodehp_probe_grid_barrier(int32_t blocks, int32_t n, int32_t ordered, uint32_t* state, uint32_t* sink,
                                void* stream);
int decodehp_probe_read(const void* buf, size_t bytes, int32_t blocks_per_cu, int32_t loads_in_flight,
                        uint32_t* sink, int32_t sink_words, void* stream);

/* Workspace bytes an entry point needs (0 when none). Pure host arithmetic. */
size_t decodehp_workspace_bytes(int32_t op, int32_t a, int32_t b, int32_t c);

/* Message for the last nonzero return on this thread ("" if none). */
const char* decodehp_last_error(void);

/* Library ABI version, (major << 16) | minor. */
int32_t decodehp_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DECODEHP_H */
