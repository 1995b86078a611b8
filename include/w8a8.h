/*
 * w8a8.h — C ABI of the MI355X (gfx950) W8A8_DYNAMIC hot path.
 *
 * W8A8_DYNAMIC linear: per-token symmetric INT8 activation quantization, an
 * INT8 x INT8 -> INT32 matmul against offline per-channel INT8 weights, and a
 * dequant epilogue (acc * x_scale[m] * w_scale[n] + bias[n] -> BF16). The MoE
 * form runs the same matmul as a grouped GEMM driven by per-expert row counts:
 * W13 -> SwiGLU -> per-token requant -> W2.
 *
 * Page tags used in the comments:
 *   [DSV4]  "DeepSeek-V4 W8A8 执行链从量化权重到 Ascend INT8 算子"
 *
 * Conventions for every entry point:
 *   - Pointers named as device buffers are HIP device pointers on the current
 *     device. BF16 values travel as their uint16_t bit patterns.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream). Every call
 *     only enqueues work on it and returns without synchronizing.
 *   - The caller owns every buffer. The library never allocates or frees device
 *     memory and keeps no pointer after a call returns.
 *   - Arguments are checked on the host before anything is launched. A failed
 *     check launches nothing and returns a non-zero w8a8_status;
 *     w8a8_last_error() then returns a message for the calling thread.
 *   - Device-side problems (e.g. a group_list whose counts do not sum to R)
 *     are not detected by default. The kernels stay in bounds anyway (a
 *     negative count owns no rows; rows past R are never read or written),
 *     but the results are then not meaningful. With W8A8_CHECK set to
 *     anything but "" or "0" in the environment (read at every call), each
 *     call that takes a group_list first copies it to the host, which
 *     synchronizes the call's stream, and returns W8A8_ERR_SHAPE, launching
 *     nothing, for a negative count or counts summing past R. A debugging
 *     aid: it cannot be used under graph capture.
 *   - Sizes are int64_t element counts. M == 0 or R == 0 is a valid no-op.
 */
#ifndef W8A8_H
#define W8A8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  W8A8_OK = 0,
  W8A8_ERR_NULL = 1,        /* a required pointer is NULL */
  W8A8_ERR_SHAPE = 2,       /* a size is negative, zero where not allowed, or too large */
  W8A8_ERR_ALIGN = 3,       /* a buffer is not aligned as documented */
  W8A8_ERR_UNSUPPORTED = 4, /* a valid request this library does not implement */
  W8A8_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required */
  W8A8_ERR_LAUNCH = 6       /* a HIP launch failed (message from hipGetLastError) */
} w8a8_status;

typedef enum {
  W8A8_OUT_BF16 = 0,  /* epilogue output: BF16 bits, uint16_t */
  W8A8_OUT_I32 = 1    /* raw INT32 accumulator (no epilogue), int32_t */
} w8a8_out;

/* Flag OR-ed into the `out` argument of w8a8_linear: q is in the packed block
 * layout written by w8a8_dynamic_quant_packed instead of row-major. */
#define W8A8_A_PACKED 4

/* Input of w8a8_mx_grouped_gemm: the rows themselves, or the SwiGLU of
 * [gate | up] rows rounded to BF16. */
typedef enum {
  W8A8_ACT_NONE = 0,
  W8A8_ACT_SWIGLU = 1
} w8a8_act;

/* Largest K (reduction length) accepted: K * 127 * 127 stays below 2^31. */
#define W8A8_MAX_K 133144

const char* w8a8_status_str(int status);
/* Message of the last failed call on this thread ("" if none). */
const char* w8a8_last_error(void);
/* ABI version, bumped on any signature change. */
int w8a8_abi_version(void);

/*
 * Per-token symmetric INT8 quantization.  [DSV4 §一 recipe "act: per_token,
 * int8, symmetric"; §二 npu_dynamic_quant]
 *   x       device, BF16 [M, K] row-major (row stride K)
 *   q       device, int8 [M, K] row-major (row stride K), written
 *   x_scale device, float [M], written
 * For each row: amax = max_k |x[m,k]|; x_scale[m] = amax / 127 (one IEEE fp32
 * division); q[m,k] = round-half-even(x[m,k] / x_scale[m]) (one IEEE fp32
 * division) clamped to [-127, 127]. A row with amax == 0 gets scale 0 and
 * all-zero codes. K >= 1.
 */
int w8a8_dynamic_quant(const uint16_t* x, int64_t M, int64_t K, int8_t* q,
                       float* x_scale, void* stream);

/*
 * w8a8_dynamic_quant_ld [DSV4 §二 npu_dynamic_quant]: w8a8_dynamic_quant on
 *   row-strided buffers: row m of
 *   x at x + m * ldx (ldx >= K BF16 elements), its codes at q + m * ldq
 *   (ldq >= K bytes); codes and scales identical to w8a8_dynamic_quant
 *   (which is the case ldx = ldq = K). A ld below K is W8A8_ERR_SHAPE. For a
 *   column slice of a wider activation without a copy.
 */
int w8a8_dynamic_quant_ld(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int8_t* q, int64_t ldq,
                          float* x_scale, void* stream);

/*
 * The same quantization with the codes written in the packed block layout of
 * the weights (w8a8_prepack_weight with E = 1, the activation rows in the
 * place of the weight rows): 1 KB blocks [ceil(M/16)][ceil(K/64)], byte
 * (l*16 + j) of block (b, c) holding q[16 b + l%16][64 c + 16 (l/16) + j].
 * Codes of rows >= M and columns >= K inside the last blocks are left as
 * they are (they only ever meet zero weight padding or unstored outputs).
 * The tiled and decode GEMMs read such blocks as whole 1 KB pieces.
 *   q_packed device, w8a8_packed_weight_bytes(1, M, K) bytes, 16-byte aligned
 *   x        16-byte aligned; K % 8 == 0 (else W8A8_ERR_UNSUPPORTED)
 */
int w8a8_dynamic_quant_packed(const uint16_t* x, int64_t M, int64_t K, void* q_packed,
                              float* x_scale, void* stream);

/*
 * Load-time weight prepack.  [DSV4 §二: the INT8 [N, K] weight is transposed
 * and format-cast once at load and reused by every forward]
 * Packed layout ("P16x64"): K is zero-padded to Kp = ceil(K/64)*64 and N to
 * Np = ceil(N/16)*16. The packed buffer is a sequence of 1024-byte blocks
 * ordered [e][n/16][k/64]; inside a block byte (l*16 + j), l in [0,64),
 * j in [0,16), holds w[e][16*(n/16) + l%16][64*(k/64) + 16*(l/16) + j] — the
 * operand order of one 16x16x64 INT8 MFMA.
 *   w        device, int8 [E, N, K] row-major
 *   w_packed device, w8a8_packed_weight_bytes(E, N, K) bytes, 16-byte aligned
 * The packed buffer can be rewritten in place by a later call (stable address).
 */
int64_t w8a8_packed_weight_bytes(int64_t E, int64_t N, int64_t K);
int w8a8_prepack_weight(const int8_t* w, int64_t E, int64_t N, int64_t K,
                        void* w_packed, void* stream);

/*
 * Dense W8A8 quant matmul with the fused dequant epilogue.  [DSV4 §二:
 * npu_quant_matmul(q, weight, weight_scale, pertoken_scale, bias,
 * output_dtype=BF16)]
 *   q        device, int8 [M, K] row-major (from w8a8_dynamic_quant), or,
 *            with W8A8_A_PACKED in `out`, the packed blocks of
 *            w8a8_dynamic_quant_packed; or, when x_scale == NULL, the BF16
 *            activation x [M, K] row-major, quantized inside exactly as
 *            w8a8_dynamic_quant does ([DSV4 §三]: quantize only when the
 *            per-token scale is missing) — for M <= 2, or M <= 16 with
 *            M * K <= 16384 (K <= 16384, K % 8 == 0, x 16-byte aligned; every
 *            workgroup quantizes the rows again) in the same kernel as the
 *            product, else through the
 *            workspace; the result equals quant + linear bit for bit
 *   x_scale  device, float [M], or NULL for BF16 input
 *   w_packed device, packed weight of one [N, K] matrix (E = 1)
 *   w_scale  device, float [N]
 *   bias     device, BF16 [N] or NULL
 *   y        device, [M, N] row-major; BF16 bits when out == W8A8_OUT_BF16,
 *            int32 raw accumulators when out == W8A8_OUT_I32
 *   workspace/ws_bytes: device scratch of w8a8_linear_workspace_bytes(M, N,
 *            K) bytes, 256-byte aligned; needed only by the BF16-input branch
 *            beyond the fused case (INT8 input: NULL / 0 is fine)
 * y[m,n] = BF16(((float(acc[m,n]) * x_scale[m]) * w_scale[n]) + bias[n]),
 * each step one fp32 rounding (round to nearest even), acc exact in INT32.
 * 1 <= K <= W8A8_MAX_K.
 */
int64_t w8a8_linear_workspace_bytes(int64_t M, int64_t N, int64_t K);
int w8a8_linear(const int8_t* q, const float* x_scale, int64_t M, int64_t K,
                const void* w_packed, const float* w_scale, int64_t N,
                const uint16_t* bias, void* y, int out, void* workspace,
                int64_t ws_bytes, void* stream);

/*
 * w8a8_linear_ld [DSV4] §二: w8a8_linear on row-major INT8 codes with row
 *   strides: row m of q at q + m * ldq (ldq >= K), row m of y at y + m * ldy
 *   elements (ldy >= N; BF16 or INT32 by out). x_scale is required (codes
 *   input; the BF16-input and W8A8_A_PACKED forms stay with w8a8_linear).
 *   Results identical to w8a8_linear, which is the case ldq = K, ldy = N.
 *   Workspace as w8a8_linear's for codes input. A ld below K / N is
 *   W8A8_ERR_SHAPE.
 */
int w8a8_linear_ld(const int8_t* q, int64_t ldq, const float* x_scale, int64_t M, int64_t K,
                   const void* w_packed, const float* w_scale, int64_t N, const uint16_t* bias, void* y,
                   int64_t ldy, int out, void* workspace, int64_t ws_bytes, void* stream);

/*
 * Grouped INT8 matmul over experts.  [DSV4 §三: npu_grouped_matmul(x, weight,
 * scale, per_token_scale, group_list=expert_tokens); group_list gives the
 * number of rows of every expert]
 *   a          device, int8 [R, K] row-major; rows grouped by expert in
 *              expert order (expert e owns rows [off_e, off_e + n_e) where
 *              off_e = n_0 + ... + n_{e-1})
 *   a_scale    device, float [R]
 *   group_list device, int64 [E] row counts n_e >= 0 with sum R (read on the
 *              device only; never copied to the host)
 *   w_packed   device, packed [E, N, K] weight
 *   w_scale    device, float [E, N]
 *   y          device, [R, N]; BF16 bits or int32 as for w8a8_linear
 *   workspace  device scratch of w8a8_grouped_workspace_bytes(R, E, N, K)
 *              bytes, 256-byte aligned: the schedule the call builds first
 *              (per-expert row and tile offsets, the list of experts with at
 *              most 64 rows, the work-queue counters). Every call rewrites it,
 *              so two calls that share a workspace must not run concurrently.
 * Experts with n_e == 0 cost no work. No bias. E <= 1024.
 */
int64_t w8a8_grouped_workspace_bytes(int64_t R, int64_t E, int64_t N, int64_t K);
int w8a8_grouped_gemm(const int8_t* a, const float* a_scale,
                      const int64_t* group_list, int64_t R, int64_t E,
                      int64_t N, int64_t K, const void* w_packed,
                      const float* w_scale, void* y, int out, void* workspace,
                      int64_t ws_bytes, void* stream);

/*
 * Grouped GEMM for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * arguments, kernels and results as w8a8_grouped_gemm, without the workspace.
 * The schedule goes to a device array of this library (one copy per GPU,
 * 17,408 bytes: the schedule of E = 1024 experts, the most any call accepts;
 * held until the process ends). The device is the caller's current one, which
 * must own `stream`. Its device address is looked up on the first call on
 * each device; the call itself allocates nothing. Every call on one GPU shares
 * that array and rewrites it, so calls that overlap on one GPU (other streams,
 * other threads) race and must be serialized by the caller. Returns
 * W8A8_ERR_UNSUPPORTED for E > 1024, the other errors as w8a8_grouped_gemm.
 */
int w8a8_grouped_gemm_noalloc(const int8_t* a, const float* a_scale,
                              const int64_t* group_list, int64_t R, int64_t E,
                              int64_t N, int64_t K, const void* w_packed,
                              const float* w_scale, void* y, int out,
                              void* stream);

/*
 * Fused SwiGLU + per-token requant.  [DSV4 §三 and §五: "SwiGLU + Requant"
 * produces a new INT8 payload and a new per-token scale between W13 and W2;
 * §一: W13 is gate_proj + up_proj]
 *   h     device, BF16 [R, 2I]; columns [0, I) gate, [I, 2I) up
 *   q     device, int8 [R, I], written
 *   scale device, float [R], written
 * a[r,j] = silu(gate) * up evaluated in fp32 (exp by a fixed Cody-Waite +
 * degree-7 Taylor sequence, each step one fp32 rounding); then the
 * w8a8_dynamic_quant rule on a (no BF16 rounding of a). I >= 1.
 */
int w8a8_swiglu_quant(const uint16_t* h, int64_t R, int64_t I, int8_t* q,
                      float* scale, void* stream);

/*
 * MoE expert chain.  [DSV4 §三: routed hidden -> W13 grouped matmul -> SwiGLU
 * -> requant -> W2 grouped matmul -> BF16; the hidden states are quantized
 * only when they arrive without a per-token scale]
 *   x_rows     device; if x_scale == NULL: BF16 [R, H], quantized inside;
 *              else int8 [R, H] with its per-token scale x_scale [R]
 *   group_list device, int64 [E], as for w8a8_grouped_gemm
 *   w13_packed packed [E, 2I, H]; w13_scale float [E, 2I]
 *   w2_packed  packed [E, H, I];  w2_scale  float [E, H]
 *   y          device, BF16 [R, H] (rows in the same expert-grouped order,
 *              not combined across top-k)
 *   workspace  at least w8a8_moe_workspace_bytes(R, E, H, I) bytes
 */
int64_t w8a8_moe_workspace_bytes(int64_t R, int64_t E, int64_t H, int64_t I);
int w8a8_moe_grouped(const void* x_rows, const float* x_scale,
                     const int64_t* group_list, int64_t R, int64_t E, int64_t H,
                     int64_t I, const void* w13_packed, const float* w13_scale,
                     const void* w2_packed, const float* w2_scale, uint16_t* y,
                     void* workspace, int64_t ws_bytes, void* stream);

/*
 * Around the MoE chain on one GPU.  [DSV4 §三: the INT8 dispatch quantizes the
 * local BF16 hidden states once, to INT8 with one scale per token, and hands
 * the runner those rows together with topk_ids, topk_weights and the number
 * of rows of every expert; the runner feeds them to W13 without quantizing
 * again. The order of the rows and the combine arithmetic are not on the
 * page; the readings below are this library's.]
 *
 * w8a8_moe_route: topk_ids device int32 [T, top_k] -> group_list int64 [E]
 *   (rows per expert), row_token int32 [T * top_k] (the token of every
 *   expert-major row; entries past sum(group_list) are 0) and pair_row int32
 *   [T, top_k] (the row of pair (t, j), -1 for an id outside [0, E), which is
 *   dropped). Rows of one expert keep the order of the pair index
 *   t * top_k + j. 1 <= E <= 1024, T * top_k < 2^31. Work grows linearly
 *   with T * top_k; no workspace (past 32 * 1024 pairs pair_row holds
 *   per-chunk counts between the call's launches).
 * w8a8_moe_gather: q int8 [T, H] and scale float [T] of the tokens (from
 *   w8a8_dynamic_quant) -> q_rows int8 [R, H], s_rows float [R] with row p =
 *   token row_token[p]; a token outside [0, T) gives a zero row, scale 0.
 * w8a8_moe_combine: y_rows BF16 [R, H] (from w8a8_moe_grouped), pair_row int32
 *   [T, top_k], topk_weights float [T, top_k] -> out BF16 [T, H] with
 *   out[t] = BF16(sum over j = 0 .. top_k - 1 in that order of
 *   fl32(w[t, j] * y_rows[pair_row[t, j]])), every product and every partial
 *   sum one fp32 rounding (no fused multiply-add) from +0.0; pair rows outside
 *   [0, R) contribute nothing.
 * w8a8_moe_layer: the whole layer, x BF16 [T, H] -> out BF16 [T, H]:
 *   w8a8_dynamic_quant of the T tokens, route, gather, the w8a8_moe_grouped
 *   chain on the INT8 rows (R = T * top_k; rows past sum(group_list) are not
 *   computed), combine. w13/w2 as for w8a8_moe_grouped; workspace of
 *   w8a8_moe_layer_workspace_bytes(T, top_k, E, H, I) bytes, 256-byte aligned,
 *   rewritten by every call.
 * All buffers are device memory owned by the caller; int32 / float arrays
 * 4-byte aligned, group_list 8-byte aligned.
 */
int w8a8_moe_route(const int32_t* topk_ids, int64_t T, int64_t top_k, int64_t E,
                   int64_t* group_list, int32_t* row_token, int32_t* pair_row, void* stream);
int w8a8_moe_gather(const int8_t* q, const float* scale, int64_t T, int64_t H,
                    const int32_t* row_token, int64_t R, int8_t* q_rows, float* s_rows,
                    void* stream);
int w8a8_moe_combine(const uint16_t* y_rows, int64_t R, int64_t H, const int32_t* pair_row,
                     const float* topk_weights, int64_t T, int64_t top_k, uint16_t* out,
                     void* stream);
int64_t w8a8_moe_layer_workspace_bytes(int64_t T, int64_t top_k, int64_t E, int64_t H,
                                       int64_t I);
int w8a8_moe_layer(const uint16_t* x, int64_t T, int64_t H, const int32_t* topk_ids,
                   const float* topk_weights, int64_t top_k, int64_t E, int64_t I,
                   const void* w13_packed, const float* w13_scale, const void* w2_packed,
                   const float* w2_scale, uint16_t* out, void* workspace, int64_t ws_bytes,
                   void* stream);

/*
 * MXFP8 variant.  [MXFP8] = "Qwen3.8-FP8 on Ascend 950: Why Weights Become
 * MXFP8 at Load Time". E4M3 = OCP E4M3FN (largest finite 448); E8M0 byte b
 * stands for 2^(b - 127). Scales are row-major [rows, K/32] at this boundary.
 * K must be a multiple of 32 (else W8A8_ERR_UNSUPPORTED; [MXFP8] "Where It
 * Breaks or Falls Back": such layers do not take the MX path).
 *
 * w8a8_mx_quant  [MXFP8 Deep Dive 3 and 5]: BF16 x [M, K] -> E4M3 payload
 *   e4m3 [M, K] + e8m0 [M, K/32], one shared exponent per 32 values along K:
 *   scale_alg 0: E = floor(log2(amax)) - 8; scale_alg 1: the smallest E with
 *   amax / 2^E <= 448; E clamped to [-127, 127], amax == 0 -> byte 0. Payload =
 *   E4M3(x / 2^E), round to nearest even, subnormals kept, saturating at 448,
 *   sign of zero kept. x 16-byte aligned, e4m3 8-byte aligned.
 */
int w8a8_mx_quant(const uint16_t* x, int64_t M, int64_t K, uint8_t* e4m3, uint8_t* e8m0,
                  int scale_alg, void* stream);

/*
 * w8a8_mx_resolve_block_fp8  [MXFP8 Deep Dive 1 and 2, resolve equation]:
 *   w_bf16[i, j] = BF16(fp32(w_e4m3[i, j]) * scale_inv[i / BN, j / BK]), the
 *   product one fp32 rounding, BF16 round to nearest even; scale_inv is fp32
 *   [ceil(N/BN), ceil(K/BK)] (edge tiles cropped). All device pointers.
 */
int w8a8_mx_resolve_block_fp8(const uint8_t* w_e4m3, const float* scale_inv, int64_t N,
                              int64_t K, int64_t BN, int64_t BK, uint16_t* w_bf16, void* stream);

/*
 * w8a8_mx_prepack_weight  [MXFP8 Deep Dive 4: the MX weight and its scales
 *   are re-laid out once for the kernel, into stable buffers]: E4M3 [N, K] +
 *   E8M0 [N, K/32] -> one packed buffer of w8a8_mx_packed_bytes(N, K) bytes,
 *   256-byte aligned (payload in the P16x64 block layout of
 *   w8a8_prepack_weight, then the scales k-block major).
 */
int64_t w8a8_mx_packed_bytes(int64_t N, int64_t K);
int w8a8_mx_prepack_weight(const uint8_t* w_e4m3, const uint8_t* w_e8m0, int64_t N, int64_t K,
                           void* packed, void* stream);

/*
 * w8a8_mx_linear  [MXFP8 Deep Dive 5]: y [M, N] BF16 = block-scaled product of
 *   the MX activation and the packed MX weight: both operands dequantized
 *   exactly to BF16 (E4M3 x 2^E), exact products on the BF16 MFMA, fp32
 *   accumulation, BF16 round to nearest even.
 *   x: BF16 [M, K] (MX-quantized inside with scale_alg) when x_e8m0 == NULL,
 *   else an E4M3 payload [M, K] with its E8M0 scales x_e8m0 [M, K/32].
 *   workspace: w8a8_mx_linear_workspace_bytes(M, K) bytes, 256-byte aligned.
 */
int64_t w8a8_mx_linear_workspace_bytes(int64_t M, int64_t K);
int w8a8_mx_linear(const void* x, const uint8_t* x_e8m0, int64_t M, int64_t K,
                   const void* w_packed, int64_t N, uint16_t* y, int scale_alg, void* workspace,
                   int64_t ws_bytes, void* stream);

/*
 * w8a8_mx_gemm  [MXFP8 Deep Dive 5, the block-scaled matmul alone]: the GEMM
 *   stage of w8a8_mx_linear, for stage-wise tests and timing. a_e4m3: the
 *   E4M3 activation in the packed block layout of w8a8_prepack_weight (1 KB
 *   blocks [ceil(M/16)][ceil(K/64)], K zero-padded to 64), 256-byte aligned;
 *   a_scale_kb: E8M0 bytes "k-block major", [ceil(K/64)][Mp][2] with Mp = M
 *   rounded up to even, 4-byte aligned (the two 32-groups of one 64-deep
 *   k-block of a row adjacent; when K/32 is odd the last k-block's second
 *   byte of every row must be 0; the pad row, if any, is never used).
 *   After a call of w8a8_mx_linear its workspace holds exactly these two
 *   operands: the blocks at offset 0, the scales at offset
 *   ceil(M/16) * 16 * ceil(K/64) * 64 rounded up to 256. w_packed as for
 *   w8a8_mx_linear; y BF16 [M, N].
 */
int w8a8_mx_gemm(const uint8_t* a_e4m3, const uint8_t* a_scale_kb, int64_t M, int64_t K,
                 const void* w_packed, int64_t N, uint16_t* y, void* stream);

/*
 * MXFP8 MoE path.  [MXFP8] Deep Dive 6: the fused-MoE weights take the dense
 * contract (resolve -> MX re-quantization -> kernel layout) one expert at a
 * time, the expert's MXFP8 bytes written back over its FP8 source bytes and
 * its E8M0 scales into a separate buffer, so that the staging memory is one
 * dense expert; at run time the expert chain gets MX-quantized activations
 * (Deep Dive 5) and the routing metadata (group_list). The chain itself is
 * the INT8 path's ([DSV4] §三): W13 -> SwiGLU -> W2, with the SwiGLU output
 * rounded to BF16 and MX-quantized like any activation (a reading).
 *
 * w8a8_mx_moe_prepare (load time): w_e4m3 device uint8 [E, N, K], block-FP8
 *   E4M3 codes on entry, overwritten expert by expert with the MX payload
 *   (8-byte aligned, N * K % 8 == 0); scale_inv float [E, ceil(N/BN),
 *   ceil(K/BK)]; w_e8m0 uint8 [E, N, K/32] written; packed (optional, may be
 *   NULL) receives every expert's kernel layout at e * w8a8_mx_packed_bytes(N,
 *   K) (w8a8_mx_moe_packed_bytes(E, N, K) bytes, 256-byte aligned); staging
 *   at least w8a8_mx_moe_staging_bytes(N, K) bytes (one BF16 expert, 16-byte
 *   aligned). Per expert: w8a8_mx_resolve_block_fp8, w8a8_mx_quant (scale_alg),
 *   w8a8_mx_prepack_weight.
 * w8a8_mx_swiglu_quant: h BF16 [R, 2I] (gate | up, 16-byte aligned) -> e4m3
 *   [R, I] and e8m0 [R, I/32]: a = BF16(silu(gate) * up) by the fixed fp32
 *   sequence of w8a8_swiglu_quant, rounded once to BF16, then the MX quant of a.
 * w8a8_mx_grouped_gemm: rows grouped by expert as for w8a8_grouped_gemm
 *   (group_list int64 [E], counts cut to R rows in total); x BF16 [R, K]
 *   (act W8A8_ACT_NONE) or [R, 2K] = [gate | up] (act W8A8_ACT_SWIGLU, the
 *   input is then the BF16 SwiGLU above), 16-byte aligned; each row is
 *   MX-quantized at run time (scale_alg), multiplied with its expert's
 *   prepared weight (w_packed: E x w8a8_mx_packed_bytes(N, K), from
 *   w8a8_mx_moe_prepare) with exact BF16 products and fp32 accumulation ->
 *   y BF16 [R, N]. workspace: w8a8_mx_grouped_workspace_bytes(R, E, K), 256-byte
 *   aligned (tile schedule and the MX activation, every expert padded to 16
 *   rows). K % 32 == 0, E <= 1024.
 * w8a8_mx_moe_grouped: the chain on expert-grouped BF16 rows x [R, H] ->
 *   y BF16 [R, H]: w8a8_mx_grouped_gemm with w13 (N = 2I, K = H), then with
 *   w2 (N = H, K = I) on the SwiGLU of its output. workspace:
 *   w8a8_mx_moe_workspace_bytes(R, E, H, I). H % 32 == 0 and I % 32 == 0.
 * Results of the matmuls are the fp32 sums of exactly dequantized products,
 * rounded to BF16 (not bit-exact against a float64 sum; see w8a8_mx_linear).
 */
int64_t w8a8_mx_moe_staging_bytes(int64_t N, int64_t K);
int64_t w8a8_mx_moe_packed_bytes(int64_t E, int64_t N, int64_t K);
int w8a8_mx_moe_prepare(uint8_t* w_e4m3, const float* scale_inv, int64_t E, int64_t N, int64_t K,
                        int64_t BN, int64_t BK, int scale_alg, uint8_t* w_e8m0, void* packed,
                        void* staging, int64_t staging_bytes, void* stream);
int w8a8_mx_swiglu_quant(const uint16_t* h, int64_t R, int64_t I, int scale_alg, uint8_t* e4m3,
                         uint8_t* e8m0, void* stream);
int64_t w8a8_mx_grouped_workspace_bytes(int64_t R, int64_t E, int64_t K);
int w8a8_mx_grouped_gemm(const uint16_t* x, const int64_t* group_list, int64_t R, int64_t E,
                         int64_t N, int64_t K, int act, const void* w_packed, int scale_alg,
                         uint16_t* y, void* workspace, int64_t ws_bytes, void* stream);
int64_t w8a8_mx_moe_workspace_bytes(int64_t R, int64_t E, int64_t H, int64_t I);
int w8a8_mx_moe_grouped(const uint16_t* x_rows, const int64_t* group_list, int64_t R, int64_t E,
                        int64_t H, int64_t I, const void* w13_packed, const void* w2_packed,
                        int scale_alg, uint16_t* y, void* workspace, int64_t ws_bytes,
                        void* stream);

/*
 * Static W8A8  [DSV4, the static W8A8 comparison at the end of the page:
 * deq_scale = input_scale * weight_scale; quant_bias = round(fp_bias /
 * deq_scale - sum_k(Qw) * input_offset) as int32; BF16 X -> npu_quantize with
 * a fixed input_scale / input_offset -> INT8 X -> npu_quant_matmul(x, W,
 * deq_scale, bias=quant_bias) -> BF16 Y]. Per-tensor input_scale > 0 and
 * input_offset, both finite, passed by value.
 *
 * w8a8_static_quant: q[i] = clamp(rint(fl32(fl32(x[i] / input_scale) +
 *   input_offset)), -128, 127) elementwise (IEEE fp32 division and add, round
 *   half to even). x device BF16 [M, K] row-major, q device int8 [M, K].
 *   Non-finite x give unspecified codes.
 * w8a8_static_quant_packed: the same codes written in the packed block layout
 *   of w8a8_dynamic_quant_packed (1 KB blocks [ceil(M/16)][ceil(K/64)]; codes
 *   of rows past M and of columns past K are 0), w8a8_packed_weight_bytes(1,
 *   M, K) bytes, 16-byte aligned; for w8a8_static_linear with W8A8_A_PACKED.
 * w8a8_static_prepare (load time): from the INT8 weight w [N, K] row-major
 *   (the one given to w8a8_prepack_weight, E = 1), w_scale float [N] (every
 *   entry > 0, finite) and an optional BF16 bias [N] (NULL: fp_bias = 0),
 *   writes deq_scale[n] = fl32(input_scale * w_scale[n]) and quant_bias[n] =
 *   saturate_int32(rint(fl32(fl32(fp_bias[n] / deq_scale[n]) -
 *   fl32(fp32(S_n) * input_offset)))), S_n the exact sum of row n (float
 *   [N] and int32 [N], caller-owned, 4-byte aligned).
 * w8a8_static_linear: y[m, n] = BF16(fl32(fp32(acc[m, n] + quant_bias[n]) *
 *   deq_scale[n])) for out == W8A8_OUT_BF16, or the raw INT32 acc for
 *   W8A8_OUT_I32; q int8 [M, K] row-major (from w8a8_static_quant), or with
 *   W8A8_A_PACKED in `out` the blocks of w8a8_static_quant_packed; w_packed
 *   from w8a8_prepack_weight (E = 1). acc + quant_bias must fit in int32.
 *   Same kernels and plans as w8a8_linear.
 */
int w8a8_static_quant(const uint16_t* x, int64_t M, int64_t K, float input_scale,
                      float input_offset, int8_t* q, void* stream);
int w8a8_static_quant_packed(const uint16_t* x, int64_t M, int64_t K, float input_scale,
                             float input_offset, void* q_packed, void* stream);
int w8a8_static_prepare(const int8_t* w, int64_t N, int64_t K, const float* w_scale,
                        const uint16_t* bias, float input_scale, float input_offset,
                        float* deq_scale, int32_t* quant_bias, void* stream);
int w8a8_static_linear(const int8_t* q, int64_t M, int64_t K, const void* w_packed,
                       const float* deq_scale, const int32_t* quant_bias, int64_t N, void* y,
                       int out, void* stream);

/*
 * W4A16 weight variant.  [LOWBIT] = "超大 MoE 的低比特推理：INT4、FP4 与量化感知训练":
 * the INT4 format with one BF16 scale per 32 weights ("4 比特对万亿 MoE 意味着
 * 什么"), the symmetric per-32-input-channel quantizer of its QAT section
 * (scale = group amax / 7, codes clamped to [-8, 7]), and the W4A16 kernel row
 * of "不同硬件上的 kernel" (weights dequantized to BF16 in registers, BF16
 * matrix units; decode, where reading the weights is the bound).
 *
 * w8a8_w4a16_quant_weight (load time): BF16 w [N, K] (K % 32 == 0, else
 *   W8A8_ERR_UNSUPPORTED) -> per row and group of 32 along K:
 *   s = BF16(fl32(amax / 7)) (round half to even), q = clamp(rint(fl32(w /
 *   s)), -8, 7) against that stored scale; amax 0 gives s = 0 and q = 0.
 *   Writes any of: q int8 [N, K], scale BF16 bits [N, K/32], packed (16-byte
 *   aligned, w8a8_w4a16_packed_bytes(N, K) bytes); null outputs are skipped,
 *   at least one must be given.
 * w8a8_w4a16_pack: pre-quantized codes (int8; each is clamped to [-8, 7]
 *   before packing) and BF16 scales -> the packed layout.
 * w8a8_w4a16_linear: x BF16 [M, K] (16-byte aligned; M <= 16 * 65535, the
 *   rows of one launch, else W8A8_ERR_SHAPE) -> y BF16 [M, N] =
 *   BF16(sum_k x[m, k] * BF16(q * s)[n, k]): each weight dequantized once to
 *   BF16 (round half to even of the exact q * s), exact BF16 products,
 *   fp32 accumulation (not bit-exact against a float64 sum; no bias).
 *   workspace: w8a8_w4a16_linear_workspace_bytes(M, K) bytes, which is 0
 *   for every shape (NULL / 0 accepted; the linear stages its activation
 *   rows in LDS); the argument stays so that the signature does not change.
 * Packed layout: per 16-column block and 128-deep k-chunk 1152 bytes (codes +
 *   8 in nibbles in the BF16 MFMA's operand order, then the 16 x 4 BF16
 *   scales); K padded to 128 with zero weights.
 */
int64_t w8a8_w4a16_packed_bytes(int64_t N, int64_t K);
int w8a8_w4a16_quant_weight(const uint16_t* w, int64_t N, int64_t K, int8_t* q, uint16_t* scale,
                            void* packed, void* stream);
int w8a8_w4a16_pack(const int8_t* q, const uint16_t* scale, int64_t N, int64_t K, void* packed,
                    void* stream);
int64_t w8a8_w4a16_linear_workspace_bytes(int64_t M, int64_t K);
int w8a8_w4a16_linear(const uint16_t* x, int64_t M, int64_t K, const void* w_packed, int64_t N,
                      uint16_t* y, void* workspace, int64_t ws_bytes, void* stream);

/*
 * FP4 weights for the same W4A16 path ([LOWBIT]: the W4A16 row lists INT4 /
 * FP4 weights; MXFP4 = E2M1 values with one E8M0 scale per 32, 0.5 + 1/32
 * bytes per parameter).
 * w8a8_fp4_quant_weight (load time): BF16 w [N, K] (K % 32 == 0) -> per row
 *   and group of 32 along K: E = floor(log2 amax) - 2 (2 = E2M1's largest
 *   exponent), clamped to [-127, 127], scale byte E + 127 (0 for an all-zero
 *   group); each w / 2^E encoded to the nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6
 *   (ties to the even code, saturating at 6), sign bit 8 (-0 kept). Writes any
 *   of: codes uint8 [N, K] (0..15), scales uint8 [N, K/32], packed (16-byte
 *   aligned, w8a8_fp4_packed_bytes(N, K) bytes: per 16-column block and
 *   128-deep k-chunk 1088 bytes, the 1 KB of codes as nibbles in the order of
 *   w8a8_w4a16_quant_weight's layout, then the E8M0 bytes [16 columns][4
 *   groups]; K padded to 128 with zero codes).
 * w8a8_fp4_linear: x BF16 [M, K] (16-byte aligned) -> y BF16 [M, N] =
 *   BF16(sum_k x[m, k] * 2^E value[n, k]): the dequantized weights are exact
 *   in BF16, products exact, fp32 accumulation from +0 (a -0 weight adds
 *   nothing). Workspace as for w8a8_w4a16_linear.
 */
int64_t w8a8_fp4_packed_bytes(int64_t N, int64_t K);
int w8a8_fp4_quant_weight(const uint16_t* w, int64_t N, int64_t K, uint8_t* codes, uint8_t* scales,
                          void* packed, void* stream);
int w8a8_fp4_linear(const uint16_t* x, int64_t M, int64_t K, const void* w_packed, int64_t N,
                    uint16_t* y, void* workspace, int64_t ws_bytes, void* stream);

/*
 * Grouped form of the W4A16 / FP4 weight variant: the MoE experts' matmul with
 * low-bit expert weights ([LOWBIT]: MoE weights published as MXFP4 or INT4,
 * and in its kernel-table section 4-bit weights halve the bytes a decode step
 * reads; [DSV4] §三 for the grouping: rows sorted by expert, group_list =
 * rows per expert).
 *
 * fmt: W8A8_LOWBIT_INT4 (w8a8_w4a16_quant_weight's packed layout) or
 *   W8A8_LOWBIT_FP4 (w8a8_fp4_quant_weight's). Expert e's packed [N, K]
 *   weight starts at w_packed + e * w8a8_w4a16_packed_bytes(N, K) (INT4) or
 *   + e * w8a8_fp4_packed_bytes(N, K) (FP4); with N % 16 == 0 this is the
 *   packed layout of the stacked weight [E * N, K], so one quant call on the
 *   stack prepares every expert.
 * w8a8_w4a16_grouped_gemm: x BF16 rows [R, K] (16-byte aligned), grouped by
 *   expert: rows [off_e, off_e + n_e) with n_e = group_list[e] (device int64
 *   [E], E <= 1024, negative counts own no rows, counts summing past R are a
 *   caller error whose rows at or past R are never touched) times expert e's
 *   dequantized weight -> y BF16 [R, N] (8-byte aligned), each output as in
 *   w8a8_w4a16_linear / w8a8_fp4_linear: BF16 weights, exact products, fp32
 *   accumulation. N % 16 == 0 and K % 32 == 0, else W8A8_ERR_UNSUPPORTED. No
 *   workspace; group_list is read on the device only.
 * w8a8_w4a16_swiglu: h BF16 [R, 2I] = [gate | up] -> a BF16 [R, I] =
 *   BF16(silu(gate) * up), silu(g) * u = (g / (1 + exp(-g))) * u by the same
 *   fixed fp32 sequence as w8a8_swiglu_quant (bit-exact, round half to even).
 * w8a8_w4a16_moe_grouped: the expert chain on expert-grouped BF16 rows x_rows
 *   [R, H] -> y BF16 [R, H]: w8a8_w4a16_grouped_gemm with w13 (N = 2I, K = H;
 *   columns [0, I) gate, [I, 2I) up) into h BF16 [R, 2I], w8a8_w4a16_swiglu
 *   into a BF16 [R, I], w8a8_w4a16_grouped_gemm with w2 (N = H, K = I). No
 *   requantization between them (A16: the activations stay BF16). workspace:
 *   w8a8_w4a16_moe_workspace_bytes(R, H, I) bytes, 256-byte aligned: h at
 *   offset 0, a at the next 256-byte boundary after h (both left there);
 *   H % 32 == 0 and I % 32 == 0.
 */
#define W8A8_LOWBIT_INT4 0
#define W8A8_LOWBIT_FP4 1
int w8a8_w4a16_grouped_gemm(int fmt, const uint16_t* x, const int64_t* group_list, int64_t R, int64_t E,
                            int64_t N, int64_t K, const void* w_packed, uint16_t* y, void* stream);
int w8a8_w4a16_swiglu(const uint16_t* h, int64_t R, int64_t I, uint16_t* a, void* stream);
int64_t w8a8_w4a16_moe_workspace_bytes(int64_t R, int64_t H, int64_t I);
int w8a8_w4a16_moe_grouped(int fmt, const uint16_t* x_rows, const int64_t* group_list, int64_t R, int64_t E,
                           int64_t H, int64_t I, const void* w13_packed, const void* w2_packed, uint16_t* y,
                           void* workspace, int64_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* W8A8_H */
