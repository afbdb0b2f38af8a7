/*
 * mx.h - C ABI of the MXFP8 W8A8 linear layer for AMD Instinct MI355X (gfx950).
 *
 * The format is the one the model card "Wan2.2-I2V-A14B-Lightning · MXFP8
 * (AutoRound OptRTN)" states in its section "Quantization Details": 8-bit
 * weights and activations of data type mx_fp, group_size 32 along the
 * reduction axis K, symmetric, activations quantized dynamically at run time;
 * elements are FP8 E4M3, each group of 32 shares one E8M0 scale; the linear
 * layers carry F16 biases. Accumulation is FP32 (the FP32-accumulation FP8
 * mode of "Model Quantization Techniques", Conv3D mode table, which also fixes
 * the E4M3 range at 448).
 *
 * Quantization rule for one group of 32 values (OCP MX conversion):
 *   amax   = max |x_i|
 *   e      = clamp(floor(log2 amax) - 8, -127, 127)   (amax = 0 gives -127)
 *   scale  = E8M0 code e + 127
 *   code_i = E4M3(x_i * 2^-e), round to nearest even after saturating to
 *            +-448; the sign of zero is kept (-0 gives 0x80)
 *   A group holding NaN or Inf gets scale 0xFF and every code 0x7F.
 *
 * Conventions for every call:
 *   - All tensor pointers are DEVICE pointers; the caller allocates and frees
 *     them. The library keeps no tensor state and allocates nothing per call.
 *   - Layouts are row-major with K contiguous and no padding:
 *       activations  x  bf16  [M][K]   (mx_quantize_act also takes a row pitch)
 *       weights      w  fp32 or bf16 [N][K]  (nn.Linear orientation)
 *       codes        q  uint8 [rows][K]      (E4M3)
 *       scales       s  uint8 [rows][K/32]   (E8M0; group g covers K 32g..32g+31)
 *       bias            f16 [N], or NULL for none
 *       output       y  bf16  [M][N]
 *   - `stream` is a hipStream_t (NULL is the default stream). Calls enqueue
 *     work and return; faults inside a kernel surface at the caller's next
 *     synchronisation.
 *   - Arguments are checked on the host before anything is launched. Every
 *     call returns an mx_status; nothing is thrown and nothing aborts.
 *     MX_ERR_INVALID_ARGUMENT: a required pointer is NULL; M, N < 0; K not a
 *       positive multiple of 32; a pitch below K; x, q, w codes or y not
 *       16-byte aligned (bias 2-byte aligned); an output overlapping an input;
 *       an unknown epilogue or dtype.
 *     MX_ERR_UNSUPPORTED: the current device is not gfx950 (or the environment
 *       sets MX_FORCE_UNSUPPORTED=1).
 *     MX_ERR_HIP: a HIP runtime call or a launch failed; mx_last_hip_error()
 *       gives its hipError_t.
 *     M = 0 or N = 0 is an empty call: MX_OK, nothing launched.
 *   - Results are deterministic: the same inputs give the same bytes.
 */
#ifndef MX_H
#define MX_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MX_ABI_VERSION 12

typedef enum {
  MX_OK = 0,
  MX_ERR_INVALID_ARGUMENT = 1,
  MX_ERR_UNSUPPORTED = 2,
  MX_ERR_HIP = 3
} mx_status;

/* Epilogue applied to acc + bias before the bf16 rounding. GELU is the tanh
 * form, 0.5 v (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3))), the activation of
 * the Wan2.2 feed-forward up-projection (ffn.net.0.proj). */
typedef enum { MX_EPI_NONE = 0, MX_EPI_GELU_TANH = 1 } mx_epilogue;

/* Element type of the weights handed to mx_quantize_weight. */
typedef enum { MX_DT_BF16 = 0, MX_DT_F32 = 1 } mx_dtype;

/* MX_ABI_VERSION of the built library. */
int mx_abi_version(void);

/* Static, human-readable name of a status code. */
const char* mx_status_string(int status);

/* hipError_t of the last MX_ERR_HIP returned on the calling thread (0 if none). */
int mx_last_hip_error(void);

/* Detail of the last non-OK status returned on the calling thread (static
 * storage of that thread; "" if none). */
const char* mx_last_error_message(void);

/* Dynamic activation quantization ("act_dynamic", "act_group_size 32").
 * x: bf16 [M][ldx] with ldx >= K and ldx % 8 == 0; q: uint8 [M][K];
 * s: uint8 [M][K/32]. Bit-exact with the rule above. */
int mx_quantize_act(const void* x, int64_t M, int64_t K, int64_t ldx,
                    uint8_t* q, uint8_t* s, void* stream);

/* Weight quantization by the same rule: the model card keeps its weights as
 * E4M3 codes with one E8M0 scale for each 32 along K (section "Quantization
 * Details"). w: [N][ldw] of type wdtype (MX_DT_F32 or MX_DT_BF16),
 * ldw >= K, ldw * sizeof(element) % 16 == 0; q: uint8 [N][K]; s: uint8 [N][K/32]. */
int mx_quantize_weight(const void* w, int wdtype, int64_t N, int64_t K, int64_t ldw,
                       uint8_t* q, uint8_t* s, void* stream);

/* The MXFP8 W8A8 linear on row-major weights with the activation
 * quantization fused into the GEMM's prologue (each 256-token tile quantized
 * in the kernel, once for every 256 weight rows, no workspace):
 *   y[m][n] = bf16_rne( epi( sum_k xhat[m][k] * what[n][k] + f32(bias[n]) ) )
 * with xhat the MX quantization of x (same rule as mx_quantize_act) and what
 * the dequantized weights (wq, ws). Products are exact, sums are FP32.
 * x: bf16 [M][K]; wq: uint8 [N][K]; ws: uint8 [N][K/32]; bias: f16 [N] or
 * NULL; epilogue: mx_epilogue; y: bf16 [M][N]. Correct for any K % 32 == 0
 * but slow: every 256 x 256 tile quantizes its bf16 token rows again, and the
 * kernel holds them beside 256 accumulators per lane and spills (about 760
 * TFLOP/s at 75348 x 5120 x 15360, against about 2600 for mx_linear). Kept
 * for callers without slab weights or workspace.
 * Passage: model card "Wan2.2-I2V-A14B-Lightning · MXFP8 (AutoRound OptRTN)",
 * section "Quantization Details" (activations quantized at run time). */
int mx_linear_fused(const void* x, int64_t M, int64_t K,
                    const uint8_t* wq, const uint8_t* ws, int64_t N,
                    const void* bias, int epilogue, void* y, void* stream);

/* The same linear on activations already quantized (e.g. by
 * mx_quantize_act): xq: uint8 [M][K], xs: uint8 [M][K/32].
 * Passage: model card "Wan2.2-I2V-A14B-Lightning · MXFP8 (AutoRound OptRTN)",
 * section "Quantization Details". */
int mx_linear_q(const uint8_t* xq, const uint8_t* xs, int64_t M, int64_t K,
                const uint8_t* wq, const uint8_t* ws, int64_t N,
                const void* bias, int epilogue, void* y, void* stream);

/* ------------------------------------------------------------------------
 * Slab layout. The same codes and scales, stored for the GEMM's tiles rather
 * than by row: with R = mx_slab_rows(rows) (rows rounded up to 256) and K a
 * multiple of 64,
 *   codes   q  uint8 [K/64][R][64]   q[j][r][i] = code of row r, k = 64 j + i
 *   scales  s  uint8 [K/64][R][2]    s[j][r][h] = scale of row r, group 2 j + h
 * Rows rows..R-1 hold zero codes and zero scales. One 256-row tile's share of
 * a 64-K slab is then one contiguous run (16 KB of codes, 512 B of scales),
 * which the GEMM streams with whole-line loads. Values are bit-identical to
 * the row-major calls above; only the placement differs.
 * ------------------------------------------------------------------------ */

/* R for a slab-layout operand of `rows` rows; -1 if rows < 0. */
int64_t mx_slab_rows(int64_t rows);

/* mx_quantize_act writing the slab layout. K % 64 == 0; q: uint8
 * [K/64][R][64], s: uint8 [K/64][R][2] with R = mx_slab_rows(M).
 * Passage: model card "Wan2.2-I2V-A14B-Lightning · MXFP8 (AutoRound OptRTN)",
 * section "Quantization Details" (dynamic MXFP8 activations). */
int mx_quantize_act_slab(const void* x, int64_t M, int64_t K, int64_t ldx,
                         uint8_t* q, uint8_t* s, void* stream);

/* mx_quantize_weight writing the slab layout (R = mx_slab_rows(N)).
 * Passage: model card "Wan2.2-I2V-A14B-Lightning · MXFP8 (AutoRound OptRTN)",
 * section "Quantization Details" (E4M3 weights, one E8M0 scale per 32). */
int mx_quantize_weight_slab(const void* w, int wdtype, int64_t N, int64_t K, int64_t ldw,
                            uint8_t* q, uint8_t* s, void* stream);

/* Row-major codes q [rows][K] and scales s [rows][K/32] (e.g. weights that
 * were stored quantized) to the slab layout qslab, sslab. K % 64 == 0; codes
 * 16-byte aligned, scales 2-byte aligned; outputs must not overlap inputs.
 * Passage: model card "Wan2.2-I2V-A14B-Lightning · MXFP8 (AutoRound OptRTN)",
 * section "Quantization Details" (weights stored quantized). */
int mx_slab_pack(const uint8_t* q, const uint8_t* s, int64_t rows, int64_t K,
                 uint8_t* qslab, uint8_t* sslab, void* stream);

/* The linear of mx_linear_q on slab-layout operands: xq [K/64][RM][64],
 * xs [K/64][RM][2] (RM = mx_slab_rows(M)), wq [K/64][RN][64], ws [K/64][RN][2]
 * (RN = mx_slab_rows(N)); bias f16 [N] or NULL; y bf16 [M][N] row-major.
 * K % 64 == 0 (else MX_ERR_INVALID_ARGUMENT), N % 16 == 0 (else
 * MX_ERR_UNSUPPORTED); codes and y 16-byte aligned, scales 4-byte aligned.
 * The result is bit-identical to mx_linear_q on the same codes and scales.
 * Passage: model card "Wan2.2-I2V-A14B-Lightning · MXFP8 (AutoRound OptRTN)",
 * section "Quantization Details". */
int mx_linear_slab(const uint8_t* xq, const uint8_t* xs, int64_t M, int64_t K,
                   const uint8_t* wq, const uint8_t* ws, int64_t N,
                   const void* bias, int epilogue, void* y, void* stream);

/* mx_linear_slab on 256 (weight rows) x 128 (tokens) tiles: the same
 * arguments, checks and result bit for bit (every output is the same chain
 * of MFMAs from the bias), with twice as many tiles. For a few hundred tokens
 * (the 512 text tokens of Wan2.2's attn2 k/v: 80 tiles of 256 x 256 on the
 * MI355X's 256 CUs) the 256 x 256 tiles leave most CUs idle; this form
 * fills more of them without splitting K, so there are no partial sums to
 * write and reduce (model card "Wan2.2-I2V-A14B-Lightning · MXFP8 (AutoRound
 * OptRTN)", section "Quantization Details": the cross-attention projections
 * are among the quantized linears). */
int mx_linear_slab_m128(const uint8_t* xq, const uint8_t* xs, int64_t M, int64_t K,
                        const uint8_t* wq, const uint8_t* ws, int64_t N,
                        const void* bias, int epilogue, void* y, void* stream);

/* The same linear, writing instead of y the MX quantization of bf16 y (by
 * the rule above, bit-identical to mx_quantize_act_slab of mx_linear_slab's
 * output) in the slab layout of an operand with rows M and K' = N:
 * hq [N/64][RM][64], hs [N/64][RM][2], RM = mx_slab_rows(M); pad rows are
 * zero. This is the feed-forward pair of Wan2.2 (ffn.net.0.proj with GELU,
 * then ffn.net.2 on the requantized intermediate) without the bf16
 * intermediate in memory. N % 64 == 0 (else MX_ERR_INVALID_ARGUMENT);
 * RM * N < 2^31 (else MX_ERR_UNSUPPORTED); hq 16-byte aligned; outputs must
 * not overlap the inputs or each other.
 * Passage: model card "Wan2.2-I2V-A14B-Lightning · MXFP8 (AutoRound OptRTN)",
 * section "Quantization Details" (ffn.net.0.proj and ffn.net.2 are both
 * quantized linears). */
int mx_linear_slab_requant(const uint8_t* xq, const uint8_t* xs, int64_t M, int64_t K,
                           const uint8_t* wq, const uint8_t* ws, int64_t N,
                           const void* bias, int epilogue, uint8_t* hq, uint8_t* hs, void* stream);

/* ------------------------------------------------------------------------
 * Split-K for few token tiles. With M of a few hundred tokens (the 128-token
 * linear, the 512 text tokens of attn2 k/v) the 256 x 256 tiles are too few to
 * occupy the GPU's CUs, and each one runs the whole K loop. The split-K form
 * gives each tile `splits` consecutive ranges of the K/64 slabs, one
 * workgroup per (tile, range), writing fp32 partial sums into a workspace;
 * a second kernel adds the ranges in order 0, 1, ..., adds the bias, applies
 * the epilogue and rounds to bf16. The reduction order is fixed, so results
 * are deterministic; splits = 1 runs mx_linear_slab's kernel (same bits, no
 * workspace used), otherwise the fp32 sums are associated differently (same
 * tolerance).
 * ------------------------------------------------------------------------ */

/* Workspace bytes for mx_linear_slab_splitk: splits * T * 256 KiB with
 * T = ceil(M/256) * ceil(N/256) (fp32 partial tiles); -1 on bad arguments. */
int64_t mx_linear_splitk_ws_bytes(int64_t M, int64_t N, int splits);

/* A split count that gives at most one workgroup per CU of an MI355X (256),
 * at most 8 ranges (the partial sums' traffic grows with the count) and at
 * least two 64-K slabs per range; 1 when the tiles alone fill the CUs. */
int mx_linear_splitk_choose(int64_t M, int64_t K, int64_t N);

/* mx_linear_slab with split-K (operands, bias, epilogue and y as there).
 * 1 <= splits <= K/64 (else MX_ERR_INVALID_ARGUMENT); T * splits <= 2^24
 * (else MX_ERR_UNSUPPORTED). workspace: device memory of at least
 * mx_linear_splitk_ws_bytes(M, N, splits) bytes, 256-byte aligned, not
 * overlapping the operands, bias or y; overwritten. Two kernels on `stream`;
 * nothing is allocated.
 * Passage: model card "Wan2.2-I2V-A14B-Lightning · MXFP8 (AutoRound OptRTN)",
 * section "Quantization Details"; ragged token counts as in "Wan2.2 I2V A14B,
 * four-step 720p: native LightX2V FP8 and NVFP4", section "Runtime setup". */
int mx_linear_slab_splitk(const uint8_t* xq, const uint8_t* xs, int64_t M, int64_t K,
                          const uint8_t* wq, const uint8_t* ws, int64_t N,
                          const void* bias, int epilogue, void* y, int splits,
                          void* workspace, int64_t workspace_bytes, void* stream);

/* Few-token tiles. For M up to a few hundred the result is computed by a
 * kernel with 128-token x 64-weight-row tiles (four waves of 32 tokens), which
 * streams each weight row once per K range while the token slab stays in
 * the L2, instead of padding the tokens to 256. K is split into `splits`
 * ranges: splits = 1 writes y directly, bit-identical to mx_linear_slab (the
 * same chain of MFMAs in K order, started at the bias, and the same
 * epilogue); splits > 1 writes fp32
 * partials [splits][M][N] that a second kernel adds in range order before
 * bias, epilogue and bf16: fixed order, deterministic, the tolerance of
 * mx_linear_slab. */

/* Workspace bytes for mx_linear_slab_small: splits * M * N * 4 when
 * splits > 1, else 0; -1 on bad arguments. */
int64_t mx_linear_small_ws_bytes(int64_t M, int64_t N, int splits);

/* A split count for mx_linear_slab_small on the current device: about one
 * workgroup per CU (C / ceil(M/128) / ceil(N/64)), at most 8 ranges and at
 * least two 64-K slabs per range; 1 when the tiles alone fill the CUs or on
 * bad arguments. */
int mx_linear_small_choose(int64_t M, int64_t K, int64_t N);

/* mx_linear_slab through the few-token kernel (operands, bias, epilogue, y
 * and their errors as there). 1 <= splits <= K/64 (else
 * MX_ERR_INVALID_ARGUMENT); ceil(M/128) * ceil(N/64) * splits <= 2^24 and
 * (K/64 + 16) * 64 * R < 2^31 for R = M and N rounded up to 256 (else
 * MX_ERR_UNSUPPORTED). workspace: at least mx_linear_small_ws_bytes(M, N,
 * splits) bytes, 256-byte aligned, not overlapping an operand, bias or y; may
 * be NULL when that is 0; overwritten. One or two kernels on `stream`;
 * nothing is allocated.
 * Passage: model card "Wan2.2-I2V-A14B-Lightning · MXFP8 (AutoRound OptRTN)",
 * section "Quantization Details"; ragged token counts as in "Wan2.2 I2V A14B,
 * four-step 720p: native LightX2V FP8 and NVFP4", section "Runtime setup". */
int mx_linear_slab_small(const uint8_t* xq, const uint8_t* xs, int64_t M, int64_t K,
                         const uint8_t* wq, const uint8_t* ws, int64_t N,
                         const void* bias, int epilogue, void* y, int splits,
                         void* workspace, int64_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Per-shape plans. A plan names the kernel for one slab-linear shape and its
 * K split: MX_PLAN_SLAB (mx_linear_slab, splits 1), MX_PLAN_SPLITK
 * (mx_linear_slab_splitk), MX_PLAN_SMALL (mx_linear_slab_small),
 * MX_PLAN_BALANCED (mx_linear_slab_balanced, splits 1), MX_PLAN_SLAB_M128
 * (mx_linear_slab_m128, splits 1). Every plan computes the same linear (same
 * operands, tolerance and determinism; SLAB, SLAB_M128, and SPLITK or SMALL
 * with splits 1, bit-identical). The library keeps a process-local
 * cache of tuned plans keyed by (device, M, K, N, epilogue), guarded by a
 * mutex; mx_linear_tune fills it, mx_linear_slab_auto reads it.
 * ------------------------------------------------------------------------ */
enum { MX_PLAN_SLAB = 0, MX_PLAN_SPLITK = 1, MX_PLAN_SMALL = 2, MX_PLAN_BALANCED = 3, MX_PLAN_SLAB_M128 = 4 };

/* The rule used without tuning: MX_PLAN_SMALL with mx_linear_small_choose
 * splits for 1 <= M <= 256; else MX_PLAN_SLAB_M128 when the 256 x 256 tiles
 * number 32 to 128 (one round of twice as many 128-token tiles then keeps a
 * quarter to all of an MI355X's 256 CUs busy); else MX_PLAN_SPLITK with
 * mx_linear_splitk_choose splits when that is above 1; else MX_PLAN_SLAB.
 * MX_ERR_INVALID_ARGUMENT on NULL outputs or a bad shape (M, N < 0; K not a
 * positive multiple of 64; sizes past the slab linear's limits). */
int mx_linear_plan_default(int64_t M, int64_t K, int64_t N, int* kind, int* splits);

/* Workspace bytes of a plan for this shape (0 when it needs none); -1 on a
 * bad kind, split count or shape. */
int64_t mx_linear_plan_ws_bytes(int kind, int splits, int64_t M, int64_t K, int64_t N);

/* mx_linear_slab through the given plan: the arguments, checks and errors of
 * that plan's entry point (workspace unused by MX_PLAN_SLAB).
 * Passage: per-shape kernel choice, "Model Quantization Techniques", section
 * "MiniMax-H3 FP8 with FP16 Accumulation". */
int mx_linear_slab_plan(int kind, int splits, const uint8_t* xq, const uint8_t* xs,
                        int64_t M, int64_t K, const uint8_t* wq, const uint8_t* ws,
                        int64_t N, const void* bias, int epilogue, void* y,
                        void* workspace, int64_t workspace_bytes, void* stream);

/* The largest workspace a candidate of mx_linear_tune uses for this shape
 * (so also enough for the plan it picks); -1 on a bad shape. */
int64_t mx_linear_tune_ws_bytes(int64_t M, int64_t K, int64_t N);

/* Warm-up tuning of one shape on the caller's operands: runs each candidate
 * plan once, then `reps` times between two HIP events on `stream` (1 <=
 * reps <= 1000), queued behind a short delay kernel so that they run back to
 * back (GPU time, as under graph replay), and keeps the fastest. Candidates: the default plan; the
 * slab GEMM; split-K with 2, 3, 4, 6, 8 ranges when the 256 x 256 tiles are
 * fewer than the device's CUs; for M > 128 the 128-token tiles when the
 * 256 x 256 tiles are fewer than twice the CUs; the few-token kernel with 1, 2, 3, 4, 6, 8
 * ranges for M <= 1024; the balanced GEMM when the tiles leave a partial
 * last round. Candidates whose workspace exceeds workspace_bytes, or that
 * their entry point rejects, are skipped. The choice is cached for (current
 * device, M, K, N, epilogue) and written to *kind, *splits. y is
 * overwritten; the stream is synchronized (not for use under graph
 * capture). Errors: those of the slab linear's checks, MX_ERR_INVALID_ARGUMENT
 * when no candidate fits the workspace, MX_ERR_HIP from the runs.
 * Passage: per-shape tuning at warm-up, "Model Quantization Techniques",
 * section "MiniMax-H3 FP8 with FP16 Accumulation". */
int mx_linear_tune(const uint8_t* xq, const uint8_t* xs, int64_t M, int64_t K,
                   const uint8_t* wq, const uint8_t* ws, int64_t N,
                   const void* bias, int epilogue, void* y,
                   void* workspace, int64_t workspace_bytes, int reps, void* stream,
                   int* kind, int* splits);

/* The cached plan of (current device, M, K, N, epilogue) if tuned, else the
 * default plan. */
int mx_linear_plan_lookup(int64_t M, int64_t K, int64_t N, int epilogue, int* kind, int* splits);

/* mx_linear_slab through mx_linear_plan_lookup's plan. workspace: at least
 * mx_linear_plan_ws_bytes of that plan (mx_linear_tune_ws_bytes always
 * suffices); may be NULL when the plan needs none. Nothing is allocated.
 * Passage: per-shape tuning at warm-up, "Model Quantization Techniques",
 * section "MiniMax-H3 FP8 with FP16 Accumulation". */
int mx_linear_slab_auto(const uint8_t* xq, const uint8_t* xs, int64_t M, int64_t K,
                        const uint8_t* wq, const uint8_t* ws, int64_t N,
                        const void* bias, int epilogue, void* y,
                        void* workspace, int64_t workspace_bytes, void* stream);

/* Empties the plan cache. */
void mx_linear_plan_clear(void);

/* ------------------------------------------------------------------------
 * The linear in one call: the production entry point. What the model card
 * "Wan2.2-I2V-A14B-Lightning · MXFP8 (AutoRound OptRTN)" describes in
 * "Quantization Details" for each of its quantized linears: bf16 activations
 * quantized to MXFP8 at run time, multiplied against E4M3 weight codes that
 * carry one E8M0 scale per 32 elements, F16 bias; FP32 accumulation, bf16
 * output:
 *   y[m][n] = bf16_rne( epi( sum_k xhat[m][k] * what[n][k] + f32(bias[n]) ) )
 * ------------------------------------------------------------------------ */

/* Bytes of workspace mx_linear needs for an M x K x N linear: the activation
 * slab (mx_slab_rows(M) * K * 33 / 32) and the partial sums of any plan
 * mx_linear_tune may pick for the shape, each rounded up to 256 bytes. 0 for
 * M = 0 or N = 0; -1 on a bad shape (K not a positive multiple of 64, sizes
 * past the limits). */
int64_t mx_linear_ws_bytes(int64_t M, int64_t K, int64_t N);

/* The whole quantized linear in one call: the activations quantized to MXFP8
 * at run time, then the block-scaled product with the stored MXFP8 weights
 * (model card "Wan2.2-I2V-A14B-Lightning · MXFP8 (AutoRound OptRTN)",
 * section "Quantization Details"). This is the production entry point.
 * x bf16 [M][ldx] (ldx >= K, ldx % 8 == 0) is quantized into `workspace`
 * (mx_quantize_act_slab's layout), then multiplied by the slab weights
 * wq [K/64][RN][64], ws [K/64][RN][2] (mx_quantize_weight_slab or
 * mx_slab_pack) with bias (f16 [N] or NULL) and epilogue into y bf16 [M][N],
 * through the shape's plan (mx_linear_plan_lookup: tuned if mx_linear_tune
 * ran for it, else the default rule; a tuned plan that needs more workspace
 * than given gives way to the default one): two kernels on `stream` (the
 * quantizer, then the GEMM), plus the ordered reduction of the partial sums
 * for plans with several K ranges. Nothing is allocated. workspace: device
 * memory of mx_linear_ws_bytes(M, K, N) bytes (at least what the chosen
 * plan needs), 256-byte aligned, not overlapping x, the weights, bias or y;
 * its contents are overwritten and need no initial value. K % 64 == 0, N % 16 == 0.
 * Results: deterministic; bit-identical to mx_quantize_act_slab +
 * mx_linear_slab_plan with the same plan. Errors: as mx_linear_slab, plus
 * MX_ERR_INVALID_ARGUMENT for a bad pitch, a short or misplaced workspace. */
int mx_linear(const void* x, int64_t M, int64_t K, int64_t ldx,
              const uint8_t* wq, const uint8_t* ws, int64_t N,
              const void* bias, int epilogue, void* y,
              void* workspace, int64_t workspace_bytes, void* stream);

/* mx_linear for callers that cannot allocate: code under HIP graph capture,
 * serving loops that keep allocation out of their hot path, harnesses that
 * forbid hipMalloc. The same linear, plan and results (bit for bit) as
 * mx_linear, with no workspace argument: its workspace is a scratch array
 * the library owns, 64 MiB of static device memory per GPU, held until the
 * process ends; its device address is looked up once per device, on the
 * first call. Limit: the activation slab and the plan's partial sums must
 * fit in those 64 MiB (a tuned plan that does not fit gives way to the
 * default plan first); larger shapes are MX_ERR_UNSUPPORTED (checked before
 * anything is launched; e.g. up to about 12000 tokens at K = 5120). Every
 * call on a GPU shares that GPU's array and leaves its contents behind (no
 * kernel relies on them: each call writes what it reads): calls that
 * overlap in time on one GPU (several streams, concurrent graph replays)
 * race and give wrong results, so serialise them. Nothing is allocated.
 * Other errors: as mx_linear. */
int mx_linear_noalloc(const void* x, int64_t M, int64_t K, int64_t ldx,
                      const uint8_t* wq, const uint8_t* ws, int64_t N,
                      const void* bias, int epilogue, void* y, void* stream);

/* ------------------------------------------------------------------------
 * Measurement. The MFMA peak that the 5.0 PFLOP/s figure assumes needs the
 * full clock, which the chip does not hold when the matrix cores work on
 * real operand bits. This probe measures what the scaled FP8 MFMA sustains
 * with no memory traffic at all, on codes the caller chooses (for instance
 * the workload's own codes, or zeros).
 * ------------------------------------------------------------------------ */

/* Launches `blocks` workgroups of 4 waves (one per CU gives the whole GPU):
 * each lane reads 128 bytes of A codes and 128 bytes of B codes (32-bit words
 * taken modulo bytes / 4 from a and b, any E4M3 bytes), then issues 16 * iters
 * independent v_mfma_scale_f32_32x32x64_f8f6f4 (unit block scales) from
 * registers and writes one float per thread to sink (blocks * 256 floats).
 * Work: blocks * 4 * 16 * iters * 2 * 32 * 32 * 64 FLOP; time it with events
 * on `stream`. a, b, sink: device pointers, 4-byte aligned; 4 <= bytes <=
 * 2^31, a multiple of 4; 1 <= iters <= 2^20; 1 <= blocks <= 65536 (else
 * MX_ERR_INVALID_ARGUMENT). */
int mx_probe_mfma(const uint8_t* a, const uint8_t* b, int64_t bytes, int iters, int blocks,
                  float* sink, void* stream);

/* Workspace bytes mx_linear_slab_balanced needs on the current device: the
 * fp32 partial tiles of its split last round, 0 when it splits nothing; -1 on
 * bad arguments (M, N < 0; K not a positive multiple of 64). */
int64_t mx_linear_balanced_ws_bytes(int64_t M, int64_t K, int64_t N);

/* mx_linear_slab with its last, partial round of tiles split over K. The
 * T = ceil(M/256) * ceil(N/256) tiles run as full rounds of one tile per CU
 * (C = the device's compute units) and a last round of T mod C tiles that
 * would leave most CUs idle (75348 x 5120: 5900 tiles, 12 in the last round);
 * those tiles are split into s = min(C / (T mod C), 8, K/128) K ranges, their
 * fp32 partial sums reduced in fixed order (as mx_linear_slab_splitk). Tiles
 * of the full rounds are bit-identical to mx_linear_slab's, the split ones
 * equal up to the order of the fp32 sums; the split depends only on the shape
 * and C, so results are deterministic on a given device. workspace: at least
 * mx_linear_balanced_ws_bytes(M, K, N) bytes, 256-byte aligned, not
 * overlapping an operand, bias or y (may be NULL when that is 0). Up to three
 * kernels on `stream`; nothing is allocated. Other arguments and errors as
 * mx_linear_slab.
 * Passage: model card "Wan2.2-I2V-A14B-Lightning · MXFP8 (AutoRound OptRTN)",
 * section "Quantization Details". */
int mx_linear_slab_balanced(const uint8_t* xq, const uint8_t* xs, int64_t M, int64_t K,
                            const uint8_t* wq, const uint8_t* ws, int64_t N,
                            const void* bias, int epilogue, void* y,
                            void* workspace, int64_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Per-output-channel FP8: the second FP8 scheme of the pages ("Wan2.2 I2V
 * A14B, four-step 720p: native LightX2V FP8 and NVFP4", section "Conversion
 * and compatibility": E4M3 weight codes scaled by one FP32 factor per
 * output channel, rounded to nearest; "Model Quantization Techniques", mode
 * table: FP8 weights symmetric per channel, FP8 activations symmetric per
 * row and computed on the fly as max(abs(x)) / qmax, qmax 448, FP32
 * accumulation). One f32 scale per row instead of one E8M0 scale per 32
 * elements:
 *   s    = f32(max_k |x[r][k]|) / 448        (f32 division, nearest even)
 *   code = E4M3(f32(x[r][k]) / s)            (f32 division, then nearest even,
 *                                             saturating at +-448, sign of
 *                                             zero kept)
 *   s == 0: every code a signed zero. A row holding NaN or Inf: s = NaN and
 *   every code 0x7F.
 * Codes use the slab layout above ([K/64][R][64], R = mx_slab_rows(rows),
 * pad rows zero); scales are f32 [R] (pad rows 0).
 * ------------------------------------------------------------------------ */

/* Dynamic per-token quantization of bf16 x [M][ldx] (ldx >= K, ldx % 8 == 0,
 * K % 64 == 0): q uint8 [K/64][RM][64], s f32 [RM]. Codes 16-byte aligned,
 * scales 4-byte aligned; outputs must not overlap x or each other. */
int mx_pc_quantize_act_slab(const void* x, int64_t M, int64_t K, int64_t ldx,
                            uint8_t* q, float* s, void* stream);

/* Per-output-channel quantization of weights w [N][ldw] of type wdtype
 * (MX_DT_F32 or MX_DT_BF16; ldw * sizeof(element) % 16 == 0): q uint8
 * [K/64][RN][64], s f32 [RN].
 * Passage: "Wan2.2 I2V A14B, four-step 720p: native LightX2V FP8 and NVFP4",
 * section "Conversion and compatibility". */
int mx_pc_quantize_weight_slab(const void* w, int wdtype, int64_t N, int64_t K, int64_t ldw,
                               uint8_t* q, float* s, void* stream);

/* The per-channel FP8 linear:
 *   y[m][n] = bf16_rne( epi( xs[m] * ws[n] * sum_k dec(xq[m][k]) dec(wq[n][k])
 *                            + f32(bias[n]) ) )
 * with products exact and sums in f32 (the block-scaled MFMAs of the MX path
 * with unit scales; the row scales are applied to the f32 sums). Operands in
 * the layout above; bias f16 [N] or NULL; y bf16 [M][N]. K % 64 == 0, N % 16
 * == 0 (else MX_ERR_UNSUPPORTED); codes and y 16-byte aligned, scales 4-byte
 * aligned; y must not overlap an input.
 * Passage: "Wan2.2 I2V A14B, four-step 720p: native LightX2V FP8 and NVFP4",
 * section "Conversion and compatibility"; FP32 accumulation as in "Model
 * Quantization Techniques", mode table. */
int mx_pc_linear_slab(const uint8_t* xq, const float* xs, int64_t M, int64_t K,
                      const uint8_t* wq, const float* ws, int64_t N,
                      const void* bias, int epilogue, void* y, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MX_H */
