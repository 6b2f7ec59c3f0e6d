/*
 * qlora.h -- C ABI of the MI355X (gfx950) QLoRA hot-path library (libqlora.so).
 *
 * What the library computes (sources: web pages on QLoRA, cited by page and
 * section):
 *   - nlp-lineage milestone page on QLoRA (2023), section "The idea": the NF4
 *     bullet (16 levels placed at equal shares of a normal distribution, with
 *     an exact zero), the double-quantisation bullet (blocks of 64 with a
 *     32-bit scale each, those scales quantised again to 8 bits), and the
 *     notation paragraph (Y = X doubleDequant(c1, c2, W_NF4) + X L1 L2, bf16
 *     adapters, only L1 and L2 receive gradients).
 *   - inferensys glossary entry "QLoRA": the double-quantization paragraph
 *     (the scales become 8-bit floats) and the frozen-base paragraph (gradients
 *     pass through the 4-bit weights but only the adapters are updated).
 *   - examadda page "QLoRA (Quantized LoRA)", "The Core Idea" (the base is
 *     quantised once and dequantised on the fly) and "Practical Notes" (bf16
 *     compute).
 *
 * Conventions shared by every entry point
 *   - Tensor pointers are DEVICE pointers, allocated and owned by the caller.
 *     The library never allocates, frees or synchronises, and keeps no mutable
 *     global state; all work is enqueued on `stream` (a hipStream_t passed as
 *     void*, NULL = the null stream) and completes asynchronously.
 *   - bf16 tensors are passed as uint16_t bit patterns. All matrices are dense
 *     row-major with no padding.
 *   - The weight is stored out x in: W[N, K] row-major. First-level blocks are
 *     64 consecutive elements of the flat matrix (so they run along K and K
 *     must be a multiple of 64). Codes are packed two per byte, the element
 *     with the even flat index in the low nibble. Code k means NF4 level k in
 *     ascending order (code 7 is 0.0, code 0 is -1.0, code 15 is +1.0).
 *   - Second level: groups of 256 consecutive first-level scales; c2 holds one
 *     OCP FP8 E4M3FN byte per block, c1 one fp32 per group (the last group may
 *     be partial).
 *   - Device pointers must be 16-byte aligned.
 *   - Return value: QL_OK (0) or a negative ql_status. Arguments are checked on
 *     the host before anything is enqueued: for every status except
 *     QL_ERR_HIP nothing has been enqueued and no output is written. QL_ERR_HIP
 *     means a kernel launch was refused; launches of the same call that came
 *     before it may already be enqueued, and the outputs are unspecified.
 *     Device faults are asynchronous and surface at the caller's next
 *     synchronisation. No C++ exception crosses this interface.
 *   - Inputs must be finite; for non-finite weights the outputs are
 *     unspecified.
 */
#ifndef QLORA_H
#define QLORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QL_OK = 0,
  QL_ERR_NULL = -1,      /* a required pointer is NULL                            */
  QL_ERR_SHAPE = -2,     /* a size <= 0, K % 64 != 0, r outside [1, 64], a matrix
                            of the layer calls at 2^31 bytes or more, ...       */
  QL_ERR_DTYPE = -3,     /* unsupported dtype, code book or scale code            */
  QL_ERR_ALIGN = -4,     /* a device pointer is not 16-byte aligned               */
  QL_ERR_WORKSPACE = -5, /* workspace NULL or smaller than the query returns      */
  QL_ERR_HIP = -6,       /* a HIP launch failed (see ql_status_string)            */
  QL_ERR_VALUE = -7      /* a hyper-parameter outside its range                   */
} ql_status;

enum { QL_F32 = 0, QL_BF16 = 1 };

/* 4-bit code books of the q4_* calls (QL_CB_NF4 is the layer's format). */
enum { QL_CB_NF4 = 0, QL_CB_FP4 = 1, QL_CB_INT4 = 2 };
/* Block-scale codes of the q4_* calls: QL_SC_GROUPMAX is nf4_double_quant's. */
enum { QL_SC_GROUPMAX = 0, QL_SC_FULLRANGE = 1, QL_SC_MEAN = 2, QL_SC_ABSMAX = 3 };

/* First quantisation level (nlp-lineage page, "The idea", NF4 and
 * double-quantisation bullets).
 * W [rows, cols] (fp32 or bf16 per w_dtype), cols % 64 == 0.
 * For every block b of 64 consecutive elements: absmax[b] = max |w| (exact, fp32);
 * every element is normalised n = fl32(w / absmax[b]) (correctly rounded fp32
 * division; an all-zero block gives n = 0) and replaced by the code of the
 * nearest NF4 level (an exact tie between two levels takes the smaller code).
 * Outputs: codes [rows * cols / 2] bytes, absmax [rows * cols / 64] fp32.      */
int nf4_quantize(const void* W, int w_dtype, int64_t rows, int64_t cols,
                 uint8_t* codes, float* absmax, void* stream);

/* Second quantisation level ("double quantization": inferensys glossary,
 * double-quantization paragraph; nlp-lineage page, double-quantisation bullet).
 * absmax [n_blocks] fp32 >= 0. For every group g of 256 consecutive scales:
 * c1[g] = max of the group; c2[b] = E4M3FN code of fl32(absmax[b] / c1[g]),
 * rounded to nearest, ties to even (0 when c1[g] == 0).
 * Outputs: c2 [n_blocks] bytes, c1 [ceil(n_blocks / 256)] fp32.                 */
int nf4_double_quant(const float* absmax, int64_t n_blocks,
                     uint8_t* c2, float* c1, void* stream);

/* nf4_quantize followed by nf4_double_quant in one pass over W (same
 * passages): codes [rows, cols/2], c2 [n_blocks], c1 [ceil(n_blocks / 256)],
 * bit-identical to the two calls; absmax [n_blocks] is written too when
 * non-NULL. Errors as nf4_quantize.                                             */
int nf4_quantize_dq(const void* W, int w_dtype, int64_t rows, int64_t cols,
                    uint8_t* codes, float* absmax, uint8_t* c2, float* c1, void* stream);

/* doubleDequant(c1, c2, W_NF4) written out as bf16 (nlp-lineage page, notation
 * paragraph): s'_b = fl32(dec(c2[b]) * c1[b / 256]); W'[e] = bf16(fl32(q[code_e] * s'_b)),
 * both roundings to nearest-even. Output W_bf16 [rows, cols]. This is the exact
 * weight that the linear-layer entry points multiply with; it is provided for
 * checking, merging and debugging (the layer kernels never store it).          */
int nf4_dequantize(const uint8_t* codes, const uint8_t* c2, const float* c1,
                   int64_t rows, int64_t cols, uint16_t* W_bf16, void* stream);

/* Workspace (bytes) that qlora_linear_fwd needs for these sizes.               */
size_t qlora_linear_fwd_workspace(int64_t M, int64_t K, int64_t N, int r);

/* Forward of one quantised LoRA linear (nlp-lineage page, notation paragraph):
 *   T = bf16(X L1),  Y = bf16(X W'^T + lora_scale * (T L2)),
 * fp32 accumulation, W' as in nf4_dequantize (never materialised).
 * X [M, K] bf16; codes/c2/c1 describe W [N, K]; L1 [K, r] bf16; L2 [r, N] bf16;
 * 1 <= r <= 64, K % 64 == 0; X (2 M K bytes), Y (2 M N bytes) and the codes
 * (N K / 2 bytes) must each stay below 2^31 bytes (split larger batches).
 * Outputs: Y [M, N] bf16; T_out [M, r] bf16 when non-NULL (keep it
 * for the backward). workspace: ws_bytes >= qlora_linear_fwd_workspace(...),
 * contents need no initialisation and are clobbered; calls that overlap in
 * time must not share a workspace.
 * Decode sizes with small X (M <= 16, 2 M K <= 32 KB, r % 4 == 0) run as ONE
 * kernel launch that also forms T: its first work groups compute T's slices
 * and publish them behind flags and T records tagged with a per-call epoch,
 * which the other work groups wait for (bounded; past the bound a wave forms
 * them itself, with the same bits). Under stream capture the call issues the
 * two-launch form instead (T's slices, then the decode kernel), because a
 * replayed graph would repeat the epoch; both forms give the same bits. The
 * environment variable QLORA_DECODE_T_SPINS, read at each call, sets the
 * bound in polls (default 4096; 0 makes waves take their own path whenever
 * the slices are not yet there, for testing).                                  */
int qlora_linear_fwd(const uint16_t* X, int64_t M, int64_t K, int64_t N,
                     const uint8_t* codes, const uint8_t* c2, const float* c1,
                     const uint16_t* L1, const uint16_t* L2, int r, float lora_scale,
                     uint16_t* Y, uint16_t* T_out,
                     void* workspace, size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 * qlora_linear_fwd without a workspace argument: same formulas, kernels and
 * results, bit for bit. Its scratch is a file-scope device array of
 * QL_NOALLOC_SCRATCH_BYTES per GPU (allocated by the HIP runtime when the
 * library's code is loaded on that GPU and held until the process ends); the
 * first call on each GPU looks up that array's address (hipGetSymbolAddress,
 * with that GPU current), so a caller that captures graphs makes one call
 * outside capture first. The call itself allocates nothing. Every call on a
 * GPU shares that GPU's array: calls that overlap in time on one GPU (on
 * different streams, or from several threads) race and give unspecified
 * results. The array needs no clearing: each call writes every scratch
 * element it reads. `stream` must belong to the current GPU.
 * Errors as qlora_linear_fwd, plus QL_ERR_WORKSPACE when
 * qlora_linear_fwd_workspace(M, K, N, r) exceeds QL_NOALLOC_SCRATCH_BYTES
 * (checked before anything is enqueued).                                       */
#define QL_NOALLOC_SCRATCH_BYTES 16777216u
int qlora_linear_fwd_noalloc(const uint16_t* X, int64_t M, int64_t K, int64_t N,
                             const uint8_t* codes, const uint8_t* c2, const float* c1,
                             const uint16_t* L1, const uint16_t* L2, int r, float lora_scale,
                             uint16_t* Y, uint16_t* T_out, void* stream);

/* Workspace (bytes) that qlora_linear_bwd needs for these sizes.               */
size_t qlora_linear_bwd_workspace(int64_t M, int64_t K, int64_t N, int r);

/* Backward of one quantised LoRA linear. The frozen 4-bit base receives no
 * gradient: there is no dW argument (nlp-lineage page, notation paragraph;
 * inferensys glossary, frozen-base paragraph; examadda page, "The Flow").
 *   G   = bf16(lora_scale * dY L2^T)          [M, r]
 *   dX  = bf16(dY W' + G L1^T)                [M, K]   (skipped when dX == NULL)
 *   dL1 = fp32(X^T G)                         [K, r]
 *   dL2 = fp32(lora_scale * T^T dY)           [r, N]
 * T [M, r] bf16 is the forward's T_out; when NULL it is recomputed from X and L1
 * (gradient-checkpointing style). dY [M, N] bf16. Shapes and workspace as in
 * the forward; ws_bytes >= qlora_linear_bwd_workspace(...).
 * Streams: when the dX product's tiles (256 x 256) leave the last round of its
 * persistent grid partly empty, dL1 and dL2 are computed on a second stream
 * that the library creates once per calling thread and device (default
 * priority, never destroyed), forked from `stream` after G and joined back into
 * it before the call returns, also when it fails with QL_ERR_HIP. Work the
 * caller enqueues on `stream` afterwards is ordered after all of the call's
 * work, as on one stream, and the results are bit-identical to the one-stream
 * order. Calls from one thread share that second stream, so their dL1 / dL2
 * products run in call order even when the callers' streams differ.           */
int qlora_linear_bwd(const uint16_t* X, const uint16_t* dY, int64_t M, int64_t K, int64_t N,
                     const uint8_t* codes, const uint8_t* c2, const float* c1,
                     const uint16_t* L1, const uint16_t* L2, int r, float lora_scale,
                     const uint16_t* T, uint16_t* dX, float* dL1, float* dL2,
                     void* workspace, size_t ws_bytes, void* stream);

/* Stage entry points: the single fused kernels of the layer, for callers that
 * keep the LoRA intermediates themselves (activation checkpointing, graph
 * capture of individual stages, per-kernel timing). Same formulas, layouts,
 * rounding points and size limits as the calls above.
 *
 * qlora_lora_down: T = bf16(X L1) [M, r] (nlp-lineage page, notation paragraph,
 * the X L1 factor of the adapter path). ws_bytes >= qlora_lora_down_workspace().  */
size_t qlora_lora_down_workspace(int64_t M, int64_t K, int r);
int qlora_lora_down(const uint16_t* X, int64_t M, int64_t K, const uint16_t* L1, int r,
                    uint16_t* T, void* workspace, size_t ws_bytes, void* stream);

/* qlora_linear_fwd_t: Y = bf16(X W'^T + lora_scale * (T L2)) given T; one kernel,
 * no workspace (same paragraph; W' rebuilt on the fly as in qlora_linear_fwd).  */
int qlora_linear_fwd_t(const uint16_t* X, int64_t M, int64_t K, int64_t N,
                       const uint8_t* codes, const uint8_t* c2, const float* c1,
                       const uint16_t* T, const uint16_t* L2, int r, float lora_scale,
                       uint16_t* Y, void* stream);

/* qlora_lora_grad_in: G = bf16(lora_scale * dY L2^T) [M, r], the gradient that
 * reaches the adapter's inner activation (inferensys glossary, frozen-base
 * paragraph: gradients flow through to the adapters).
 * ws_bytes >= qlora_lora_grad_in_workspace().                                    */
size_t qlora_lora_grad_in_workspace(int64_t M, int64_t N, int r);
int qlora_lora_grad_in(const uint16_t* dY, int64_t M, int64_t N, const uint16_t* L2, int r,
                       float lora_scale, uint16_t* G, void* workspace, size_t ws_bytes, void* stream);

/* qlora_linear_dx: dX = bf16(dY W' + G L1^T) given G; one kernel, no workspace
 * (the transposed-weight path through the frozen base: examadda page,
 * "The Flow"; nlp-lineage page, "The idea", mechanism paragraph).               */
int qlora_linear_dx(const uint16_t* dY, int64_t M, int64_t K, int64_t N,
                    const uint8_t* codes, const uint8_t* c2, const float* c1,
                    const uint16_t* G, const uint16_t* L1, int r, uint16_t* dX, void* stream);

/* Adapter merge for export (examadda page, "Practical Notes": to merge, the
 * base is dequantised first and the adapter product is added to it):
 *   W_m = bf16(W' + lora_scale * (L1 L2)^T)                [N, K]
 * W' as in nf4_dequantize; (L1 L2)^T in fp32 accumulation, added to W' in fp32
 * and rounded once to bf16 (nearest-even). codes/c2/c1 describe W [N, K];
 * L1 [K, r] bf16; L2 [r, N] bf16; 1 <= r <= 64; K % 64 == 0; N * K <= 2^36.
 * Output W_out [N, K] bf16, owned by the caller, must not overlap the inputs.
 * With L1 or L2 all zero the result equals nf4_dequantize's in value (a zero
 * may change sign). The merged weight is bf16: re-quantising it to NF4 is
 * lossy and is left to the caller (nf4_quantize). Errors: QL_ERR_NULL,
 * QL_ERR_SHAPE, QL_ERR_ALIGN before anything is enqueued; QL_ERR_HIP.          */
int qlora_merge(const uint8_t* codes, const uint8_t* c2, const float* c1, int64_t N, int64_t K,
                const uint16_t* L1, const uint16_t* L2, int r, float lora_scale,
                uint16_t* W_out, void* stream);

/* Stacked linears that read the same input (q|k|v, gate|up of a Transformer
 * block; adapters go on every linear: nlp-lineage page, "The idea"). W [G N, K]
 * is G matrices of N rows stacked along the output dimension and quantized as
 * one (codes/c2/c1 as nf4_quantize/nf4_double_quant of the stack; when each
 * matrix's N K / 64 blocks are a multiple of 256 this is bit-identical to the
 * G separate quantizations). Segment g has its own adapter: L1 holds G
 * consecutive [K, r] blocks, L2 G consecutive [r, N] blocks.
 *   qlora_group_fwd: Y [M, G N] = [Y_0 | ... | Y_{G-1}], Y_g exactly as
 *     qlora_linear_fwd of segment g; T_out (G consecutive [M, r]) optional.
 *   qlora_group_bwd: dY [M, G N]; per segment G_g, dL1_g [K, r], dL2_g [r, N]
 *     exactly as qlora_linear_bwd of segment g (dL1, dL2: G consecutive blocks);
 *     dX = bf16(sum_g (dY_g W'_g + G_g L1_g^T)), one rounding (NULL: skipped).
 *     The per-segment dL1 / dL2 products may run on the second stream
 *     described at qlora_linear_bwd, under the same rule and guarantees.
 * Requirements beyond qlora_linear_*: 1 <= G <= 16; for G > 1, N % 256 == 0 and
 * M > 16, except that qlora_group_fwd also takes decode sizes, 1 <= M <= 16,
 * when X fits the decode kernel's LDS (M K <= 16384) and r % 4 == 0: then every
 * segment's T and the whole stacked output come from two launches (Y_g and T
 * bit-identical to qlora_linear_fwd of segment g). QL_ERR_SHAPE otherwise.
 * Workspace from the _workspace queries.                                        */
size_t qlora_group_fwd_workspace(int64_t M, int64_t K, int64_t N, int G, int r);
int qlora_group_fwd(const uint16_t* X, int64_t M, int64_t K, int64_t N, int G,
                    const uint8_t* codes, const uint8_t* c2, const float* c1,
                    const uint16_t* L1, const uint16_t* L2, int r, float lora_scale,
                    uint16_t* Y, uint16_t* T_out, void* workspace, size_t ws_bytes, void* stream);
size_t qlora_group_bwd_workspace(int64_t M, int64_t K, int64_t N, int G, int r);
int qlora_group_bwd(const uint16_t* X, const uint16_t* dY, int64_t M, int64_t K, int64_t N, int G,
                    const uint8_t* codes, const uint8_t* c2, const float* c1,
                    const uint16_t* L1, const uint16_t* L2, int r, float lora_scale,
                    const uint16_t* T, uint16_t* dX, float* dL1, float* dL2,
                    void* workspace, size_t ws_bytes, void* stream);

/* Adapter-only optimizer step (inferensys glossary, frozen-base paragraph: the
 * optimizer keeps momentum and variance for the adapters only). AdamW with
 * decoupled weight decay over n fp32 values (typically every adapter of a
 * block, laid out in one flat array so that one call updates them all):
 *   theta <- theta (1 - lr wd);  m <- b1 m + (1 - b1) g;  v <- b2 v + (1 - b2) g^2;
 *   theta <- theta - lr/(1 - b1^step) * m / (sqrt(v)/sqrt(1 - b2^step) + eps)
 * param, exp_avg, exp_avg_sq updated in place (fp32); grad fp32 (as
 * qlora_linear_bwd writes dL1/dL2); param_bf16 (optional) receives bf16(theta),
 * the copy the layers read. step >= 1 counts calls from 1. QL_ERR_VALUE unless
 * lr >= 0, 0 <= beta1, beta2 < 1, eps > 0, weight_decay >= 0.                  */
int qlora_adamw_step(float* param, float* exp_avg, float* exp_avg_sq, const float* grad,
                     uint16_t* param_bf16, int64_t n, float lr, float beta1, float beta2, float eps,
                     float weight_decay, int64_t step, void* stream);

/* The 4-bit baselines the pages rank NF4 against (nlp-lineage page, "What it
 * showed": NF4 with double quantization against a standard 4-bit float and
 * 4-bit integers; inferensys glossary, NF4 paragraph), run through the same
 * blockwise-absmax encoder and table dequantizer, and two further ways to
 * code the block scales. Code books (16 fp32 levels, ascending; code 7 is 0):
 *   QL_CB_NF4   the layer's NF4 table,
 *   QL_CB_FP4   OCP E2M1 values / 6 (the block absmax maps to the largest, 6),
 *   QL_CB_INT4  k / 7 for k = -7..7;
 * FP4 and INT4 have 15 distinct values and code 15 repeats +1 (never produced:
 * ties go to the smaller code).
 *
 * q4_quantize: as nf4_quantize with the chosen table: absmax a per 64, n =
 * fl32(w / a) correctly rounded (0 for an all-zero block), code = nearest
 * level. Same layouts and errors as nf4_quantize; QL_ERR_DTYPE for an unknown
 * code book.                                                                    */
int q4_quantize(const void* W, int w_dtype, int64_t rows, int64_t cols, int codebook,
                uint8_t* codes, float* absmax, void* stream);

/* q4_double_quant: block scales absmax [n_blocks] to one E4M3FN byte each plus
 * per-group fp32 values (groups of 256, the last may be partial):
 *   QL_SC_GROUPMAX   exactly nf4_double_quant (mu unused, may be NULL);
 *   QL_SC_FULLRANGE  c1 = fl32(max / 448), c2 = E4M3FN(fl32(a / c1)) (0 if c1 = 0);
 *   QL_SC_MEAN       mu = fl32(S / count), S the fp32 sum over the zero-padded
 *                    group taken pairwise (i with i + h, h = 128, 64, ..., 1);
 *                    d = fl32(a - mu); c1 = fl32(max |d| / 448);
 *                    c2 = signed E4M3FN of fl32(d / c1) (0 if c1 = 0).
 * Outputs c2 [n_blocks], c1 [groups], mu [groups] (QL_SC_MEAN only; required).  */
int q4_double_quant(const float* absmax, int64_t n_blocks, int scale_code,
                    uint8_t* c2, float* c1, float* mu, void* stream);

/* q4_dequantize: W'[e] = bf16(fl32(q[code_e] * s_b)) for the chosen table, with
 *   QL_SC_ABSMAX               s_b = absmax[b] (c2, c1, mu unused);
 *   QL_SC_GROUPMAX, _FULLRANGE s_b = fl32(dec(c2[b]) * c1[b / 256]);
 *   QL_SC_MEAN                 s_b = fl32(mu[b / 256] + fl32(dec(c2[b]) * c1[b / 256])).
 * With QL_CB_NF4 and QL_SC_GROUPMAX this is nf4_dequantize.                    */
int q4_dequantize(const uint8_t* codes, int64_t rows, int64_t cols, int codebook, int scale_code,
                  const float* absmax, const uint8_t* c2, const float* c1, const float* mu,
                  uint16_t* W_bf16, void* stream);

/* Host helper: the 16 levels of a code book, copied to out16 (QL_ERR_DTYPE for
 * an unknown id).                                                               */
int q4_levels(int codebook, float* out16);

/* LoRA over a bf16 base: the same layer with a 16-bit frozen weight W [N, K]
 * (bf16, row-major, out x in) in place of the 4-bit one, computed by the same
 * GEMM kernels with the dequantisation replaced by plain bf16 tile loads. This
 * is the baseline the pages compare QLoRA with (examadda page, "The Trade-off:
 * Speed": QLoRA trains more slowly than LoRA because the 4-bit weights are
 * dequantised on every pass; inferensys glossary, paragraph on the
 * dequantising kernel: the overhead is small where the product is
 * compute-bound), and with W = nf4_dequantize(...) it is the
 * dequantise-then-multiply strategy.
 *   lora_linear_fwd:   T = bf16(X L1), Y = bf16(X W^T + lora_scale T L2)
 *   lora_linear_bwd:   G = bf16(lora_scale dY L2^T), dX = bf16(dY W + G L1^T)
 *                      (NULL: skipped), dL1 = fp32(X^T G), dL2 = fp32(lora_scale T^T dY);
 *                      W gets no gradient.
 *   lora_linear_fwd_t: Y given T (one kernel);  lora_linear_dx: dX given G (one kernel).
 * Shapes, layouts, alignment and errors as qlora_linear_*, with W replacing
 * codes/c2/c1; workspaces as qlora_linear_fwd_workspace / _bwd_workspace; also
 * QL_ERR_SHAPE unless N % 8 == 0 (rows of dY and W are read in 16-byte pieces),
 * or when W (2 N K bytes) or an activation matrix reaches 2^31 bytes.          */
int lora_linear_fwd(const uint16_t* X, int64_t M, int64_t K, int64_t N, const uint16_t* W,
                    const uint16_t* L1, const uint16_t* L2, int r, float lora_scale,
                    uint16_t* Y, uint16_t* T_out, void* workspace, size_t ws_bytes, void* stream);
int lora_linear_bwd(const uint16_t* X, const uint16_t* dY, int64_t M, int64_t K, int64_t N,
                    const uint16_t* W, const uint16_t* L1, const uint16_t* L2, int r, float lora_scale,
                    const uint16_t* T, uint16_t* dX, float* dL1, float* dL2,
                    void* workspace, size_t ws_bytes, void* stream);
int lora_linear_fwd_t(const uint16_t* X, int64_t M, int64_t K, int64_t N, const uint16_t* W,
                      const uint16_t* T, const uint16_t* L2, int r, float lora_scale,
                      uint16_t* Y, void* stream);
int lora_linear_dx(const uint16_t* dY, int64_t M, int64_t K, int64_t N, const uint16_t* W,
                   const uint16_t* G, const uint16_t* L1, int r, uint16_t* dX, void* stream);

/* Host-only helpers (no GPU needed). */
/* The 16 NF4 levels (fp32, ascending) that the kernels use, copied to out[16].  */
int qlora_nf4_levels(float* out16);
/* Static description of a status code (and of the last HIP error on this
 * thread for QL_ERR_HIP).                                                       */
const char* ql_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_H */
