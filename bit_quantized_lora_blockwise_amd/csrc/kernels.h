// Internal launcher interface between the C ABI (abi.cpp) and the kernels.
// Every launcher enqueues on `s` and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.h"

// Keeps a HIP error for ql_status_string and returns QL_ERR_HIP (abi.cpp).
int ql_record_hip_error(hipError_t e);

const Nf4Params& nf4_params();
const Nf4Buckets& nf4_buckets();
// Level table of a 4-bit code book: 0 NF4, 1 4-bit float (E2M1 / 6), 2 4-bit
// integer (k / 7); nullptr for any other id.
const Nf4Params* codebook_params(int codebook);

// --- encoder (encode.hip) ---------------------------------------------------
hipError_t launch_nf4_encode(const void* W, bool bf16, int64_t elems, uint8_t* codes, float* absmax,
                             hipStream_t s);
hipError_t launch_double_quant(const float* absmax, int64_t n_blocks, uint8_t* c2, float* c1, hipStream_t s);
// Both in one pass (absmax optional: may be null).
hipError_t launch_nf4_encode_dq(const void* W, bool bf16, int64_t elems, uint8_t* codes, float* absmax, uint8_t* c2,
                                float* c1, hipStream_t s);
hipError_t launch_dequant(const uint8_t* codes, const uint8_t* c2, const float* c1, int64_t elems,
                          uint16_t* out, hipStream_t s);

// --- code-book and scale-code variants (variants.hip) ------------------------
// Blockwise absmax encoder with level table p (exact division, threshold count).
hipError_t launch_q4_encode(const void* W, bool bf16, int64_t elems, const Nf4Params& p, uint8_t* codes,
                            float* absmax, hipStream_t s);
// Second-level codes over the full E4M3FN range; mean = true codes the signed
// differences from the group mean (mu[g] written), else the scales themselves.
hipError_t launch_double_quant_full(const float* absmax, int64_t n_blocks, bool mean, uint8_t* c2, float* c1,
                                    float* mu, hipStream_t s);
// Table dequantizer; mode 0: s = dec(c2) c1, 1: s = absmax, 2: s = mu + dec(c2) c1.
hipError_t launch_q4_dequant(const uint8_t* codes, int mode, const float* absmax, const uint8_t* c2,
                             const float* c1, const float* mu, int64_t elems, const Nf4Params& p, uint16_t* out,
                             hipStream_t s);

// --- skinny LoRA products (lora.hip) -----------------------------------------
// Split plan of a reduction of length R over tiles of `tiles` outputs.
struct SplitPlan {
  int splits;      // number of reduction slices
  int64_t chunk;   // reduction length per slice (multiple of 64)
};
SplitPlan plan_rowsplit(int64_t tiles, int64_t R);

// C[M, r] = A[M, R] * B, A with row stride lda, B(k, c) = L1[k][c] (b_is_kr =
// true, L1 is [R, r]) or B(k, c) = L2[c][k] (false, L2 is [r, R]).  Result
// scaled by `scale`, rounded to bf16 into out[M, r].  ws holds the fp32 partials.
size_t lora_skinny_ws(int64_t M, int64_t R, int r);
// Decode-sized T = X L1 (M <= 16, X rows 16-byte aligned, K % 64 == 0): fp32
// partial sums part[s][m][c] over S = decode_t_slices(K) <= kDecodeTSlices
// slices of the reduction.  launch_lora_skinny adds them in order s = 0..S-1 for
// such shapes, and so does the decode kernel, so T is the same on every path.
// G > 1: stacked adapters L1_g [K, r] at L1 + g K r, slices of segment g at
// part + g S M r (one launch for all).
constexpr int kDecodeTSlices = 8;
int decode_t_slices(int64_t K);
int64_t decode_t_rows(int64_t K);   // rows of K per slice (a multiple of 32)
bool decode_t_ok(int64_t M, int64_t K, const void* X, const void* L1);
hipError_t launch_lora_part(const uint16_t* X, int64_t M, int64_t K, const uint16_t* L1, int r, float* part,
                            hipStream_t s, int G = 1);
hipError_t launch_lora_skinny(const uint16_t* A, int64_t M, int64_t R, int64_t lda, const uint16_t* B, bool b_is_kr,
                              int r, float scale, uint16_t* out, float* ws, hipStream_t s);

// C[p, c] = scale * sum_m A[m][p] * B[m][c] with A [M, P] (row stride lda),
// B [M, r]; stored as out[P, r] (transpose_out = false) or out[r, P] (true), fp32.
size_t lora_tn_ws(int64_t M, int64_t P, int r);
// Two such products in one launch (and their sums in one more): the first
// stored out0[P0, r], the second transposed out1_t[r, P1]; the workspace holds
// both products' partials (lora_tn_pair_ws).
size_t lora_tn_pair_ws(int64_t M, int64_t P0, int64_t P1, int r);
hipError_t launch_lora_tn_pair(const uint16_t* A0, int64_t lda0, const uint16_t* B0, int64_t P0, float scale0,
                               float* out0, const uint16_t* A1, int64_t lda1, const uint16_t* B1, int64_t P1,
                               float scale1, float* out1_t, int64_t M, int r, float* ws, hipStream_t s);
hipError_t launch_lora_tn(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t M, int64_t P, int r,
                          float scale, bool transpose_out, float* out, float* ws, hipStream_t s);

// --- adapter merge (merge.hip) ---------------------------------------------
// W[n][k] = bf16(W'[n][k] + scale * sum_c L1[k][c] L2[c][n]), W' the bf16
// dequantised base; W [N, K], K a multiple of 64.
hipError_t launch_merge(const uint8_t* codes, const uint8_t* c2, const float* c1, int64_t N, int64_t K,
                        const uint16_t* L1, const uint16_t* L2, int r, float scale, uint16_t* W, hipStream_t s);

// --- adapter optimizer (adamw.hip) -------------------------------------------
// One AdamW step over n fp32 weights (decoupled decay), optional bf16 copy.
hipError_t launch_adamw(float* param, float* exp_avg, float* exp_avg_sq, const float* grad, uint16_t* param_bf16,
                        int64_t n, float lr, float beta1, float beta2, float eps, float weight_decay, int64_t step,
                        hipStream_t s);

// --- quantised GEMMs (gemm_big.hip, gemm.hip, decode.hip) ----------------------
// Y[M, N] = bf16(X W'^T + scale * T L2) for small M (M <= 16), streaming the
// packed weight once (training-sized M: launch_qgemm_big below).
hipError_t launch_qgemv_fwd(const uint16_t* X, int64_t M, int64_t K, int64_t N, const uint8_t* codes,
                            const uint8_t* c2, const float* c1, const uint16_t* T, const uint16_t* L2, int r,
                            float scale, uint16_t* Y, hipStream_t s);
// Same, with T = bf16(sum over s of Tpart[s]) formed by the kernel from the S
// fp32 slices of launch_lora_part (r % 4 == 0, Tpart 16-byte aligned); T_out
// (optional) receives that T.
// Stacked linears at decode size: G segments of N rows of one packed matrix
// [G N, K] sharing X, each with its own T (formed from the slices of
// launch_lora_part(..., G)) and L2_g [r, N] (at L2 + g r N); Y [M, G N].  Only
// for X that fits the kernel's LDS (M K <= 16384) and N % 16 == 0.
bool qgemv_group_ok(int64_t M, int64_t K, int64_t N, int G);
hipError_t launch_qgemv_group_tpart(const uint16_t* X, int64_t M, int64_t K, int64_t N, int G, const uint8_t* codes,
                                    const uint8_t* c2, const float* c1, const float* Tpart, int S, uint16_t* T_out,
                                    const uint16_t* L2, int r, float scale, uint16_t* Y, hipStream_t s);
hipError_t launch_qgemv_fwd_tpart(const uint16_t* X, int64_t M, int64_t K, int64_t N, const uint8_t* codes,
                                  const uint8_t* c2, const float* c1, const float* Tpart, int S, uint16_t* T_out,
                                  const uint16_t* L2, int r, float scale, uint16_t* Y, hipStream_t s);
// The same decode forward with T formed inside the one launch (no separate
// partial-sum launch): M * K * 2 <= 32 KB, r % 4 == 0, r <= 64.  part: S M r
// fp32 (16-byte aligned); sync: qgemv_fused_sync_bytes(M, r) bytes (16-byte
// aligned) of flags and T records, holding anything but data tagged with
// `epoch`, which must differ from every earlier call's epoch on the same memory
// (in its low 32 bits too, which must not be 0); spins bounds each wave's wait
// (past it the wave forms T's slices itself, same bits).
bool qgemv_fused_ok(int64_t M, int64_t K, int r);
size_t qgemv_fused_sync_bytes(int64_t M, int r);
hipError_t launch_qgemv_fwd_fused(const uint16_t* X, int64_t M, int64_t K, int64_t N, const uint8_t* codes,
                                  const uint8_t* c2, const float* c1, const uint16_t* L1, int r, float* part,
                                  void* sync, uint64_t epoch, uint32_t spins, uint16_t* T_out,
                                  const uint16_t* L2, float scale, uint16_t* Y, hipStream_t s);
// Large-tile (256 x 256) versions of both GEMMs: dx = false computes the forward
// (A = X, LA = T, LB = L2, C = Y), dx = true the dX product (A = dY, LA = G,
// LB = L1, C = dX).  qgemm_big_ok says whether the shapes qualify.  nseg > 1:
// W [N, K] is nseg matrices of N / nseg rows stacked (N / nseg a multiple of
// 256), each with its own adapter: LA holds nseg [M, r] blocks, LB nseg L2
// [r, N / nseg] (fwd) or L1 [K, r] (dX) blocks.
bool qgemm_big_ok(bool dx, int64_t M, int64_t K, int64_t N);
hipError_t launch_qgemm_big(bool dx, const uint16_t* A, int64_t M, int64_t K, int64_t N, const uint8_t* codes,
                            const uint8_t* c2, const float* c1, const uint16_t* LA, const uint16_t* LB, int r,
                            float scale, uint16_t* C, hipStream_t s, int nseg = 1);
// The same two GEMMs with a bf16 weight W [N, K] in place of the packed one
// (LoRA over a bf16 base): dx = false Y = bf16(X W^T + scale T L2), dx = true
// dX = bf16(dY W + G L1^T).  bgemm_ok says whether the shapes qualify.
bool bgemm_ok(bool dx, int64_t M, int64_t K, int64_t N);
hipError_t launch_bgemm_big(bool dx, const uint16_t* A, int64_t M, int64_t K, int64_t N, const uint16_t* W,
                            const uint16_t* LA, const uint16_t* LB, int r, float scale, uint16_t* C, hipStream_t s);
// dX[M, K] = bf16(dY W' + G L1^T)
hipError_t launch_qgemm_dx(const uint16_t* dY, int64_t M, int64_t K, int64_t N, const uint8_t* codes,
                           const uint8_t* c2, const float* c1, const uint16_t* G, const uint16_t* L1, int r,
                           uint16_t* dX, hipStream_t s);
