// C ABI of libqlora.so: argument checks, workspace sizing and kernel dispatch.
// Declarations and the contract of each entry point are in include/qlora.h.
#include <unistd.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cstdlib>
#include <cmath>
#include <cstdio>
#include <cstring>

#include "../../include/qlora.h"
#include "kernels.h"

namespace {

thread_local hipError_t g_last_hip = hipSuccess;
thread_local char g_msg[256];

constexpr size_t kAlign = 256;

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int hip_status(hipError_t e) {
  if (e == hipSuccess) return QL_OK;
  g_last_hip = e;
  return QL_ERR_HIP;
}

#define QL_TRY(expr)                       \
  do {                                     \
    hipError_t e_ = (expr);                \
    if (e_ != hipSuccess) return hip_status(e_); \
  } while (0)

// The kernels address activations and packed codes with 32-bit buffer offsets:
// X and dX (M K bf16), Y and dY (M N bf16) and W's codes (N K / 2 bytes) must
// each stay below 2^31 bytes; larger batches are split by the caller.
bool shapes_ok(int64_t M, int64_t K, int64_t N, int r) {
  constexpr int64_t kLim = int64_t(1) << 31;
  return M > 0 && K > 0 && N > 0 && (K % 64) == 0 && r >= 1 && r <= 64 && M < kLim && K < kLim && N < kLim &&
         M * K * 2 < kLim && M * N * 2 < kLim && N * (K / 2) < kLim;
}

// Workspace layout of the forward: [T (M x r bf16) when the caller gives no T_out][fp32 partials].
struct FwdWs {
  size_t t_bytes, part_bytes, flag_bytes, total;
};
FwdWs fwd_ws(int64_t M, int64_t K, int64_t N, int r) {
  (void)N;
  FwdWs w;
  w.t_bytes = round_up((size_t)M * r * 2);
  w.part_bytes = round_up(lora_skinny_ws(M, K, r));
  w.flag_bytes = qgemv_fused_ok(M, K, r) ? round_up(qgemv_fused_sync_bytes(M, r)) : 0;
  w.total = w.t_bytes + w.part_bytes + w.flag_bytes;
  return w;
}

// Epochs of the decode forward's flags and T records: never the same twice in a
// process (nor in their low 32 bits, never 0), and started at a value that no
// earlier process is likely to have left in reused memory.
uint64_t next_epoch() {
  static std::atomic<uint64_t> ctr{[] {
    const uint64_t t = (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count();
    return (t * 0x9E3779B97F4A7C15ull) ^ ((uint64_t)getpid() << 40) ^ (uint64_t)(uintptr_t)&ctr;
  }()};
  uint64_t e;
  do e = ctr.fetch_add(1, std::memory_order_relaxed);
  while ((uint32_t)e == 0);
  return e;
}

// Whether work issued to `s` is being captured into a graph (an error in the
// query counts as capturing: the caller then gets the path that is safe to replay).
bool capturing(hipStream_t s) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  return hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone;
}

// Polls of the decode forward's wait for its slices before a wave forms them
// itself.  QLORA_DECODE_T_SPINS overrides it (a test sets 0 to exercise the
// wave's own path).
uint32_t decode_spins() {
  const char* e = std::getenv("QLORA_DECODE_T_SPINS");
  if (e && *e) return (uint32_t)std::strtoul(e, nullptr, 10);
  return 1u << 12;
}

// Backward: [T (recomputed when NULL)][G (M x r bf16)][fp32 partials, reused by each step].
struct BwdWs {
  size_t t_bytes, g_bytes, part_bytes, total;
};
BwdWs bwd_ws(int64_t M, int64_t K, int64_t N, int r) {
  BwdWs w;
  w.t_bytes = round_up((size_t)M * r * 2);
  w.g_bytes = round_up((size_t)M * r * 2);
  size_t p = lora_skinny_ws(M, K, r);
  p = std::max(p, lora_skinny_ws(M, N, r));
  p = std::max(p, lora_tn_pair_ws(M, K, N, r));
  w.part_bytes = round_up(p);
  w.total = w.t_bytes + w.g_bytes + w.part_bytes;
  return w;
}

// Forward product for M > 16: the large-tile kernel, which takes every shape
// shapes_ok accepts (K % 64 == 0 makes its rows 16-byte aligned).
hipError_t run_fwd_gemm(const uint16_t* X, int64_t M, int64_t K, int64_t N, const uint8_t* codes, const uint8_t* c2,
                        const float* c1, const uint16_t* T, const uint16_t* L2, int r, float scale, uint16_t* Y,
                        hipStream_t s) {
  if (!qgemm_big_ok(false, M, K, N)) return hipErrorInvalidValue;
  return launch_qgemm_big(false, X, M, K, N, codes, c2, c1, T, L2, r, scale, Y, s);
}

hipError_t run_dx_gemm(const uint16_t* dY, int64_t M, int64_t K, int64_t N, const uint8_t* codes, const uint8_t* c2,
                       const float* c1, const uint16_t* G, const uint16_t* L1, int r, uint16_t* dX, hipStream_t s) {
  if (qgemm_big_ok(true, M, K, N))
    return launch_qgemm_big(true, dY, M, K, N, codes, c2, c1, G, L1, r, 1.0f, dX, s);
  return launch_qgemm_dx(dY, M, K, N, codes, c2, c1, G, L1, r, dX, s);
}

// ---- dL1 / dL2 beside the dX product -----------------------------------------
// The dX product's persistent grid takes its tiles in rounds of one work group
// per CU (the CU count rounded down to a multiple of 8).  When the tiles leave
// the last round partly empty, the CUs without a tile in it would idle while
// the others finish; the two TN products (dL1 = X^T G, dL2 = s T^T dY), which
// read nothing the dX product writes, then run on a second stream and take
// those CUs.  A dX tile occupies all of a CU's registers, so the TN work
// groups only start where a work group of the dX product has finished.  With
// whole rounds there is no idle round to fill and the products stay in order
// on the caller's stream.  The kernels, their work split and the order of
// every sum are the same on both paths, so the results are identical.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  int cus = 0;
  bool failed = false;
};

constexpr int kMaxDevices = 64;

// The calling thread's second stream on the current device (default priority,
// created on first use and kept until the process ends), or nullptr when it
// cannot be had; the caller then keeps everything on its own stream.
SideStream* side_stream() {
  thread_local SideStream per_dev[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  SideStream& d = per_dev[dev];
  if (d.failed) return nullptr;
  if (!d.s) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 8 ||
        hipEventCreateWithFlags(&d.fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&d.join, hipEventDisableTiming) != hipSuccess ||
        hipStreamCreateWithFlags(&d.s, hipStreamNonBlocking) != hipSuccess) {
      d.failed = true;
      d.s = nullptr;
      return nullptr;
    }
    d.cus = cus;
  }
  return &d;
}

// Joins the second stream back into the caller's stream s, also after a failed
// launch `e` on it, so that what was enqueued there stays ordered before s's
// later work; returns the first error.
hipError_t join_side(SideStream& d, hipStream_t s, hipError_t e) {
  hipError_t j = hipEventRecord(d.join, d.s);
  if (j == hipSuccess) j = hipStreamWaitEvent(s, d.join, 0);
  return e != hipSuccess ? e : j;
}

// True when the dX product [M, K] runs on the persistent grid and its last
// round of tiles (256 x 256 each) is partly empty.
bool dx_last_round_partial(const SideStream& d, int64_t M, int64_t K, int64_t NG) {
  if (!qgemm_big_ok(true, M, K, NG)) return false;
  const int64_t tiles = ((M + 255) / 256) * ((K + 255) / 256);
  const int64_t grid = d.cus / 8 * 8;
  return tiles > grid && tiles % grid != 0;
}

// ---- stacked linears -------------------------------------------------------
bool group_ok(int64_t M, int64_t K, int64_t N, int G, int r) {
  if (G < 1 || G > 16 || N <= 0 || N > (int64_t(1) << 31) / G) return false;
  if (!shapes_ok(M, K, N * G, r)) return false;
  if (G == 1) return true;
  return N % 256 == 0 && M > 16 && qgemm_big_ok(false, M, K, N * G) && qgemm_big_ok(true, M, K, N * G);
}

// Stacked forward at decode size (M <= 16, G > 1): one T-slice launch for all
// adapters and one decode launch over the stacked rows; X must fit the decode
// kernel's LDS (M K <= 16384) and r be a multiple of 4.
bool group_decode_ok(int64_t M, int64_t K, int64_t N, int G, int r) {
  return G > 1 && G <= 16 && M >= 1 && M <= 16 && N > 0 && N % 256 == 0 && N <= (int64_t(1) << 31) / G &&
         shapes_ok(M, K, N * G, r) && (r % 4) == 0 && qgemv_group_ok(M, K, N, G);
}

bool group_fwd_ok(int64_t M, int64_t K, int64_t N, int G, int r) {
  return group_ok(M, K, N, G, r) || group_decode_ok(M, K, N, G, r);
}

struct GroupWs {
  size_t t_bytes, g_bytes, part_bytes, total;
};
GroupWs group_ws(int64_t M, int64_t K, int64_t N, int G, int r) {
  GroupWs w;
  w.t_bytes = round_up((size_t)G * M * r * 2);
  w.g_bytes = round_up((size_t)G * M * r * 2);
  size_t p = lora_skinny_ws(M, K, r);
  p = std::max(p, lora_skinny_ws(M, N, r));
  p = std::max(p, lora_tn_pair_ws(M, K, N, r));
  w.part_bytes = round_up(p);
  w.total = w.t_bytes + w.g_bytes + w.part_bytes;
  return w;
}

}  // namespace

int ql_record_hip_error(hipError_t e) { return e == hipSuccess ? QL_OK : hip_status(e); }

extern "C" {

int nf4_quantize(const void* W, int w_dtype, int64_t rows, int64_t cols, uint8_t* codes, float* absmax,
                 void* stream) {
  if (!W || !codes || !absmax) return QL_ERR_NULL;
  if (w_dtype != QL_F32 && w_dtype != QL_BF16) return QL_ERR_DTYPE;
  if (rows <= 0 || cols <= 0 || cols % 64 != 0 || rows > (int64_t(1) << 40) / cols) return QL_ERR_SHAPE;
  if (!aligned16(W) || !aligned16(codes) || !aligned16(absmax)) return QL_ERR_ALIGN;
  QL_TRY(launch_nf4_encode(W, w_dtype == QL_BF16, rows * cols, codes, absmax, (hipStream_t)stream));
  return QL_OK;
}

int nf4_quantize_dq(const void* W, int w_dtype, int64_t rows, int64_t cols, uint8_t* codes, float* absmax,
                    uint8_t* c2, float* c1, void* stream) {
  if (!W || !codes || !c2 || !c1) return QL_ERR_NULL;
  if (w_dtype != QL_F32 && w_dtype != QL_BF16) return QL_ERR_DTYPE;
  if (rows <= 0 || cols <= 0 || cols % 64 != 0 || rows > (int64_t(1) << 40) / cols) return QL_ERR_SHAPE;
  if (!aligned16(W) || !aligned16(codes) || !aligned16(c2) || !aligned16(c1) || (absmax && !aligned16(absmax)))
    return QL_ERR_ALIGN;
  QL_TRY(launch_nf4_encode_dq(W, w_dtype == QL_BF16, rows * cols, codes, absmax, c2, c1, (hipStream_t)stream));
  return QL_OK;
}

int nf4_double_quant(const float* absmax, int64_t n_blocks, uint8_t* c2, float* c1, void* stream) {
  if (!absmax || !c2 || !c1) return QL_ERR_NULL;
  if (n_blocks <= 0 || n_blocks > (int64_t(1) << 36)) return QL_ERR_SHAPE;
  if (!aligned16(absmax) || !aligned16(c2) || !aligned16(c1)) return QL_ERR_ALIGN;
  QL_TRY(launch_double_quant(absmax, n_blocks, c2, c1, (hipStream_t)stream));
  return QL_OK;
}

int nf4_dequantize(const uint8_t* codes, const uint8_t* c2, const float* c1, int64_t rows, int64_t cols,
                   uint16_t* W_bf16, void* stream) {
  if (!codes || !c2 || !c1 || !W_bf16) return QL_ERR_NULL;
  if (rows <= 0 || cols <= 0 || cols % 64 != 0 || rows > (int64_t(1) << 40) / cols) return QL_ERR_SHAPE;
  if (!aligned16(codes) || !aligned16(c2) || !aligned16(c1) || !aligned16(W_bf16)) return QL_ERR_ALIGN;
  QL_TRY(launch_dequant(codes, c2, c1, rows * cols, W_bf16, (hipStream_t)stream));
  return QL_OK;
}

int qlora_merge(const uint8_t* codes, const uint8_t* c2, const float* c1, int64_t N, int64_t K, const uint16_t* L1,
                const uint16_t* L2, int r, float lora_scale, uint16_t* W_out, void* stream) {
  if (!codes || !c2 || !c1 || !L1 || !L2 || !W_out) return QL_ERR_NULL;
  if (N <= 0 || K <= 0 || K % 64 != 0 || r < 1 || r > 64 || N > (int64_t(1) << 31) || K > (int64_t(1) << 31) ||
      N > (int64_t(1) << 36) / K)
    return QL_ERR_SHAPE;
  if (!aligned16(codes) || !aligned16(c2) || !aligned16(c1) || !aligned16(L1) || !aligned16(L2) ||
      !aligned16(W_out))
    return QL_ERR_ALIGN;
  QL_TRY(launch_merge(codes, c2, c1, N, K, L1, L2, r, lora_scale, W_out, (hipStream_t)stream));
  return QL_OK;
}

int q4_quantize(const void* W, int w_dtype, int64_t rows, int64_t cols, int codebook, uint8_t* codes,
                float* absmax, void* stream) {
  if (!W || !codes || !absmax) return QL_ERR_NULL;
  const Nf4Params* p = codebook_params(codebook);
  if ((w_dtype != QL_F32 && w_dtype != QL_BF16) || !p) return QL_ERR_DTYPE;
  if (rows <= 0 || cols <= 0 || cols % 64 != 0 || rows > (int64_t(1) << 40) / cols) return QL_ERR_SHAPE;
  if (!aligned16(W) || !aligned16(codes) || !aligned16(absmax)) return QL_ERR_ALIGN;
  QL_TRY(launch_q4_encode(W, w_dtype == QL_BF16, rows * cols, *p, codes, absmax, (hipStream_t)stream));
  return QL_OK;
}

int q4_double_quant(const float* absmax, int64_t n_blocks, int scale_code, uint8_t* c2, float* c1, float* mu,
                    void* stream) {
  if (scale_code != QL_SC_GROUPMAX && scale_code != QL_SC_FULLRANGE && scale_code != QL_SC_MEAN)
    return QL_ERR_DTYPE;
  if (!absmax || !c2 || !c1 || (scale_code == QL_SC_MEAN && !mu)) return QL_ERR_NULL;
  if (n_blocks <= 0 || n_blocks > (int64_t(1) << 36)) return QL_ERR_SHAPE;
  if (!aligned16(absmax) || !aligned16(c2) || !aligned16(c1) || (scale_code == QL_SC_MEAN && !aligned16(mu)))
    return QL_ERR_ALIGN;
  if (scale_code == QL_SC_GROUPMAX) {
    QL_TRY(launch_double_quant(absmax, n_blocks, c2, c1, (hipStream_t)stream));
  } else {
    QL_TRY(launch_double_quant_full(absmax, n_blocks, scale_code == QL_SC_MEAN, c2, c1, mu, (hipStream_t)stream));
  }
  return QL_OK;
}

int q4_dequantize(const uint8_t* codes, int64_t rows, int64_t cols, int codebook, int scale_code,
                  const float* absmax, const uint8_t* c2, const float* c1, const float* mu, uint16_t* W_bf16,
                  void* stream) {
  const Nf4Params* p = codebook_params(codebook);
  if (!p || scale_code < QL_SC_GROUPMAX || scale_code > QL_SC_ABSMAX) return QL_ERR_DTYPE;
  const bool single = scale_code == QL_SC_ABSMAX, mean = scale_code == QL_SC_MEAN;
  if (!codes || !W_bf16 || (single && !absmax) || (!single && (!c2 || !c1)) || (mean && !mu)) return QL_ERR_NULL;
  if (rows <= 0 || cols <= 0 || cols % 64 != 0 || rows > (int64_t(1) << 40) / cols) return QL_ERR_SHAPE;
  if (!aligned16(codes) || !aligned16(W_bf16) || (single && !aligned16(absmax)) ||
      (!single && (!aligned16(c2) || !aligned16(c1))) || (mean && !aligned16(mu)))
    return QL_ERR_ALIGN;
  const int mode = single ? 1 : (mean ? 2 : 0);
  QL_TRY(launch_q4_dequant(codes, mode, absmax, c2, c1, mu, rows * cols, *p, W_bf16, (hipStream_t)stream));
  return QL_OK;
}

int q4_levels(int codebook, float* out16) {
  const Nf4Params* p = codebook_params(codebook);
  if (!p) return QL_ERR_DTYPE;
  if (!out16) return QL_ERR_NULL;
  std::memcpy(out16, p->q, 16 * sizeof(float));
  return QL_OK;
}


size_t group_fwd_ws(int64_t M, int64_t K, int64_t N, int G, int r) {
  const GroupWs w = group_ws(M, K, N, G, r);
  size_t part = w.part_bytes;
  if (group_decode_ok(M, K, N, G, r)) part = std::max(part, round_up((size_t)G * kDecodeTSlices * M * r * 4));
  return w.t_bytes + part;
}

size_t qlora_group_fwd_workspace(int64_t M, int64_t K, int64_t N, int G, int r) {
  if (!group_fwd_ok(M, K, N, G, r)) return 0;
  return group_fwd_ws(M, K, N, G, r);
}

int qlora_group_fwd(const uint16_t* X, int64_t M, int64_t K, int64_t N, int G, const uint8_t* codes,
                    const uint8_t* c2, const float* c1, const uint16_t* L1, const uint16_t* L2, int r,
                    float lora_scale, uint16_t* Y, uint16_t* T_out, void* workspace, size_t ws_bytes, void* stream) {
  if (!X || !codes || !c2 || !c1 || !L1 || !L2 || !Y) return QL_ERR_NULL;
  if (!group_fwd_ok(M, K, N, G, r)) return QL_ERR_SHAPE;
  if (!aligned16(X) || !aligned16(codes) || !aligned16(c2) || !aligned16(c1) || !aligned16(L1) ||
      !aligned16(L2) || !aligned16(Y) || (T_out && !aligned16(T_out)))
    return QL_ERR_ALIGN;
  if (G == 1)
    return qlora_linear_fwd(X, M, K, N, codes, c2, c1, L1, L2, r, lora_scale, Y, T_out, workspace, ws_bytes,
                            stream);
  const GroupWs w = group_ws(M, K, N, G, r);
  if (!workspace || ws_bytes < group_fwd_ws(M, K, N, G, r)) return QL_ERR_WORKSPACE;
  if (!aligned16(workspace)) return QL_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  uint16_t* T = T_out ? T_out : (uint16_t*)ws;
  float* part = (float*)(ws + w.t_bytes);
  if (M <= 16) {
    // decode size: the slices of every T_g in one launch, added and rounded in the decode kernel
    if (!decode_t_ok(M, K, X, L1)) return QL_ERR_ALIGN;
    QL_TRY(launch_lora_part(X, M, K, L1, r, part, s, G));
    QL_TRY(launch_qgemv_group_tpart(X, M, K, N, G, codes, c2, c1, part, decode_t_slices(K), T_out, L2, r,
                                    lora_scale, Y, s));
    return QL_OK;
  }
  for (int g = 0; g < G; ++g)
    QL_TRY(launch_lora_skinny(X, M, K, K, L1 + (int64_t)g * K * r, true, r, 1.0f, T + (int64_t)g * M * r, part, s));
  QL_TRY(launch_qgemm_big(false, X, M, K, N * G, codes, c2, c1, T, L2, r, lora_scale, Y, s, G));
  return QL_OK;
}

size_t qlora_group_bwd_workspace(int64_t M, int64_t K, int64_t N, int G, int r) {
  if (!group_ok(M, K, N, G, r)) return 0;
  return group_ws(M, K, N, G, r).total;
}

int qlora_group_bwd(const uint16_t* X, const uint16_t* dY, int64_t M, int64_t K, int64_t N, int G,
                    const uint8_t* codes, const uint8_t* c2, const float* c1, const uint16_t* L1, const uint16_t* L2,
                    int r, float lora_scale, const uint16_t* T, uint16_t* dX, float* dL1, float* dL2,
                    void* workspace, size_t ws_bytes, void* stream) {
  if (!X || !dY || !codes || !c2 || !c1 || !L1 || !L2 || !dL1 || !dL2) return QL_ERR_NULL;
  if (!group_ok(M, K, N, G, r)) return QL_ERR_SHAPE;
  if (!aligned16(X) || !aligned16(dY) || !aligned16(codes) || !aligned16(c2) || !aligned16(c1) ||
      !aligned16(L1) || !aligned16(L2) || !aligned16(dL1) || !aligned16(dL2) || (T && !aligned16(T)) ||
      (dX && !aligned16(dX)))
    return QL_ERR_ALIGN;
  if (G == 1)
    return qlora_linear_bwd(X, dY, M, K, N, codes, c2, c1, L1, L2, r, lora_scale, T, dX, dL1, dL2, workspace,
                            ws_bytes, stream);
  const GroupWs w = group_ws(M, K, N, G, r);
  if (!workspace || ws_bytes < w.total) return QL_ERR_WORKSPACE;
  if (!aligned16(workspace)) return QL_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  uint16_t* Tw = (uint16_t*)ws;
  uint16_t* Gm = (uint16_t*)(ws + w.t_bytes);
  float* part = (float*)(ws + w.t_bytes + w.g_bytes);
  const int64_t ldy = N * G;
  for (int g = 0; g < G; ++g) {
    const int64_t mr = (int64_t)g * M * r;
    if (!T) QL_TRY(launch_lora_skinny(X, M, K, K, L1 + (int64_t)g * K * r, true, r, 1.0f, Tw + mr, part, s));
    QL_TRY(launch_lora_skinny(dY + (int64_t)g * N, M, N, ldy, L2 + (int64_t)g * r * N, false, r, lora_scale, Gm + mr,
                              part, s));
  }
  const uint16_t* Tg = T ? T : Tw;
  SideStream* sd = dX ? side_stream() : nullptr;
  const bool fork = sd && dx_last_round_partial(*sd, M, K, N * G);
  if (fork) QL_TRY(hipEventRecord(sd->fork, s));
  if (dX) QL_TRY(launch_qgemm_big(true, dY, M, K, N * G, codes, c2, c1, Gm, L1, r, 1.0f, dX, s, G));
  hipStream_t st = s;
  if (fork) {
    QL_TRY(hipStreamWaitEvent(sd->s, sd->fork, 0));
    st = sd->s;
  }
  hipError_t e = hipSuccess;
  for (int g = 0; g < G && e == hipSuccess; ++g) {
    const int64_t mr = (int64_t)g * M * r;
    e = launch_lora_tn_pair(X, K, Gm + mr, K, 1.0f, dL1 + (int64_t)g * K * r, dY + (int64_t)g * N, ldy, Tg + mr, N,
                            lora_scale, dL2 + (int64_t)g * r * N, M, r, part, st);
  }
  if (fork) e = join_side(*sd, s, e);
  QL_TRY(e);
  return QL_OK;
}

int qlora_adamw_step(float* param, float* exp_avg, float* exp_avg_sq, const float* grad, uint16_t* param_bf16,
                     int64_t n, float lr, float beta1, float beta2, float eps, float weight_decay, int64_t step,
                     void* stream) {
  if (!param || !exp_avg || !exp_avg_sq || !grad) return QL_ERR_NULL;
  if (n <= 0 || n > (int64_t(1) << 40) || step < 1) return QL_ERR_SHAPE;
  if (!(lr >= 0.0f) || !(beta1 >= 0.0f && beta1 < 1.0f) || !(beta2 >= 0.0f && beta2 < 1.0f) || !(eps > 0.0f) ||
      !(weight_decay >= 0.0f) || !std::isfinite(lr) || !std::isfinite(eps) || !std::isfinite(weight_decay))
    return QL_ERR_VALUE;
  if (!aligned16(param) || !aligned16(exp_avg) || !aligned16(exp_avg_sq) || !aligned16(grad) ||
      (param_bf16 && !aligned16(param_bf16)))
    return QL_ERR_ALIGN;
  QL_TRY(launch_adamw(param, exp_avg, exp_avg_sq, grad, param_bf16, n, lr, beta1, beta2, eps, weight_decay, step,
                      (hipStream_t)stream));
  return QL_OK;
}

size_t qlora_linear_fwd_workspace(int64_t M, int64_t K, int64_t N, int r) {
  if (!shapes_ok(M, K, N, r)) return 0;
  return fwd_ws(M, K, N, r).total;
}

int qlora_linear_fwd(const uint16_t* X, int64_t M, int64_t K, int64_t N, const uint8_t* codes, const uint8_t* c2,
                     const float* c1, const uint16_t* L1, const uint16_t* L2, int r, float lora_scale, uint16_t* Y,
                     uint16_t* T_out, void* workspace, size_t ws_bytes, void* stream) {
  if (!X || !codes || !c2 || !c1 || !L1 || !L2 || !Y) return QL_ERR_NULL;
  if (!shapes_ok(M, K, N, r)) return QL_ERR_SHAPE;
  if (!aligned16(X) || !aligned16(codes) || !aligned16(c2) || !aligned16(c1) || !aligned16(L1) ||
      !aligned16(L2) || !aligned16(Y) || (T_out && !aligned16(T_out)))
    return QL_ERR_ALIGN;
  const FwdWs w = fwd_ws(M, K, N, r);
  if (!workspace || ws_bytes < w.total) return QL_ERR_WORKSPACE;
  if (!aligned16(workspace)) return QL_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  uint16_t* T = T_out ? T_out : (uint16_t*)ws;
  float* part = (float*)(ws + w.t_bytes);
  if (qgemv_fused_ok(M, K, r) && decode_t_ok(M, K, X, L1) && !capturing(s)) {
    // decode, small X: the slices of T = X L1 formed, added and rounded in the decode launch itself
    // (not under graph capture: a replay would reuse this call's epoch and could take an earlier
    // replay's T; the two launches below are safe to replay)
    void* sync = ws + w.t_bytes + w.part_bytes;
    QL_TRY(launch_qgemv_fwd_fused(X, M, K, N, codes, c2, c1, L1, r, part, sync, next_epoch(), decode_spins(),
                                  T_out, L2, lora_scale, Y, s));
    return QL_OK;
  }
  if (M <= 16 && (r % 4) == 0 && decode_t_ok(M, K, X, L1)) {
    // decode: the slices of T = X L1, added and rounded inside the decode kernel
    QL_TRY(launch_lora_part(X, M, K, L1, r, part, s));
    QL_TRY(launch_qgemv_fwd_tpart(X, M, K, N, codes, c2, c1, part, decode_t_slices(K), T_out, L2, r, lora_scale, Y,
                                  s));
    return QL_OK;
  }
  QL_TRY(launch_lora_skinny(X, M, K, K, L1, true, r, 1.0f, T, part, s));
  if (M <= 16)
    QL_TRY(launch_qgemv_fwd(X, M, K, N, codes, c2, c1, T, L2, r, lora_scale, Y, s));
  else
    QL_TRY(run_fwd_gemm(X, M, K, N, codes, c2, c1, T, L2, r, lora_scale, Y, s));
  return QL_OK;
}

size_t qlora_linear_bwd_workspace(int64_t M, int64_t K, int64_t N, int r) {
  if (!shapes_ok(M, K, N, r)) return 0;
  return bwd_ws(M, K, N, r).total;
}

int qlora_linear_bwd(const uint16_t* X, const uint16_t* dY, int64_t M, int64_t K, int64_t N, const uint8_t* codes,
                     const uint8_t* c2, const float* c1, const uint16_t* L1, const uint16_t* L2, int r,
                     float lora_scale, const uint16_t* T, uint16_t* dX, float* dL1, float* dL2, void* workspace,
                     size_t ws_bytes, void* stream) {
  if (!X || !dY || !codes || !c2 || !c1 || !L1 || !L2 || !dL1 || !dL2) return QL_ERR_NULL;
  if (!shapes_ok(M, K, N, r)) return QL_ERR_SHAPE;
  if (!aligned16(X) || !aligned16(dY) || !aligned16(codes) || !aligned16(c2) || !aligned16(c1) ||
      !aligned16(L1) || !aligned16(L2) || !aligned16(dL1) || !aligned16(dL2) || (T && !aligned16(T)) ||
      (dX && !aligned16(dX)))
    return QL_ERR_ALIGN;
  const BwdWs w = bwd_ws(M, K, N, r);
  if (!workspace || ws_bytes < w.total) return QL_ERR_WORKSPACE;
  if (!aligned16(workspace)) return QL_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  uint16_t* Tw = (uint16_t*)ws;
  uint16_t* G = (uint16_t*)(ws + w.t_bytes);
  float* part = (float*)(ws + w.t_bytes + w.g_bytes);
  if (!T) {
    QL_TRY(launch_lora_skinny(X, M, K, K, L1, true, r, 1.0f, Tw, part, s));
    T = Tw;
  }
  QL_TRY(launch_lora_skinny(dY, M, N, N, L2, false, r, lora_scale, G, part, s));
  SideStream* sd = dX ? side_stream() : nullptr;
  if (sd && dx_last_round_partial(*sd, M, K, N)) {
    QL_TRY(hipEventRecord(sd->fork, s));
    QL_TRY(run_dx_gemm(dY, M, K, N, codes, c2, c1, G, L1, r, dX, s));
    QL_TRY(hipStreamWaitEvent(sd->s, sd->fork, 0));
    const hipError_t e = launch_lora_tn_pair(X, K, G, K, 1.0f, dL1, dY, N, T, N, lora_scale, dL2, M, r, part, sd->s);
    QL_TRY(join_side(*sd, s, e));
    return QL_OK;
  }
  if (dX) QL_TRY(run_dx_gemm(dY, M, K, N, codes, c2, c1, G, L1, r, dX, s));
  QL_TRY(launch_lora_tn_pair(X, K, G, K, 1.0f, dL1, dY, N, T, N, lora_scale, dL2, M, r, part, s));
  return QL_OK;
}

size_t qlora_lora_down_workspace(int64_t M, int64_t K, int r) {
  if (!shapes_ok(M, K, 1, r)) return 0;
  return round_up(lora_skinny_ws(M, K, r));
}

int qlora_lora_down(const uint16_t* X, int64_t M, int64_t K, const uint16_t* L1, int r, uint16_t* T,
                    void* workspace, size_t ws_bytes, void* stream) {
  if (!X || !L1 || !T) return QL_ERR_NULL;
  if (!shapes_ok(M, K, 1, r)) return QL_ERR_SHAPE;
  if (!aligned16(X) || !aligned16(L1) || !aligned16(T)) return QL_ERR_ALIGN;
  if (!workspace || ws_bytes < qlora_lora_down_workspace(M, K, r)) return QL_ERR_WORKSPACE;
  if (!aligned16(workspace)) return QL_ERR_ALIGN;
  QL_TRY(launch_lora_skinny(X, M, K, K, L1, true, r, 1.0f, T, (float*)workspace, (hipStream_t)stream));
  return QL_OK;
}

int qlora_linear_fwd_t(const uint16_t* X, int64_t M, int64_t K, int64_t N, const uint8_t* codes,
                       const uint8_t* c2, const float* c1, const uint16_t* T, const uint16_t* L2, int r,
                       float lora_scale, uint16_t* Y, void* stream) {
  if (!X || !codes || !c2 || !c1 || !T || !L2 || !Y) return QL_ERR_NULL;
  if (!shapes_ok(M, K, N, r)) return QL_ERR_SHAPE;
  if (!aligned16(X) || !aligned16(codes) || !aligned16(c2) || !aligned16(c1) || !aligned16(T) ||
      !aligned16(L2) || !aligned16(Y))
    return QL_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  if (M <= 16)
    QL_TRY(launch_qgemv_fwd(X, M, K, N, codes, c2, c1, T, L2, r, lora_scale, Y, s));
  else
    QL_TRY(run_fwd_gemm(X, M, K, N, codes, c2, c1, T, L2, r, lora_scale, Y, s));
  return QL_OK;
}

size_t qlora_lora_grad_in_workspace(int64_t M, int64_t N, int r) {
  if (!(M > 0 && N > 0 && r >= 1 && r <= 64 && M < (int64_t(1) << 31) && N < (int64_t(1) << 31) &&
        M * N * 2 < (int64_t(1) << 31)))
    return 0;
  return round_up(lora_skinny_ws(M, N, r));
}

int qlora_lora_grad_in(const uint16_t* dY, int64_t M, int64_t N, const uint16_t* L2, int r, float lora_scale,
                       uint16_t* G, void* workspace, size_t ws_bytes, void* stream) {
  if (!dY || !L2 || !G) return QL_ERR_NULL;
  const size_t need = qlora_lora_grad_in_workspace(M, N, r);
  if (need == 0) return QL_ERR_SHAPE;
  if (!aligned16(dY) || !aligned16(L2) || !aligned16(G)) return QL_ERR_ALIGN;
  if (!workspace || ws_bytes < need) return QL_ERR_WORKSPACE;
  if (!aligned16(workspace)) return QL_ERR_ALIGN;
  QL_TRY(launch_lora_skinny(dY, M, N, N, L2, false, r, lora_scale, G, (float*)workspace, (hipStream_t)stream));
  return QL_OK;
}

int qlora_linear_dx(const uint16_t* dY, int64_t M, int64_t K, int64_t N, const uint8_t* codes, const uint8_t* c2,
                    const float* c1, const uint16_t* G, const uint16_t* L1, int r, uint16_t* dX, void* stream) {
  if (!dY || !codes || !c2 || !c1 || !G || !L1 || !dX) return QL_ERR_NULL;
  if (!shapes_ok(M, K, N, r)) return QL_ERR_SHAPE;
  if (!aligned16(dY) || !aligned16(codes) || !aligned16(c2) || !aligned16(c1) || !aligned16(G) ||
      !aligned16(L1) || !aligned16(dX))
    return QL_ERR_ALIGN;
  QL_TRY(run_dx_gemm(dY, M, K, N, codes, c2, c1, G, L1, r, dX, (hipStream_t)stream));
  return QL_OK;
}

// ---- LoRA over a bf16 base (the same GEMM kernels with a bf16 weight) -------
int lora_linear_fwd_t(const uint16_t* X, int64_t M, int64_t K, int64_t N, const uint16_t* W, const uint16_t* T,
                      const uint16_t* L2, int r, float lora_scale, uint16_t* Y, void* stream) {
  if (!X || !W || !T || !L2 || !Y) return QL_ERR_NULL;
  if (!shapes_ok(M, K, N, r) || !bgemm_ok(false, M, K, N)) return QL_ERR_SHAPE;
  if (!aligned16(X) || !aligned16(W) || !aligned16(T) || !aligned16(L2) || !aligned16(Y)) return QL_ERR_ALIGN;
  QL_TRY(launch_bgemm_big(false, X, M, K, N, W, T, L2, r, lora_scale, Y, (hipStream_t)stream));
  return QL_OK;
}

int lora_linear_dx(const uint16_t* dY, int64_t M, int64_t K, int64_t N, const uint16_t* W, const uint16_t* G,
                   const uint16_t* L1, int r, uint16_t* dX, void* stream) {
  if (!dY || !W || !G || !L1 || !dX) return QL_ERR_NULL;
  if (!shapes_ok(M, K, N, r) || !bgemm_ok(true, M, K, N)) return QL_ERR_SHAPE;
  if (!aligned16(dY) || !aligned16(W) || !aligned16(G) || !aligned16(L1) || !aligned16(dX)) return QL_ERR_ALIGN;
  QL_TRY(launch_bgemm_big(true, dY, M, K, N, W, G, L1, r, 1.0f, dX, (hipStream_t)stream));
  return QL_OK;
}

int lora_linear_fwd(const uint16_t* X, int64_t M, int64_t K, int64_t N, const uint16_t* W, const uint16_t* L1,
                    const uint16_t* L2, int r, float lora_scale, uint16_t* Y, uint16_t* T_out, void* workspace,
                    size_t ws_bytes, void* stream) {
  if (!X || !W || !L1 || !L2 || !Y) return QL_ERR_NULL;
  if (!shapes_ok(M, K, N, r) || !bgemm_ok(false, M, K, N)) return QL_ERR_SHAPE;
  if (!aligned16(X) || !aligned16(W) || !aligned16(L1) || !aligned16(L2) || !aligned16(Y) ||
      (T_out && !aligned16(T_out)))
    return QL_ERR_ALIGN;
  const FwdWs w = fwd_ws(M, K, N, r);
  if (!workspace || ws_bytes < w.total) return QL_ERR_WORKSPACE;
  if (!aligned16(workspace)) return QL_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  uint16_t* T = T_out ? T_out : (uint16_t*)ws;
  QL_TRY(launch_lora_skinny(X, M, K, K, L1, true, r, 1.0f, T, (float*)(ws + w.t_bytes), s));
  QL_TRY(launch_bgemm_big(false, X, M, K, N, W, T, L2, r, lora_scale, Y, s));
  return QL_OK;
}

int lora_linear_bwd(const uint16_t* X, const uint16_t* dY, int64_t M, int64_t K, int64_t N, const uint16_t* W,
                    const uint16_t* L1, const uint16_t* L2, int r, float lora_scale, const uint16_t* T, uint16_t* dX,
                    float* dL1, float* dL2, void* workspace, size_t ws_bytes, void* stream) {
  if (!X || !dY || !W || !L1 || !L2 || !dL1 || !dL2) return QL_ERR_NULL;
  if (!shapes_ok(M, K, N, r) || !bgemm_ok(true, M, K, N)) return QL_ERR_SHAPE;
  if (!aligned16(X) || !aligned16(dY) || !aligned16(W) || !aligned16(L1) || !aligned16(L2) || !aligned16(dL1) ||
      !aligned16(dL2) || (T && !aligned16(T)) || (dX && !aligned16(dX)))
    return QL_ERR_ALIGN;
  const BwdWs w = bwd_ws(M, K, N, r);
  if (!workspace || ws_bytes < w.total) return QL_ERR_WORKSPACE;
  if (!aligned16(workspace)) return QL_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  uint16_t* Tw = (uint16_t*)ws;
  uint16_t* G = (uint16_t*)(ws + w.t_bytes);
  float* part = (float*)(ws + w.t_bytes + w.g_bytes);
  if (!T) {
    QL_TRY(launch_lora_skinny(X, M, K, K, L1, true, r, 1.0f, Tw, part, s));
    T = Tw;
  }
  QL_TRY(launch_lora_skinny(dY, M, N, N, L2, false, r, lora_scale, G, part, s));
  if (dX) QL_TRY(launch_bgemm_big(true, dY, M, K, N, W, G, L1, r, 1.0f, dX, s));
  QL_TRY(launch_lora_tn_pair(X, K, G, K, 1.0f, dL1, dY, N, T, N, lora_scale, dL2, M, r, part, s));
  return QL_OK;
}

int qlora_nf4_levels(float* out16) {
  if (!out16) return QL_ERR_NULL;
  std::memcpy(out16, nf4_params().q, 16 * sizeof(float));
  return QL_OK;
}

const char* ql_status_string(int status) {
  switch (status) {
    case QL_OK: return "ok";
    case QL_ERR_NULL: return "a required pointer is NULL";
    case QL_ERR_SHAPE:
      return "invalid shape (sizes must be > 0, K and cols multiples of 64, 1 <= r <= 64, each activation "
             "matrix and the packed codes below 2^31 bytes)";
    case QL_ERR_DTYPE: return "unsupported dtype, code book or scale code";
    case QL_ERR_VALUE: return "hyper-parameter out of range";
    case QL_ERR_ALIGN: return "device pointers must be 16-byte aligned";
    case QL_ERR_WORKSPACE: return "workspace missing or smaller than the size query returns";
    case QL_ERR_HIP:
      std::snprintf(g_msg, sizeof g_msg, "HIP launch failed: %s", hipGetErrorString(g_last_hip));
      return g_msg;
    default: return "unknown status";
  }
}

}  // extern "C"
