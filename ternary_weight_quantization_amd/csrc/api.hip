// C ABI of libbitnet.so (declared in include/bitnet.h): argument
// validation, then the launches on the caller's stream. Nothing here
// allocates device memory or synchronizes the host.

#include <hip/hip_runtime.h>

#include "../../include/bitnet.h"
#include "internal.h"

namespace {

constexpr int64_t kMaxDim = int64_t(1) << 30;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bitnet_status from_hip(hipError_t e) { return e == hipSuccess ? BITNET_OK : BITNET_ERR_HIP; }

bitnet_status check_sizes(int64_t a, int64_t b) {
  if (a < 1 || b < 1 || a > kMaxDim || b > kMaxDim) return BITNET_ERR_SHAPE;
  return BITNET_OK;
}

// Sizes of the GEMMs: M, N, K >= 1; the int8 accumulation stays below 2^31
// (127 * Kp < 2^31); tile and element counts fit the kernels' int indexing.
bitnet_status check_gemm_sizes(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || N < 1 || K < 1) return BITNET_ERR_SHAPE;
  if (M > kMaxDim || N > kMaxDim || K > (int64_t(1) << 24)) return BITNET_ERR_SHAPE;
  const int64_t ti = (N + 255) / 256, tk = (bitnet::k_pad(K) + 255) / 256, tm = (M + 255) / 256;
  if (ti * tm > (int64_t(1) << 30) || tk * tm > (int64_t(1) << 30) || tk * ti > (int64_t(1) << 30))
    return BITNET_ERR_SHAPE;
  return BITNET_OK;
}

// The GEMM kernels address x_q, w_packed, dY and s_x through buffer
// resources with 32-bit offsets, including rows up to 256 past an operand's
// end (read as zeros); each such range must stay below 2 GiB.
bool buffer_range_ok(int64_t rows, int64_t pitch_bytes) {
  return (rows + 256) * pitch_bytes <= (int64_t(1) << 31);
}

// out_elems: elements per output row (N for the forward, K for dX and dW).
// The epilogue addresses 32 output rows of up to 4-byte elements with 32-bit
// offsets.
bitnet_status check_gemm_ranges(int64_t M, int64_t N, int64_t K, bool need_xq, bool need_w, bool need_dy,
                                int64_t out_elems) {
  const int64_t Kp = bitnet::k_pad(K);
  if (32 * 4 * out_elems > (int64_t(1) << 31)) return BITNET_ERR_SHAPE;
  if (need_xq && !buffer_range_ok(M, Kp)) return BITNET_ERR_SHAPE;
  if (need_xq && !buffer_range_ok(M, 2 * Kp)) return BITNET_ERR_SHAPE;  // dW's bf16 x_hat
  if (need_w && !buffer_range_ok(N, Kp / 4)) return BITNET_ERR_SHAPE;
  if (need_dy && !buffer_range_ok(M, 2 * N)) return BITNET_ERR_SHAPE;
  // dX reads the codes transposed to fp4 [Kp][Np/2] (Np = N rounded up to 64)
  if (need_w && need_dy && !buffer_range_ok(Kp, (N + 63) / 64 * 32)) return BITNET_ERR_SHAPE;
  return BITNET_OK;
}

}  // namespace

extern "C" {

const char* bitnet_status_string(bitnet_status status) {
  switch (status) {
    case BITNET_OK: return "BITNET_OK";
    case BITNET_ERR_NULL: return "BITNET_ERR_NULL: a required pointer is NULL";
    case BITNET_ERR_SHAPE: return "BITNET_ERR_SHAPE: a size is out of range";
    case BITNET_ERR_DTYPE: return "BITNET_ERR_DTYPE: unsupported dtype";
    case BITNET_ERR_ALIGN: return "BITNET_ERR_ALIGN: a pointer is not aligned as required";
    case BITNET_ERR_WORKSPACE: return "BITNET_ERR_WORKSPACE: workspace missing or too small";
    case BITNET_ERR_HIP: return "BITNET_ERR_HIP: the HIP runtime reported an error";
  }
  return "BITNET_ERR_UNKNOWN";
}

int64_t bitnet_k_pad(int64_t K) { return K < 1 ? 0 : bitnet::k_pad(K); }

size_t bitnet_ternarize_workspace_bytes(int64_t, int64_t) { return bitnet::quant_workspace_bytes(); }

size_t bitlinear_fwd_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (check_gemm_sizes(M, N, K) != BITNET_OK) return 0;
  return bitnet::gemm_workspace_bytes(bitnet::GemmKind::kFwd, M, N, K);
}

size_t bitlinear_bwd_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (check_gemm_sizes(M, N, K) != BITNET_OK) return 0;
  // dX and dW run either in one launch (N % 8 == 0, both requested) or one
  // after the other, sharing the workspace
  return bitnet::gemm_workspace_bytes(bitnet::GemmKind::kBwdPair, M, N, K);
}

bitnet_status bitnet_ternarize_pack(const void* W, bitnet_dtype w_dtype, int64_t N, int64_t K,
                                    uint8_t* w_packed, float* gamma, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  if (!W || !w_packed || !gamma) return BITNET_ERR_NULL;
  if (w_dtype != BITNET_BF16 && w_dtype != BITNET_F32) return BITNET_ERR_DTYPE;
  if (bitnet_status st = check_sizes(N, K)) return st;
  if (N * K > (int64_t(1) << 53)) return BITNET_ERR_SHAPE;
  if (!aligned(W, 16) || !aligned(w_packed, 16) || !aligned(gamma, 4)) return BITNET_ERR_ALIGN;
  if (!workspace || workspace_bytes < bitnet_ternarize_workspace_bytes(N, K)) return BITNET_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return BITNET_ERR_ALIGN;
  return from_hip(bitnet::launch_ternarize_pack(W, w_dtype == BITNET_F32, N, K, w_packed, gamma,
                                                static_cast<double*>(workspace),
                                                static_cast<hipStream_t>(stream)));
}

bitnet_status bitnet_quantize(const void* W, bitnet_dtype w_dtype, int64_t N, int64_t K, const uint16_t* x,
                              int64_t M, uint8_t* w_packed, float* gamma, int8_t* x_q, float* s_x, void* workspace,
                              size_t workspace_bytes, void* stream) {
  if (!W || !w_packed || !gamma || !x || !x_q || !s_x) return BITNET_ERR_NULL;
  if (w_dtype != BITNET_BF16 && w_dtype != BITNET_F32) return BITNET_ERR_DTYPE;
  if (bitnet_status st = check_sizes(N, K)) return st;
  if (bitnet_status st = check_sizes(M, K)) return st;
  if (N * K > (int64_t(1) << 53)) return BITNET_ERR_SHAPE;
  if (!aligned(W, 16) || !aligned(w_packed, 16) || !aligned(gamma, 4) || !aligned(x, 16) || !aligned(x_q, 16) ||
      !aligned(s_x, 16))
    return BITNET_ERR_ALIGN;
  if (!workspace || workspace_bytes < bitnet_ternarize_workspace_bytes(N, K)) return BITNET_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return BITNET_ERR_ALIGN;
  return from_hip(bitnet::launch_quantize(W, w_dtype == BITNET_F32, N, K, x, M, w_packed, gamma, x_q, s_x,
                                          static_cast<double*>(workspace), static_cast<hipStream_t>(stream)));
}

bitnet_status bitnet_code_counts(const uint8_t* w_packed, int64_t N, int64_t K, uint64_t* counts, void* stream) {
  if (!w_packed || !counts) return BITNET_ERR_NULL;
  if (bitnet_status st = check_sizes(N, K)) return st;
  if (!aligned(w_packed, 16) || !aligned(counts, 8)) return BITNET_ERR_ALIGN;
  return from_hip(bitnet::launch_code_counts(w_packed, N, K, reinterpret_cast<unsigned long long*>(counts),
                                             static_cast<hipStream_t>(stream)));
}

bitnet_status bitnet_act_quant(const uint16_t* x, int64_t M, int64_t K, int8_t* x_q, float* s_x,
                               void* stream) {
  if (!x || !x_q || !s_x) return BITNET_ERR_NULL;
  if (bitnet_status st = check_sizes(M, K)) return st;
  if (!aligned(x, 16) || !aligned(x_q, 16) || !aligned(s_x, 16)) return BITNET_ERR_ALIGN;
  return from_hip(bitnet::launch_act_quant(x, M, K, x_q, s_x, static_cast<hipStream_t>(stream)));
}

bitnet_status bitlinear_fwd_bias(const int8_t* x_q, const float* s_x, const uint8_t* w_packed,
                                 const float* gamma, const uint16_t* bias, int64_t M, int64_t N, int64_t K,
                                 uint16_t* y, int32_t* acc_out, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  if (!x_q || !s_x || !w_packed || !gamma || !y) return BITNET_ERR_NULL;
  if (bitnet_status st = check_gemm_sizes(M, N, K)) return st;
  if (bitnet_status st = check_gemm_ranges(M, N, K, true, true, false, N)) return st;
  if (workspace_bytes < bitlinear_fwd_workspace_bytes(M, N, K)) return BITNET_ERR_WORKSPACE;
  if (workspace_bytes > 0 && !workspace) return BITNET_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return BITNET_ERR_ALIGN;
  if (!aligned(x_q, 16) || !aligned(s_x, 16) || !aligned(w_packed, 16) || !aligned(gamma, 4) ||
      !aligned(y, 16) || (acc_out && !aligned(acc_out, 16)) || !aligned(bias, 16))
    return BITNET_ERR_ALIGN;
  return from_hip(bitnet::launch_fwd(x_q, s_x, w_packed, gamma, bias, M, N, K, y, acc_out, workspace,
                                     workspace_bytes, static_cast<hipStream_t>(stream)));
}

bitnet_status bitlinear_fwd(const int8_t* x_q, const float* s_x, const uint8_t* w_packed,
                            const float* gamma, int64_t M, int64_t N, int64_t K, uint16_t* y,
                            int32_t* acc_out, void* workspace, size_t workspace_bytes, void* stream) {
  return bitlinear_fwd_bias(x_q, s_x, w_packed, gamma, nullptr, M, N, K, y, acc_out, workspace, workspace_bytes,
                            stream);
}

bitnet_status bitlinear_bias_grad(const uint16_t* dY, int64_t M, int64_t N, void* db, bitnet_dtype db_dtype,
                                  void* stream) {
  if (!dY || !db) return BITNET_ERR_NULL;
  if (db_dtype != BITNET_BF16 && db_dtype != BITNET_F32) return BITNET_ERR_DTYPE;
  if (bitnet_status st = check_sizes(M, N)) return st;
  if (!aligned(dY, 16) || !aligned(db, 16)) return BITNET_ERR_ALIGN;
  return from_hip(bitnet::launch_bias_grad(dY, M, N, db, db_dtype == BITNET_F32, static_cast<hipStream_t>(stream)));
}

bitnet_status bitlinear_bwd(const uint16_t* dY, const int8_t* x_q, const float* s_x,
                            const uint8_t* w_packed, const float* gamma, int64_t M, int64_t N,
                            int64_t K, uint16_t* dX, void* dW, bitnet_dtype dW_dtype,
                            void* workspace, size_t workspace_bytes, void* stream) {
  if (!dY) return BITNET_ERR_NULL;
  if (!dX && !dW) return BITNET_ERR_NULL;
  if (dX && (!w_packed || !gamma)) return BITNET_ERR_NULL;
  if (dW && (!x_q || !s_x)) return BITNET_ERR_NULL;
  if (dW && dW_dtype != BITNET_BF16 && dW_dtype != BITNET_F32 && dW_dtype != BITNET_SIGN1) return BITNET_ERR_DTYPE;
  if (bitnet_status st = check_gemm_sizes(M, N, K)) return st;
  if (bitnet_status st = check_gemm_ranges(M, N, K, dW != nullptr, dX != nullptr, true, K)) return st;
  if (workspace_bytes < bitlinear_bwd_workspace_bytes(M, N, K)) return BITNET_ERR_WORKSPACE;
  if (workspace_bytes > 0 && !workspace) return BITNET_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return BITNET_ERR_ALIGN;
  if (!aligned(dY, 16)) return BITNET_ERR_ALIGN;
  if (dX && (!aligned(w_packed, 16) || !aligned(gamma, 4) || !aligned(dX, 16))) return BITNET_ERR_ALIGN;
  if (dW && (!aligned(x_q, 16) || !aligned(s_x, 16) || !aligned(dW, 16))) return BITNET_ERR_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bitnet::DwOut dw_out = dW_dtype == BITNET_F32     ? bitnet::DwOut::kF32
                               : dW_dtype == BITNET_SIGN1 ? bitnet::DwOut::kSign1
                                                          : bitnet::DwOut::kBf16;
  if (dX && dW) {
    const hipError_t e = bitnet::launch_bwd_pair(dY, w_packed, gamma, x_q, s_x, M, N, K, dX, dW, dw_out,
                                                 workspace, workspace_bytes, st);
    if (e != hipErrorNotSupported) return from_hip(e);
  }
  if (dX) {
    if (hipError_t e = bitnet::launch_bwd_dx(dY, w_packed, gamma, M, N, K, dX, workspace, workspace_bytes, st)) return from_hip(e);
  }
  if (dW) {
    if (hipError_t e = bitnet::launch_bwd_dw(dY, x_q, s_x, M, N, K, dW, dw_out, workspace, workspace_bytes, st))
      return from_hip(e);
  }
  return BITNET_OK;
}

// ---------------------------------------------------------------------------
// TTQ
// ---------------------------------------------------------------------------

size_t ttq_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (check_gemm_sizes(M, N, K) != BITNET_OK) return 0;
  const size_t a = bitnet::gemm_workspace_bytes(bitnet::GemmKind::kTtqFwd, M, N, K);
  const size_t b = bitnet::gemm_workspace_bytes(bitnet::GemmKind::kTtqBwd, M, N, K);
  return a > b ? a : b;
}

bitnet_status ttq_init(const void* W, bitnet_dtype w_dtype, int64_t N, int64_t K, float* params, void* workspace,
                       size_t workspace_bytes, void* stream) {
  if (!W || !params) return BITNET_ERR_NULL;
  if (w_dtype != BITNET_BF16 && w_dtype != BITNET_F32) return BITNET_ERR_DTYPE;
  if (bitnet_status st = check_sizes(N, K)) return st;
  if (N * K > (int64_t(1) << 53)) return BITNET_ERR_SHAPE;
  if (!aligned(W, 16) || !aligned(params, 4)) return BITNET_ERR_ALIGN;
  if (!workspace || workspace_bytes < bitnet_ternarize_workspace_bytes(N, K)) return BITNET_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return BITNET_ERR_ALIGN;
  return from_hip(bitnet::launch_ttq_init(W, w_dtype == BITNET_F32, N, K, params, static_cast<double*>(workspace),
                                          static_cast<hipStream_t>(stream)));
}

bitnet_status ttq_quantize(const void* W, bitnet_dtype w_dtype, int64_t N, int64_t K, const float* params,
                           uint8_t* w_packed, uint16_t* wt, void* stream) {
  if (!W || !params || !w_packed || !wt) return BITNET_ERR_NULL;
  if (w_dtype != BITNET_BF16 && w_dtype != BITNET_F32) return BITNET_ERR_DTYPE;
  if (bitnet_status st = check_sizes(N, K)) return st;
  if (N * bitnet::k_pad(K) > (int64_t(1) << 53)) return BITNET_ERR_SHAPE;
  if (!aligned(W, 16) || !aligned(params, 4) || !aligned(w_packed, 16) || !aligned(wt, 16)) return BITNET_ERR_ALIGN;
  return from_hip(bitnet::launch_ttq_quantize(W, w_dtype == BITNET_F32, N, K, params, w_packed, wt,
                                              static_cast<hipStream_t>(stream)));
}

bitnet_status ttq_fwd(const uint16_t* x, const uint16_t* wt, int64_t M, int64_t N, int64_t K, uint16_t* y,
                      void* workspace, size_t workspace_bytes, void* stream) {
  if (!x || !wt || !y) return BITNET_ERR_NULL;
  if (bitnet_status st = check_gemm_sizes(M, N, K)) return st;
  const int64_t Kp = bitnet::k_pad(K);
  if (32 * 4 * N > (int64_t(1) << 31) || !buffer_range_ok(M, 2 * K) || !buffer_range_ok(N, 2 * Kp))
    return BITNET_ERR_SHAPE;
  if (workspace_bytes < ttq_workspace_bytes(M, N, K)) return BITNET_ERR_WORKSPACE;
  if (workspace_bytes > 0 && !workspace) return BITNET_ERR_WORKSPACE;
  if (!aligned(workspace, 16) || !aligned(x, 16) || !aligned(wt, 16) || !aligned(y, 16)) return BITNET_ERR_ALIGN;
  return from_hip(bitnet::launch_ttq_fwd(x, wt, M, N, K, y, workspace, workspace_bytes,
                                         static_cast<hipStream_t>(stream)));
}

size_t ttq_fwd_codes_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (check_gemm_sizes(M, N, K) != BITNET_OK) return 0;
  return bitnet::ttq_codes_workspace_bytes(M, N, K);
}

bitnet_status ttq_fwd_codes(const uint16_t* x, const uint8_t* w_packed, const float* params, int64_t M, int64_t N,
                            int64_t K, uint16_t* y, void* workspace, size_t workspace_bytes, void* stream) {
  if (!x || !w_packed || !params || !y) return BITNET_ERR_NULL;
  if (bitnet_status st = check_gemm_sizes(M, N, K)) return st;
  const int64_t Kp = bitnet::k_pad(K);
  if (32 * 4 * N > (int64_t(1) << 31) || !buffer_range_ok(M, 2 * K) || !buffer_range_ok(N, 2 * Kp) ||
      !buffer_range_ok(N, Kp / 4))
    return BITNET_ERR_SHAPE;
  const size_t need = ttq_fwd_codes_workspace_bytes(M, N, K);
  if (workspace_bytes < need || (need > 0 && !workspace)) return BITNET_ERR_WORKSPACE;
  if (!aligned(workspace, 16) || !aligned(x, 16) || !aligned(w_packed, 16) || !aligned(params, 4) ||
      !aligned(y, 16))
    return BITNET_ERR_ALIGN;
  return from_hip(bitnet::launch_ttq_fwd_codes(x, w_packed, params, M, N, K, y, workspace, workspace_bytes,
                                               static_cast<hipStream_t>(stream)));
}

bitnet_status ttq_bwd(const uint16_t* dY, const uint16_t* x, const uint16_t* wt, const uint8_t* w_packed, int64_t M,
                      int64_t N, int64_t K, uint16_t* dX, void* dW, bitnet_dtype dW_dtype, float* grads,
                      void* workspace, size_t workspace_bytes, void* stream) {
  if (!dY) return BITNET_ERR_NULL;
  if (!dX && !dW) return BITNET_ERR_NULL;
  if (dX && !wt) return BITNET_ERR_NULL;
  if (dW && !x) return BITNET_ERR_NULL;
  if (grads && (!dW || !w_packed)) return BITNET_ERR_NULL;
  if (dW && dW_dtype != BITNET_BF16 && dW_dtype != BITNET_F32) return BITNET_ERR_DTYPE;
  if (bitnet_status st = check_gemm_sizes(M, N, K)) return st;
  const int64_t Kp = bitnet::k_pad(K);
  if (32 * 4 * K > (int64_t(1) << 31) || !buffer_range_ok(M, 2 * N)) return BITNET_ERR_SHAPE;
  if (dX && !buffer_range_ok(N, 2 * Kp)) return BITNET_ERR_SHAPE;
  if (dW && !buffer_range_ok(M, 2 * K)) return BITNET_ERR_SHAPE;
  if (grads && !buffer_range_ok(N, Kp / 4)) return BITNET_ERR_SHAPE;
  if (workspace_bytes < ttq_workspace_bytes(M, N, K)) return BITNET_ERR_WORKSPACE;
  if (workspace_bytes > 0 && !workspace) return BITNET_ERR_WORKSPACE;
  if (!aligned(workspace, 16) || !aligned(dY, 16)) return BITNET_ERR_ALIGN;
  if (dX && (!aligned(wt, 16) || !aligned(dX, 16))) return BITNET_ERR_ALIGN;
  if (dW && (!aligned(x, 16) || !aligned(dW, 16))) return BITNET_ERR_ALIGN;
  if (grads && (!aligned(grads, 4) || !aligned(w_packed, 16))) return BITNET_ERR_ALIGN;
  return from_hip(bitnet::launch_ttq_bwd(dY, x, wt, w_packed, M, N, K, dX, dW, dW_dtype == BITNET_F32, grads,
                                         workspace, workspace_bytes, static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------------------
// Test hooks
// ---------------------------------------------------------------------------

void bitnet_set_test_knobs(int split_ctas, int pair_cols, int no_skinny, uint32_t spin_limit) {
  bitnet::TestKnobs& k = bitnet::test_knobs();
  k.split_ctas.store(split_ctas);
  k.pair_cols.store(pair_cols);
  k.no_skinny.store(no_skinny);
  k.spin_limit.store(spin_limit);
}

uint32_t bitnet_default_spin_limit(void) { return bitnet::kDefaultSpinLimit; }

bitnet_status bitnet_split_timeouts(uint32_t* count) {
  if (!count) return BITNET_ERR_NULL;
  unsigned int c = 0;
  const hipError_t e = bitnet::take_split_timeouts(&c);
  *count = c;
  return from_hip(e);
}

bitnet_status bitnet_quantize_recomputes(uint32_t* count) {
  if (!count) return BITNET_ERR_NULL;
  unsigned int c = 0;
  const hipError_t e = bitnet::take_onepass_recomputes(&c);
  *count = c;
  return from_hip(e);
}

int64_t bitnet_debug_split_pieces(int64_t tiles, int32_t stages, int32_t grid, int32_t* v, int32_t* t, int32_t* s0,
                                  int32_t* s1, int64_t* slot, int32_t* va, int32_t* n, int64_t cap) {
  if (tiles < 1 || stages < 1 || grid < 1 || grid > tiles * stages || !v || !t || !s0 || !s1 || !slot || !va || !n)
    return -1;
  return bitnet::debug_split_pieces(tiles, stages, grid, v, t, s0, s1, slot, va, n, cap);
}

int32_t bitnet_debug_partial_slots(int64_t tiles, int32_t grid) {
  const int64_t a = 2 * (int64_t)grid, b = grid + tiles - 1;
  return (int32_t)(a < b ? a : b);
}

bitnet_status bitnet_debug_mfma_probe(int32_t int8, int32_t iters, float* sink, double* ops, void* stream) {
  if (!sink || !ops) return BITNET_ERR_NULL;
  if (iters < 1 || iters > (1 << 24)) return BITNET_ERR_SHAPE;
  *ops = bitnet::mfma_probe_ops(int8 != 0, iters);
  return from_hip(bitnet::launch_mfma_probe(int8 != 0, iters, sink, static_cast<hipStream_t>(stream)));
}

void bitnet_debug_cta_order(int32_t grid, int32_t* out) {
  if (grid >= 1 && out) bitnet::debug_cta_order(grid, out);
}

}  // extern "C"
