// Internal launchers of libbitnet.so. Arguments are validated by the C ABI
// layer (api.hip) before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

namespace bitnet {

// Test and tuning knobs of the GEMM launchers, process-wide, set through
// bitnet_set_test_knobs(). Defaults: the cost models decide.
//  split_ctas  0: cost model; > 0: split every GEMM over that many
//              workgroups (and no paired backward launch); < 0: whole tiles
//  pair_cols   0: cost model; k >= 1: dX gets k of the 8-workgroup columns
//              of a paired backward launch
//  no_skinny   nonzero: the large-M GEMMs also for few tokens
//  spin_limit  polls before a wait for another workgroup's partial tile
//              gives up (the tile is then written as a sentinel and counted)
constexpr uint32_t kDefaultSpinLimit = 1u << 24;
struct TestKnobs {
  std::atomic<int> split_ctas{0};
  std::atomic<int> pair_cols{0};
  std::atomic<int> no_skinny{0};
  std::atomic<uint32_t> spin_limit{kDefaultSpinLimit};
};
TestKnobs& test_knobs();

// Waits for published partial tiles that gave up since the last call (read
// and cleared on the current device; synchronizes the device).
hipError_t take_split_timeouts(unsigned int* count);

// MFMA rate probe: one launch of register-only MFMA chains on every SIMD
// (bf16 32x32x16 or int8 32x32x32), `iters` rounds; mfma_probe_ops() is the
// operation count of such a launch. sink: 2048 floats (never written in
// practice).
hipError_t launch_mfma_probe(bool int8, int iters, float* sink, hipStream_t stream);
double mfma_probe_ops(bool int8, int iters);

// The pieces a split launch of T tiles x S stages over G workgroups runs,
// computed on the host by the same functions the kernels use: for each
// piece, in workgroup order, its virtual workgroup v, tile t, stages
// [s0, s1), partial slot, and the first owner va and piece count n of its
// tile. Returns the number of pieces (at most cap are written).
int64_t debug_split_pieces(int64_t T, int S, int G, int32_t* v, int32_t* t, int32_t* s0, int32_t* s1,
                           int64_t* slot, int32_t* va, int32_t* n, int64_t cap);
// The virtual index of each of G workgroups (cta_order).
void debug_cta_order(int G, int32_t* out);

// Fixed grid of the absmean partial-sum kernel: the partial order (and so
// gamma's bits) never depends on the device or the call.
constexpr int kAbsmeanBlocks = 256;
constexpr int kAbsmeanThreads = 512;

inline int64_t k_pad(int64_t K) { return ((K + 63) / 64) * 64; }

// A fresh tag for a launch that synchronizes its workgroups through tagged
// words in a workspace (nonzero, 48 bits, different for every launch).
uint64_t next_launch_tag();

// The one-pass weight ternarization (W read once, held in registers between
// gamma's reduction and the codes), alone or with the activation rows:
// used for bf16 W with K % 64 == 0 and N * K up to the register capacity.
// ws: the ternarize workspace (quant_workspace_bytes()). x == nullptr: no
// activation rows (with_rows false).
bool onepass_ok(bool w_is_f32, int64_t N, int64_t K, bool with_rows);
void launch_onepass(const uint16_t* W, int64_t N, int64_t K, void* ws, uint32_t* packed, float* gamma,
                    const uint16_t* x, int64_t M, int8_t* xq, float* s, hipStream_t st);
// Bytes of the ternarize workspace: the fp64 absmean partials, then the
// one-pass kernel's publication flags and departure counter.
size_t quant_workspace_bytes();
// Partials one-pass launches computed themselves after an absent flag,
// since the last call (read and cleared on the current device;
// synchronizes the device).
hipError_t take_onepass_recomputes(unsigned int* count);

// Weight ternarization: fp64 absmean partials, then gamma + codes + packing.
hipError_t launch_ternarize_pack(const void* W, bool w_is_f32, int64_t N, int64_t K,
                                 uint8_t* w_packed, float* gamma, double* partials,
                                 hipStream_t stream);

// The pack pass alone (gamma from the partials, codes, packing).
hipError_t launch_pack(const void* W, bool w_is_f32, int64_t N, int64_t K, uint8_t* w_packed, float* gamma,
                       const double* partials, hipStream_t stream);

// Weight ternarization + pack and activation quantization together: the
// absmean partials and the act-quant rows in one launch, then the pack.
hipError_t launch_quantize(const void* W, bool w_is_f32, int64_t N, int64_t K, const uint16_t* x, int64_t M,
                           uint8_t* w_packed, float* gamma, int8_t* x_q, float* s_x, double* partials,
                           hipStream_t stream);

// Bias gradient db[n] = sum_m dY[m][n] (fp32, fixed order), db as f32 or
// bf16 bits.
hipError_t launch_bias_grad(const uint16_t* dY, int64_t M, int64_t N, void* db, bool db_is_f32,
                            hipStream_t stream);

// Counts of the codes -1 and +1 in w_packed [N][Kp/4]: counts[0] = #(-1),
// counts[1] = #(+1) (the zeros are N*K minus both).
hipError_t launch_code_counts(const uint8_t* w_packed, int64_t N, int64_t K, unsigned long long* counts,
                              hipStream_t stream);

// Per-token absmax int8 activation quantization.
hipError_t launch_act_quant(const uint16_t* x, int64_t M, int64_t K,
                            int8_t* x_q, float* s_x, hipStream_t stream);

// The GEMMs (BitNet forward, dX, dW, the paired backward; TTQ forward and
// backward). Each may split output tiles over workgroups (stream-K)
// when its tile count leaves the CUs partly idle; that needs the workspace
// gemm_workspace_bytes() gives (fewer bytes: whole tiles, no split).
enum class GemmKind { kFwd, kBwdDx, kBwdDw, kBwdPair, kTtqFwd, kTtqBwd };
size_t gemm_workspace_bytes(GemmKind kind, int64_t M, int64_t N, int64_t K);

// INT8 forward GEMM with fused rescale, an optional bf16 bias [N] (NULL:
// none) and optional int32 accumulators.
hipError_t launch_fwd(const int8_t* x_q, const float* s_x, const uint8_t* w_packed,
                      const float* gamma, const uint16_t* bias, int64_t M, int64_t N, int64_t K,
                      uint16_t* y, int32_t* acc_out, void* ws, size_t ws_bytes,
                      hipStream_t stream);

// INT8 forward for few tokens (1 <= M <= kSkinnyMaxM): one pass over the
// codes, no workspace; same results, bit for bit, as launch_fwd's GEMM
// (which calls it for such M).
constexpr int64_t kSkinnyMaxM = 64;
hipError_t launch_fwd_skinny(const int8_t* x_q, const float* s_x, const uint8_t* w_packed,
                             const float* gamma, const uint16_t* bias, int64_t M, int64_t N, int64_t K,
                             uint16_t* y, int32_t* acc_out, hipStream_t stream);

// STE dX for few tokens (M <= kSkinnyMaxM, N % 8 == 0) from the fp4
// transposed codes wt [Kp][Np/2] (Np = N rounded up to 64).
hipError_t launch_dx_skinny(const uint8_t* wt, const uint16_t* dY, const float* gamma, int64_t M,
                            int64_t N, int64_t K, uint16_t* dX, hipStream_t stream);

// STE backward GEMMs.
hipError_t launch_bwd_dx(const uint16_t* dY, const uint8_t* w_packed, const float* gamma,
                         int64_t M, int64_t N, int64_t K, uint16_t* dX, void* ws,
                         size_t ws_bytes, hipStream_t stream);
// dW output: bf16, f32, or 1-bit signs [N][Kp/8] (bit set: negative sum).
enum class DwOut { kBf16, kF32, kSign1 };
hipError_t launch_bwd_dw(const uint16_t* dY, const int8_t* x_q, const float* s_x,
                         int64_t M, int64_t N, int64_t K, void* dW, DwOut dw_out,
                         void* ws, size_t ws_bytes, hipStream_t stream);

// Both STE backward products in one launch, each on its share of the CUs
// (N % 8 == 0). hipErrorNotSupported (nothing launched) when the shape,
// the workspace or the device does not allow it; the caller then runs the
// two products one after the other.
hipError_t launch_bwd_pair(const uint16_t* dY, const uint8_t* w_packed, const float* gamma,
                           const int8_t* x_q, const float* s_x, int64_t M, int64_t N, int64_t K,
                           uint16_t* dX, void* dW, DwOut dw_out, void* ws, size_t ws_bytes,
                           hipStream_t stream);

// TTQ ("TTQ_VERIFICATION.md"): params = {delta, Wp, Wn} fp32 on the device.
// Initialization (Eq. 2) from W: E = gamma's absmean, delta = fl32(0.7f E),
// Wp = Wn = E (partials: the ternarize workspace).
hipError_t launch_ttq_init(const void* W, bool w_is_f32, int64_t N, int64_t K, float* params, double* partials,
                           hipStream_t stream);
// Eq. 1: 2-bit codes [N][Kp/4] and bf16 values wt [N][Kp] in one pass.
hipError_t launch_ttq_quantize(const void* W, bool w_is_f32, int64_t N, int64_t K, const float* params,
                               uint8_t* w_packed, uint16_t* wt, hipStream_t stream);
// wt [N][Kp] from stored codes: the values ttq_quantize writes.
hipError_t launch_ttq_expand(const uint8_t* w_packed, int64_t N, int64_t K, const float* params, uint16_t* wt,
                             hipStream_t stream);
// TTQ forward for few tokens (M <= kSkinnyMaxM, K % 8 == 0) straight from the
// codes and params.
hipError_t launch_ttq_fwd_skinny(const uint16_t* x, const uint8_t* w_packed, const float* params, int64_t M,
                                 int64_t N, int64_t K, uint16_t* y, hipStream_t stream);
// The TTQ forward from the stored state (codes + params): the few-token
// kernel when it applies, else the codes expanded to wt at the start of the
// workspace and the bf16 GEMM. Workspace: ttq_codes_workspace_bytes().
size_t ttq_codes_workspace_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_ttq_fwd_codes(const uint16_t* x, const uint8_t* w_packed, const float* params, int64_t M,
                                int64_t N, int64_t K, uint16_t* y, void* ws, size_t ws_bytes, hipStream_t stream);
// y = x wt^T (bf16 x [M][K], no activation quantization).
hipError_t launch_ttq_fwd(const uint16_t* x, const uint16_t* wt, int64_t M, int64_t N, int64_t K, uint16_t* y,
                          void* ws, size_t ws_bytes, hipStream_t stream);
// dX = dY wt, dW = dY^T x (bf16 or f32), grads = {dL/dWp, dL/dWn} (NULL: not
// computed; needs dW). Workspace: gemm_workspace_bytes(kTtqBwd).
hipError_t launch_ttq_bwd(const uint16_t* dY, const uint16_t* x, const uint16_t* wt, const uint8_t* w_packed,
                          int64_t M, int64_t N, int64_t K, uint16_t* dX, void* dW, bool dw_f32, float* grads,
                          void* ws, size_t ws_bytes, hipStream_t stream);

}  // namespace bitnet
