/*
 * bitnet.h - C ABI of the MI355X (gfx950) BitLinear library, libbitnet.so.
 *
 * One BitNet b1.58 linear layer with ternary weights and int8 activations
 * (W1.58 / A8), for quantization-aware training: the weight ternarization
 * and 2-bit packing, the per-token int8 activation quantization, the INT8
 * forward GEMM and the straight-through-estimator (STE) backward GEMMs.
 * A TTQ variant (learned threshold and asymmetric scales, bf16 activations)
 * is declared at the end. The BitNet operations are those of the
 * "bitnet-qat-train" page (Hugging Face
 * kernels, phanerozoic): its opening bullets and its "Semantics" section,
 * with the quantizers of "bitlinear.py" (h4-polytopic-attention:
 * ternary_quantize, activation_quant_int8) and "1BitTraining.md" (Codys12
 * gist: weight_quant, activation_quant).
 *
 * Conventions for every entry point:
 *  - Tensors are dense and row-major. bf16 data is passed as its raw 16-bit
 *    patterns (uint16_t). Every array pointer is a DEVICE pointer and must be
 *    16-byte aligned, except `gamma` (4-byte aligned).
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Work is enqueued on it asynchronously; nothing synchronizes the host.
 *  - The caller owns every buffer (inputs, outputs, workspace) and keeps it
 *    alive until the stream work completes. The library allocates no device
 *    memory and keeps no pointer after it returns.
 *  - Arguments are validated before any launch; a validation failure returns
 *    its code and enqueues nothing. A failed launch returns BITNET_ERR_HIP.
 *  - Sizes are int64_t and must be >= 1 (M, N, K). Any K is accepted: the
 *    reduction axis of the int8 and 2-bit state is padded to
 *    Kp = bitnet_k_pad(K) (a multiple of 64) with zero codes and values;
 *    reductions and scales use the true K only.
 *  - Non-finite inputs (inf, NaN) give unspecified results.
 *  - Size limits (BITNET_ERR_SHAPE beyond them): M, N <= 2^30, K <= 2^24;
 *    for the GEMM entry points every operand the call reads among x_q,
 *    w_packed and dY satisfies (rows + 256) * row_bytes <= 2^31, i.e.
 *    (M + 256) * Kp, (N + 256) * Kp/4 and (M + 256) * 2N bytes, and with dW
 *    also (M + 256) * 2Kp for its bf16 x_hat, with dX also (Kp + 256) * Np/2
 *    for its fp4 transposed codes (Np = N rounded up to 64) (the kernels
 *    address them with 32-bit offsets); the forward also needs N <= 2^24
 *    (its epilogue addresses 32 output rows of up to 4-byte elements the
 *    same way).
 */
#ifndef BITNET_H
#define BITNET_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    BITNET_OK = 0,
    BITNET_ERR_NULL = 1,      /* a required pointer is NULL */
    BITNET_ERR_SHAPE = 2,     /* a size is < 1 or too large */
    BITNET_ERR_DTYPE = 3,     /* unsupported dtype enum */
    BITNET_ERR_ALIGN = 4,     /* a pointer is not aligned as required */
    BITNET_ERR_WORKSPACE = 5, /* workspace NULL or smaller than required */
    BITNET_ERR_HIP = 6        /* the HIP runtime reported an error */
} bitnet_status;

typedef enum {
    BITNET_BF16 = 0,
    BITNET_F32 = 1,
    BITNET_SIGN1 = 2  /* bitlinear_bwd's dW only: 1-bit signs (see there) */
} bitnet_dtype;

/* Human-readable name of a status code (static storage). */
const char* bitnet_status_string(bitnet_status status);

/* Padded reduction length: K rounded up to a multiple of 64 (K >= 1). */
int64_t bitnet_k_pad(int64_t K);

/* Bytes of workspace bitnet_ternarize_pack needs (fixed, a few KiB). */
size_t bitnet_ternarize_workspace_bytes(int64_t N, int64_t K);

/* Bytes of workspace bitlinear_fwd / bitlinear_bwd need for these sizes
 * (0 for sizes the call rejects). 0 means the call takes no workspace (the
 * pointer may then be NULL). The size is that of the plan the call runs on
 * the current device: a GEMM needs workspace when it splits output tiles
 * over several workgroups so that all CUs stay busy (16 bytes of tagged
 * counters per 256 x 256 output tile and 256 KiB per partial tile, at most
 * min(2G, G + T - 1) of them for G workgroups and T tiles); few tokens
 * (M <= 64) need none for the forward. The contents need no
 * initialization, and the calls leave the counters cleared, so a call
 * captured into a HIP graph may be replayed any number of times; a
 * workspace must not be shared by calls that may run at the same time
 * (calls on one stream may share it). bitlinear_bwd's size is that of its
 * call with both outputs; a call with one output uses the same size (its
 * split then uses fewer workgroups if it must). Each product first builds a
 * transient operand at the start of the workspace: dX the ternary codes
 * transposed to fp4 [Kp][Np/2] (Kp*Np/2 bytes, Np = N rounded up to 64), dW
 * a bf16 x_hat = bf16(x_q * s/127) [M][Kp] (2*M*Kp bytes); a call with
 * both outputs builds both, one after the other, in one launch. For at most
 * 64 tokens a bf16 or f32 dW converts its slices of x_hat itself and needs
 * no workspace, and a call with both outputs builds only the fp4 codes, in
 * the launch that also computes dW. */
size_t bitlinear_fwd_workspace_bytes(int64_t M, int64_t N, int64_t K);
size_t bitlinear_bwd_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * bitnet_ternarize_pack - per-tensor absmean scale, RoundClip ternarization
 * and 2-bit packing of the master weight ("bitnet-qat-train", opening
 * bullets: one fused ternarize, scale and pack pass; "bitlinear.py",
 * ternary_quantize; "1BitTraining.md", weight_quant). For bf16 W with K a
 * multiple of 64 and N*K up to about 25 M, W is read once: one launch holds
 * it in registers while its workgroups exchange their partial sums through
 * the workspace, then writes the codes. Otherwise a reduction pass over W
 * and a fused ternarize + pack pass. Both give the same bits.
 *
 *   gamma = max(fp32(S / (N*K)), 1e-8f), S = sum |W| accumulated in fp64 in
 *           a fixed order (bitwise deterministic across calls);
 *   q[n,k] = clip(round_half_even(W[n,k] / gamma), -1, 1), evaluated exactly
 *           (equivalently q = sign(w) if |w| > gamma/2, else 0).
 *
 * W         [N][K] master weights, bf16 bits (w_dtype BITNET_BF16) or float
 *           (BITNET_F32).
 * w_packed  [N][Kp/4] output bytes: row n holds Kp/16 little-endian 32-bit
 *           words of 16 codes; word w holds k = 16w..16w+15, the code of
 *           k = 16w + j at bit 8*(j%4) + 2*(j/4), as a 2-bit two's complement
 *           value: +1 = 0b01, 0 = 0b00, -1 = 0b11 (0b10 is never written).
 *           Padding codes (k >= K) are 0. (Byte b of a word holds the codes
 *           j = b, b+4, b+8, b+12, so (word >> 2t) & 0x03030303 gives the
 *           codes of k = 16w+4t..16w+4t+3 in its four bytes.)
 * gamma     [1] output float (device).
 * workspace device scratch of at least bitnet_ternarize_workspace_bytes();
 *           no initialization needed (the words that publish partial sums
 *           between workgroups carry a per-launch tag and sequence, so
 *           whatever the memory held never matches); clobbered. Calls that
 *           may run at the same time must not share a workspace.
 */
bitnet_status bitnet_ternarize_pack(const void* W, bitnet_dtype w_dtype,
                                    int64_t N, int64_t K,
                                    uint8_t* w_packed, float* gamma,
                                    void* workspace, size_t workspace_bytes,
                                    void* stream);

/*
 * bitnet_quantize - bitnet_ternarize_pack and bitnet_act_quant of one layer
 * step in one call, with the same results bit for bit (gamma, w_packed,
 * x_q, s_x). The activation rows are quantized in the weight's launch: in
 * the one-pass case each workgroup quantizes its share of the rows while
 * the others' partial sums arrive; otherwise the absmean pass and the rows
 * share one launch (two independent streams over W and x) and the codes are
 * packed after it. The two inputs share the reduction length K: W [N][K], x
 * [M][K]. Arguments, layouts and errors are those of the two calls;
 * workspace as bitnet_ternarize_pack's.
 */
bitnet_status bitnet_quantize(const void* W, bitnet_dtype w_dtype, int64_t N, int64_t K,
                              const uint16_t* x, int64_t M,
                              uint8_t* w_packed, float* gamma, int8_t* x_q, float* s_x,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * bitnet_quantize_static - bitnet_quantize for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): no workspace argument; the scratch
 * (the weight absmean's fp64 partial sums, and the one-pass launch's
 * per-workgroup records of partial and publication word) lives in a device
 * array of the library, 8192 bytes per GPU the library runs on, held until
 * the process ends. Results are bit for bit those of bitnet_quantize. The
 * array keeps the last call's contents; no call needs it cleared (partials
 * are written before they are read; publication words are tagged per launch
 * and never match a later launch's), but calls that may run at the same
 * time on one GPU race on it. Returns BITNET_ERR_WORKSPACE if a call would need more scratch
 * than the array holds (not the case for any size: the need is fixed at
 * bitnet_ternarize_workspace_bytes()), BITNET_ERR_HIP if the array's device
 * address cannot be obtained; otherwise the arguments and errors of
 * bitnet_quantize. Calls no allocating routine.
 */
bitnet_status bitnet_quantize_static(const void* W, bitnet_dtype w_dtype, int64_t N, int64_t K,
                                     const uint16_t* x, int64_t M,
                                     uint8_t* w_packed, float* gamma, int8_t* x_q, float* s_x,
                                     void* stream);

/*
 * bitnet_code_counts - how many weights each ternary value takes, for the
 * share of -1, 0 and +1 ("bitlinear.py", BitLinear.ternary_stats):
 *
 *   counts[0] = #{(n, k) : q[n,k] = -1},  counts[1] = #{(n, k) : q[n,k] = +1}
 *
 * over the true N x K weights (padding codes are 0 and count for neither;
 * the zeros are N*K - counts[0] - counts[1]).
 *
 * w_packed  [N][Kp/4] codes as written by bitnet_ternarize_pack (16-byte
 *           aligned).
 * counts    [2] uint64 output (device, 8-byte aligned).
 * No workspace. Exact and repeatable (a fixed summation order).
 */
bitnet_status bitnet_code_counts(const uint8_t* w_packed, int64_t N, int64_t K,
                                 uint64_t* counts, void* stream);

/*
 * bitnet_act_quant - per-token absmax int8 quantization ("bitlinear.py",
 * activation_quant_int8; "1BitTraining.md", activation_quant;
 * "bitnet-qat-train", opening paragraph).
 *
 *   s[m]      = max(max_k |x[m,k]|, 1e-8f)             (the row absmax)
 *   x_q[m,k]  = clip(round_half_even(127 * x[m,k] / s[m]), -127, 127),
 *               evaluated exactly.
 *
 * x    [M][K] bf16 bits.
 * x_q  [M][Kp] int8 output; columns K..Kp-1 are written as 0.
 * s_x  [M] float output: the floored absmax. The dequantization scale is
 *      s_x/127; it is applied where the int8 values are used.
 */
bitnet_status bitnet_act_quant(const uint16_t* x, int64_t M, int64_t K,
                               int8_t* x_q, float* s_x, void* stream);

/*
 * bitlinear_fwd - INT8 forward GEMM with exact INT32 accumulation and a
 * fused rescale ("bitnet-qat-train", Semantics):
 *
 *   acc[m,n] = sum_{k<Kp} x_q[m,k] * q[n,k]        (int32, exact)
 *   y[m,n]   = bf16_rne(acc[m,n] * (s_x[m]/127) * gamma)   (fp32 rescale)
 *
 * x_q, s_x  as written by bitnet_act_quant (x_q [M][Kp]).
 * w_packed, gamma as written by bitnet_ternarize_pack (w_packed [N][Kp/4]).
 * y        [M][N] bf16 bits output.
 * acc_out  [M][N] int32 output of the raw accumulators, or NULL (the
 *          production setting; it exists for bit-exact checks).
 * K        the true reduction length (Kp = bitnet_k_pad(K)).
 * workspace device scratch of bitlinear_fwd_workspace_bytes(M, N, K) bytes
 *          (NULL allowed when that is 0); clobbered.
 */
bitnet_status bitlinear_fwd(const int8_t* x_q, const float* s_x,
                            const uint8_t* w_packed, const float* gamma,
                            int64_t M, int64_t N, int64_t K,
                            uint16_t* y, int32_t* acc_out,
                            void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * bitlinear_fwd_bias - bitlinear_fwd with a bias added before the rounding
 * ("bitlinear.py", BitLinear: an optional bias, zero-initialised, added after
 * the product):
 *
 *   y[m,n] = bf16_rne(fp32(acc[m,n] * (s_x[m]/127) * gamma) + bias[n])
 *
 * (the product as in bitlinear_fwd, one fp32 add, one rounding). bias is
 * [N] bf16 bits, 16-byte aligned, or NULL (then identical to
 * bitlinear_fwd). Other arguments, the workspace and the errors are those
 * of bitlinear_fwd.
 */
bitnet_status bitlinear_fwd_bias(const int8_t* x_q, const float* s_x,
                                 const uint8_t* w_packed, const float* gamma,
                                 const uint16_t* bias,
                                 int64_t M, int64_t N, int64_t K,
                                 uint16_t* y, int32_t* acc_out,
                                 void* workspace, size_t workspace_bytes,
                                 void* stream);

/*
 * bitlinear_bias_grad - gradient of that bias: db[n] = sum_m dY[m,n], the
 * products of nothing but the bf16 values, summed in fp32 in a fixed order
 * (bitwise deterministic across calls) and rounded once to db_dtype.
 *
 * dY  [M][N] bf16 bits (16-byte aligned).
 * db  [N] output, BITNET_F32 or BITNET_BF16 bits (16-byte aligned).
 * No workspace.
 */
bitnet_status bitlinear_bias_grad(const uint16_t* dY, int64_t M, int64_t N,
                                  void* db, bitnet_dtype db_dtype, void* stream);

/*
 * bitlinear_bwd - straight-through-estimator backward with the operands
 * rebuilt from the saved 2-bit and int8 state ("bitnet-qat-train",
 * Semantics and opening bullets; gamma is treated as a constant):
 *
 *   dX[m,k] = sum_n dY[m,n] * W_hat[n,k],  W_hat = q * bf16_rne(gamma)
 *   dW[n,k] = sum_m dY[m,n] * x_hat[m,k],  x_hat = bf16_rne(x_q * s_x/127)
 *
 * Products are exact in fp32 (bf16 x bf16); sums accumulate in fp32; the
 * results are rounded once to the output dtype.
 *
 * dY        [M][N] bf16 bits.
 * x_q, s_x  saved activation state (x_q [M][Kp]); may be NULL if dW is NULL.
 * w_packed, gamma saved weight state; may be NULL if dX is NULL.
 * dX        [M][K] bf16 bits output, or NULL to skip the dX GEMM.
 * dW        [N][K] output in dW_dtype (BITNET_BF16 bits or BITNET_F32), or
 *           NULL to skip the dW GEMM. At least one of dX, dW is non-NULL.
 *           With BITNET_SIGN1, dW is [N][Kp/8] bytes of 1-bit signs for a
 *           sign-based optimiser ("1BitTraining.md", closing paragraphs: the
 *           identity-STE gradient has the sign of the gradient with respect
 *           to the quantised weight, so only 1 bit per weight is needed):
 *           bit j of byte b of row n is 1 iff the fp32 sum for dW[n, 8b + j]
 *           is negative, 0 otherwise (zero sums included); bits of k >= K
 *           are 0. No bf16 or f32 dW is written.
 * workspace device scratch of bitlinear_bwd_workspace_bytes(M, N, K) bytes
 *           (NULL allowed when that is 0); clobbered.
 */
bitnet_status bitlinear_bwd(const uint16_t* dY,
                            const int8_t* x_q, const float* s_x,
                            const uint8_t* w_packed, const float* gamma,
                            int64_t M, int64_t N, int64_t K,
                            uint16_t* dX, void* dW, bitnet_dtype dW_dtype,
                            void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * TTQ: trained ternary quantization ("TTQ_VERIFICATION.md", LabStrangeLoop
 * bitnet, summarising Zhu et al.), the variant with a learned threshold and
 * two learned scales per layer. params is a device float[3] =
 * {delta, Wp, Wn} (positive values; a caller that learns them through a
 * positivity transform passes the transformed values). Activations are the
 * layer's bf16 inputs, unquantized ("Bugs Fixed", item 4); the products run
 * on bf16 operands with fp32 accumulation. The quantized weight is kept as
 * its 2-bit codes (the w_packed format above) and as bf16 values
 * wt [N][Kp] = bf16(Wp), -bf16(Wn) or 0 (round half to even; padding 0).
 */

/* Bytes of workspace ttq_fwd and ttq_bwd need for these sizes (0 for sizes
 * they reject): the split-tile workspace of their GEMMs, as for
 * bitlinear_fwd, and for ttq_bwd 8 bytes per 128 x 128 tile of dW for the
 * scale-gradient partial sums. No initialization needed; graph replays are
 * safe; not shared by calls that may run at the same time. */
size_t ttq_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * ttq_init - the initial parameters (Algorithm Summary, Initialization,
 * Eq. 2): E = mean |W| computed exactly as bitnet_ternarize_pack's gamma
 * (the same bits, floor 1e-8 included), delta = fl32(0.7f * E) (one fp32
 * multiplication), Wp = Wn = E.
 *
 * W       [N][K] bf16 bits or float (w_dtype), 16-byte aligned.
 * params  [3] output float (device, 4-byte aligned).
 * workspace at least bitnet_ternarize_workspace_bytes(N, K); clobbered.
 */
bitnet_status ttq_init(const void* W, bitnet_dtype w_dtype, int64_t N, int64_t K,
                       float* params, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * ttq_quantize - Eq. 1 in one pass over W: code +1 where W > delta, -1
 * where W < -delta, 0 elsewhere (strict, exact comparisons).
 *
 * W         [N][K] bf16 bits or float (w_dtype).
 * params    [3] float (device): delta, Wp, Wn.
 * w_packed  [N][Kp/4] output codes (the bitnet_ternarize_pack format).
 * wt        [N][Kp] output bf16 bits: bf16(Wp), -bf16(Wn) or 0.
 * No workspace.
 */
bitnet_status ttq_quantize(const void* W, bitnet_dtype w_dtype, int64_t N, int64_t K,
                           const float* params, uint8_t* w_packed, uint16_t* wt,
                           void* stream);

/*
 * ttq_fwd - y[m,n] = sum_k x[m,k] * wt[n,k] (Eq. 1's weight applied to the
 * unquantized activations), fp32 sums rounded once to bf16.
 *
 * x   [M][K] bf16 bits.  wt [N][Kp] from ttq_quantize.  y [M][N] bf16 bits.
 * workspace ttq_workspace_bytes(M, N, K) bytes (NULL when that is 0).
 * Limits as for the GEMMs above, with (M + 256) * 2K and (N + 256) * 2Kp
 * bytes for x and wt.
 */
bitnet_status ttq_fwd(const uint16_t* x, const uint16_t* wt, int64_t M, int64_t N, int64_t K,
                      uint16_t* y, void* workspace, size_t workspace_bytes, void* stream);

/*
 * ttq_fwd_codes - the same forward from the stored state (the codes and
 * params, e.g. an exported layer): y[m,n] = sum_k x[m,k] * v(q[n,k]), with
 * v(+1) = bf16(Wp), v(-1) = -bf16(Wn), v(0) = 0, fp32 sums rounded once to
 * bf16. For few tokens (M <= 64, K % 8 == 0) one kernel reads the 2-bit
 * codes once and expands them in registers; otherwise the codes are
 * expanded to wt in the workspace and ttq_fwd's GEMM runs on it (the same
 * bits as ttq_fwd on ttq_quantize's wt).
 *
 * x         [M][K] bf16 bits.  w_packed [N][Kp/4] codes.  params [3] float
 *           (device, 4-byte aligned): delta (unused here), Wp, Wn.
 * y         [M][N] bf16 bits.
 * workspace ttq_fwd_codes_workspace_bytes(M, N, K) bytes: 0 (NULL allowed)
 *           when the few-token kernel applies, else 2*N*Kp for the expanded
 *           weight plus the GEMM's share; clobbered.
 * Limits as for ttq_fwd, and (N + 256) * Kp/4 bytes of codes.
 */
size_t ttq_fwd_codes_workspace_bytes(int64_t M, int64_t N, int64_t K);
bitnet_status ttq_fwd_codes(const uint16_t* x, const uint8_t* w_packed, const float* params,
                            int64_t M, int64_t N, int64_t K, uint16_t* y,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * ttq_bwd - the straight-through backward (Algorithm Summary, Backward
 * Pass; "Bugs Fixed", item 5):
 *
 *   dX[m,k] = sum_n dY[m,n] * wt[n,k]
 *   dW[n,k] = sum_m dY[m,n] * x[m,k]   (the latent weight's gradient is
 *                                       the quantized weight's, unchanged)
 *   grads[0] = dL/dWp =   sum of dW[n,k] over the codes +1
 *   grads[1] = dL/dWn = - sum of dW[n,k] over the codes -1
 *
 * The masked sums take the fp32 dW values before rounding, add them per
 * 128 x 128 tile in fp32 and across tiles in fp64, in a fixed order
 * (bitwise deterministic across calls), rounded once to fp32. delta gets no
 * gradient (the hard threshold has none).
 *
 * dY  [M][N] bf16 bits.  x [M][K] bf16 bits (needed for dW).
 * wt  from ttq_quantize (needed for dX); w_packed its codes (needed for
 *     grads).
 * dX  [M][K] bf16 bits output, or NULL.
 * dW  [N][K] output in dW_dtype (BITNET_BF16 or BITNET_F32), or NULL.
 * grads [2] float output (device, 4-byte aligned), or NULL; needs dW.
 * At least one of dX, dW is non-NULL.
 * workspace ttq_workspace_bytes(M, N, K) bytes; clobbered.
 */
bitnet_status ttq_bwd(const uint16_t* dY, const uint16_t* x, const uint16_t* wt,
                      const uint8_t* w_packed, int64_t M, int64_t N, int64_t K,
                      uint16_t* dX, void* dW, bitnet_dtype dW_dtype, float* grads,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Test hooks (for the library's own tests and tuning; not needed to use it).
 *
 * bitnet_set_test_knobs - process-wide knobs read by every later launch:
 *   split_ctas  0: the cost model chooses how output tiles are shared out;
 *               > 0: every large-M GEMM splits its tiles over that many
 *               workgroups (at most 256; no paired backward launch);
 *               < 0: whole tiles only.
 *   pair_cols   0: the cost model; k >= 1: a paired backward launch gives
 *               dX k of its 8-workgroup columns.
 *   no_skinny   nonzero: the large-M GEMMs also for M <= 64 (workspace
 *               sizes queried while it is set cover that route).
 *   spin_limit  polls (each a short sleep) before a workgroup waiting for
 *               another's partial tile gives up; the default,
 *               bitnet_default_spin_limit(), is about a second. A wait
 *               that gives up writes its output tile as NaN (int32
 *               accumulators: INT32_MIN) and is counted.
 *               The one-pass weight quantization waits at most the same
 *               number of polls, and at most 200 us, for the other
 *               workgroups' partial sums; when it gives up, a workgroup
 *               computes the missing sums itself (same results, more reads
 *               of W) and counts each.
 * bitnet_split_timeouts - the number of such waits that gave up on the
 *   current device since the last call (then reset to 0). Synchronizes the
 *   device. BITNET_ERR_HIP if the runtime fails.
 * bitnet_quantize_recomputes - the number of partial sums one-pass
 *   launches computed themselves on the current device since the last call
 *   (then reset to 0). Synchronizes the device.
 * bitnet_debug_split_pieces - the pieces a split launch of `tiles` tiles of
 *   `stages` reduction stages over `grid` workgroups (grid <= tiles*stages)
 *   runs, computed on the host by the functions the kernels use: for each
 *   piece in workgroup order, its virtual workgroup v, tile t, stages
 *   [s0, s1), partial-tile slot, and the first workgroup va and piece count
 *   n of its tile. Writes at most cap entries per array; returns the number
 *   of pieces, or -1 for invalid arguments. bitnet_debug_partial_slots: the
 *   slot count the plan reserves. bitnet_debug_cta_order: the virtual index
 *   of each of `grid` workgroups (workgroup b runs on XCD b % 8; each XCD
 *   gets a contiguous range).
 * bitnet_debug_mfma_probe - enqueues one launch of register-only MFMA chains
 *   on every SIMD (int8 != 0: v_mfma_i32_32x32x32_i8, else
 *   v_mfma_f32_32x32x16_bf16), `iters` rounds (1 .. 2^24), and stores in
 *   *ops (host) the operations it performs; timing it gives the MFMA rate
 *   the chip sustains under a full load. sink: device float[2048] (not
 *   written in practice).
 */
void bitnet_set_test_knobs(int split_ctas, int pair_cols, int no_skinny, uint32_t spin_limit);
uint32_t bitnet_default_spin_limit(void);
bitnet_status bitnet_split_timeouts(uint32_t* count);
bitnet_status bitnet_quantize_recomputes(uint32_t* count);
int64_t bitnet_debug_split_pieces(int64_t tiles, int32_t stages, int32_t grid, int32_t* v, int32_t* t,
                                  int32_t* s0, int32_t* s1, int64_t* slot, int32_t* va, int32_t* n,
                                  int64_t cap);
int32_t bitnet_debug_partial_slots(int64_t tiles, int32_t grid);
void bitnet_debug_cta_order(int32_t grid, int32_t* out);
bitnet_status bitnet_debug_mfma_probe(int32_t int8, int32_t iters, float* sink, double* ops, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BITNET_H */
