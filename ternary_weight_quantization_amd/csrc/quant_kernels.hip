// Quantization kernels for gfx950: weight absmean + ternarize + 2-bit pack,
// and per-token absmax int8 activation quantization. Both are HBM-bound
// streaming passes: 16-byte loads, one pass over each input where possible.
//
// Weights ("bitnet-qat-train", opening bullets: one fused ternarize, scale
// and pack pass; "bitlinear.py", ternary_quantize; "1BitTraining.md",
// weight_quant):
//   gamma   = max(fp32(S / (N*K)), 1e-8),  S = sum |W| in fp64
//   q[n,k]  = clip(RNE(W/gamma), -1, 1)  ==  sign(w) * [|w| > gamma/2]
// The threshold form is exact: gamma/2 is exact in fp32, both sides are
// exact fp32 values, and RNE sends |W/gamma| == 1/2 to 0, (1/2, 3/2) to 1
// and [3/2, inf) to >= 2, which clips to 1.
//
// Activations ("bitlinear.py", activation_quant_int8; "1BitTraining.md",
// activation_quant):
//   s[m]    = max(max_k |x[m,k]|, 1e-8)
//   x_q     = clip(RNE(127 x / s), -127, 127), exactly.

#include "device_common.h"
#include "internal.h"

namespace bitnet {

// ---------------------------------------------------------------------------
// absmean, phase 1: fixed-grid fp64 partial sums of |W|
// ---------------------------------------------------------------------------

template <bool F32>
__device__ __forceinline__ double abs_sum16(uint4 v) {
  if constexpr (F32) {
    const double a = fabs((double)__uint_as_float(v.x));
    const double b = fabs((double)__uint_as_float(v.y));
    const double c = fabs((double)__uint_as_float(v.z));
    const double d = fabs((double)__uint_as_float(v.w));
    return (a + b) + (c + d);
  } else {
    const uint32_t x = v.x & 0x7FFF7FFFu, y = v.y & 0x7FFF7FFFu;
    const uint32_t z = v.z & 0x7FFF7FFFu, w = v.w & 0x7FFF7FFFu;
    const double s0 = (double)bf16_lo(x) + (double)bf16_hi(x);
    const double s1 = (double)bf16_lo(y) + (double)bf16_hi(y);
    const double s2 = (double)bf16_lo(z) + (double)bf16_hi(z);
    const double s3 = (double)bf16_lo(w) + (double)bf16_hi(w);
    return (s0 + s1) + (s2 + s3);
  }
}

template <bool F32>
__device__ __forceinline__ float load_elem(const void* w, int64_t i) {
  if constexpr (F32) return static_cast<const float*>(w)[i];
  else return bf16_to_f32(static_cast<const uint16_t*>(w)[i]);
}

template <bool F32>
__global__ __launch_bounds__(kAbsmeanThreads) void absmean_partials_kernel(
    const void* __restrict__ w, int64_t n, double* __restrict__ partials) {
  constexpr int kVec = F32 ? 4 : 8;  // elements per 16 bytes
  constexpr int kUnroll = 8;
  const uint4* wv = static_cast<const uint4*>(w);
  const int64_t nvec = n / kVec;
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;

  double acc[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) acc[u] = 0.0;
  int64_t i = tid;
  for (; i + (kUnroll - 1) * stride < nvec; i += kUnroll * stride) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = wv[i + u * stride];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc[u] += abs_sum16<F32>(v[u]);
  }
  for (; i < nvec; i += stride) acc[0] += abs_sum16<F32>(wv[i]);
  const int64_t tail = nvec * kVec;
  if (tid < n - tail) acc[1] += fabs((double)load_elem<F32>(w, tail + tid));

  double v = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
  v = wave_sum_f64(v);
  __shared__ double sw[kAbsmeanThreads / kWave];
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  if (lane == 0) sw[wave] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
#pragma unroll
    for (int j = 0; j < kAbsmeanThreads / kWave; ++j) t += sw[j];
    partials[blockIdx.x] = t;
  }
}

// ---------------------------------------------------------------------------
// absmean, phase 2 + ternarize + pack. Every block reduces the fixed set of
// partials in the same order, so all blocks hold the same gamma; block 0
// stores it. Each thread then writes whole 32-bit words of 16 codes.
// ---------------------------------------------------------------------------

// The 16 weights W[n][k0 .. k0+15] of one code word as fp32 (exact), zeros
// past K. VEC: every row starts 16-byte aligned (K a multiple of 4 for fp32,
// of 8 for bf16).
template <bool F32, bool VEC>
__device__ __forceinline__ void load_word(const void* __restrict__ w, int64_t n, int64_t K, int64_t k0,
                                          float (&vals)[16]) {
  if (VEC && k0 + 16 <= K) {
    if constexpr (F32) {
      const uint4* p = reinterpret_cast<const uint4*>(static_cast<const float*>(w) + n * K + k0);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint4 d = p[c];
        vals[4 * c + 0] = __uint_as_float(d.x);
        vals[4 * c + 1] = __uint_as_float(d.y);
        vals[4 * c + 2] = __uint_as_float(d.z);
        vals[4 * c + 3] = __uint_as_float(d.w);
      }
    } else {
      const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(w) + n * K + k0);
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const uint4 d = p[c];
        vals[8 * c + 0] = bf16_lo(d.x); vals[8 * c + 1] = bf16_hi(d.x);
        vals[8 * c + 2] = bf16_lo(d.y); vals[8 * c + 3] = bf16_hi(d.y);
        vals[8 * c + 4] = bf16_lo(d.z); vals[8 * c + 5] = bf16_hi(d.z);
        vals[8 * c + 6] = bf16_lo(d.w); vals[8 * c + 7] = bf16_hi(d.w);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int64_t k = k0 + j;
      vals[j] = (k < K) ? load_elem<F32>(w, n * K + k) : 0.0f;
    }
  }
}

constexpr int kPackThreads = 256;
static_assert(kAbsmeanBlocks == kPackThreads, "one partial per thread");
static_assert(kPackThreads / kWave == 4, "four wave sums");

// S = the sum of the kAbsmeanBlocks partials in one fixed order (butterfly
// within each wave, then the four wave sums pairwise), so every block and
// kernel that needs it gets the same bits. Called by all kPackThreads
// threads of the block.
__device__ __forceinline__ double partials_total(const double* __restrict__ partials, double* sred) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const double v = wave_sum_f64(partials[threadIdx.x]);
  if (lane == 0) sred[wave] = v;
  __syncthreads();
  return (sred[0] + sred[1]) + (sred[2] + sred[3]);
}

template <bool F32, bool VEC>
__global__ __launch_bounds__(kPackThreads) void ternarize_pack_kernel(
    const void* __restrict__ w, int64_t N, int64_t K, int64_t words_per_row,
    const double* __restrict__ partials, uint32_t* __restrict__ packed,
    float* __restrict__ gamma_out) {
  __shared__ double sred[kPackThreads / kWave];
  __shared__ float s_half;
  const double S = partials_total(partials, sred);
  if (threadIdx.x == 0) {
    const double mean = S / (double)(N * K);
    const float g = fmaxf((float)mean, 1e-8f);
    s_half = g * 0.5f;  // exact
    if (blockIdx.x == 0) *gamma_out = g;
  }
  __syncthreads();
  const float h = s_half;

  const int64_t total = N * words_per_row;
  for (int64_t wi = (int64_t)blockIdx.x * kPackThreads + threadIdx.x; wi < total;
       wi += (int64_t)gridDim.x * kPackThreads) {
    const int64_t n = wi / words_per_row;
    const int64_t k0 = (wi - n * words_per_row) * 16;
    float vals[16];
    load_word<F32, VEC>(w, n, K, k0, vals);
    // code j of the word at bit 8*(j%4) + 2*(j/4): byte b holds the codes
    // j = b, b+4, b+8, b+12, so (word >> 2t) & 0x03030303 lists the codes
    // 4t..4t+3 in its four bytes
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t code = (vals[j] > h) ? 1u : ((vals[j] < -h) ? 3u : 0u);
      word |= code << (8 * (j & 3) + 2 * (j >> 2));
    }
    packed[wi] = word;
  }
}

hipError_t launch_ternarize_pack(const void* W, bool w_is_f32, int64_t N, int64_t K,
                                 uint8_t* w_packed, float* gamma, double* partials,
                                 hipStream_t stream) {
  const int64_t n = N * K;
  if (w_is_f32)
    absmean_partials_kernel<true><<<kAbsmeanBlocks, kAbsmeanThreads, 0, stream>>>(W, n, partials);
  else
    absmean_partials_kernel<false><<<kAbsmeanBlocks, kAbsmeanThreads, 0, stream>>>(W, n, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  const int64_t wpr = k_pad(K) / 16;
  const int64_t total = N * wpr;
  const int64_t want = (total + kPackThreads - 1) / kPackThreads;
  const int grid = (int)(want < 2048 ? want : 2048);
  uint32_t* pw = reinterpret_cast<uint32_t*>(w_packed);
  const bool vec = w_is_f32 ? (K % 4 == 0) : (K % 8 == 0);
  if (w_is_f32) {
    if (vec) ternarize_pack_kernel<true, true><<<grid, kPackThreads, 0, stream>>>(W, N, K, wpr, partials, pw, gamma);
    else ternarize_pack_kernel<true, false><<<grid, kPackThreads, 0, stream>>>(W, N, K, wpr, partials, pw, gamma);
  } else {
    if (vec) ternarize_pack_kernel<false, true><<<grid, kPackThreads, 0, stream>>>(W, N, K, wpr, partials, pw, gamma);
    else ternarize_pack_kernel<false, false><<<grid, kPackThreads, 0, stream>>>(W, N, K, wpr, partials, pw, gamma);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Activation quantization
// ---------------------------------------------------------------------------

// RNE(127 x / s) for |x| <= s, exactly, returned as the fp32 value
// 1.5 * 2^23 + q, whose low byte is q as a two's complement int8.
// Fast path: p = x * fl(127/s) is within 127 * 2^-23 (< 1.6e-5) of the
// exact quotient Q, so when p is more than 2^-15 away from the nearest
// half-integer, the integer nearest to p is the one nearest to Q and no tie
// is possible; adding 1.5 * 2^23 rounds p to that integer (RNE, |p| < 2^22)
// and subtracting it again is exact. Otherwise Q is recomputed as an fp64
// quotient of exact operands, whose rounding error (< 2^-46) is far below
// the smallest nonzero distance of Q from a half-integer (> 2^-33 for fp32
// operands), so rint of it is exact, ties included. No clamp is needed:
// |x| <= s gives |p| <= 127 (1 + 2^-24) and |Q| <= 127.
constexpr float kRoundMagic = 12582912.0f;  // 1.5 * 2^23

__device__ __forceinline__ float quant1(float xv, float r127, float s) {
  const float p = xv * r127;
  const float t = p + kRoundMagic;
  if (fabsf(p - (t - kRoundMagic)) > 0.49996948f) {  // 0.5 - 2^-15
    const double q = __builtin_rint(127.0 * (double)xv / (double)s);
    return (float)q + kRoundMagic;
  }
  return t;
}

// Low bytes of four quant1 results -> four int8 in one word (a's lowest).
__device__ __forceinline__ uint32_t pack_i8x4(float a, float b, float c, float d) {
  const uint32_t lo = perm(__float_as_uint(b), __float_as_uint(a), 0x0C0C0400u);
  const uint32_t hi = perm(__float_as_uint(d), __float_as_uint(c), 0x0C0C0400u);
  return perm(hi, lo, 0x05040100u);
}

// quant1 over the 8 values of a chunk: the fast results and one flag for
// the chunk, then (rarely) the exact recompute of the flagged values, so
// that the common path has no branch per value. Same decisions and results
// as quant1 value by value.
__device__ __forceinline__ uint2 quant8(uint4 v, float r127, float s) {
  const float x[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                      bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
  float t[8];
  bool slow = false;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float p = x[e] * r127;
    t[e] = p + kRoundMagic;
    slow |= fabsf(p - (t[e] - kRoundMagic)) > 0.49996948f;
  }
  if (slow) {
#pragma unroll
    for (int e = 0; e < 8; ++e) t[e] = quant1(x[e], r127, s);
  }
  return make_uint2(pack_i8x4(t[0], t[1], t[2], t[3]), pack_i8x4(t[4], t[5], t[6], t[7]));
}

__device__ __forceinline__ float absmax8(uint4 v) {
  const float a = fmaxf(fmaxf(fabsf(bf16_lo(v.x)), fabsf(bf16_hi(v.x))),
                        fmaxf(fabsf(bf16_lo(v.y)), fabsf(bf16_hi(v.y))));
  const float b = fmaxf(fmaxf(fabsf(bf16_lo(v.z)), fabsf(bf16_hi(v.z))),
                        fmaxf(fabsf(bf16_lo(v.w)), fabsf(bf16_hi(v.w))));
  return fmaxf(a, b);
}

// Loads the 8 bf16 of chunk `ch` of a row (zeros past K).
template <bool VEC>
__device__ __forceinline__ uint4 load_chunk(const uint16_t* xr, int64_t ch, int64_t K) {
  const int64_t k0 = ch * 8;
  if (VEC && k0 + 8 <= K) return *reinterpret_cast<const uint4*>(xr + k0);
  uint32_t d[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t k = k0 + 2 * j;
    const uint32_t lo = (k < K) ? xr[k] : 0u;
    const uint32_t hi = (k + 1 < K) ? xr[k + 1] : 0u;
    d[j] = lo | (hi << 16);
  }
  return make_uint4(d[0], d[1], d[2], d[3]);
}

// TPR threads (whole waves) per row, CPT chunks of 8 values per thread kept
// in registers: one HBM read of x, one write of x_q.
template <int TPR, int CPT, bool VEC>
__global__ __launch_bounds__(256) void act_quant_kernel(const uint16_t* __restrict__ x, int64_t M,
                                                        int64_t K, int64_t Kp,
                                                        int8_t* __restrict__ xq,
                                                        float* __restrict__ s_out) {
  static_assert(TPR % kWave == 0 && 256 % TPR == 0, "whole waves per row");
  constexpr int RPB = 256 / TPR;
  constexpr int WPR = TPR / kWave;
  __shared__ float smax[256 / kWave];
  const int r_local = threadIdx.x / TPR;
  const int t = threadIdx.x % TPR;
  const int64_t row = (int64_t)blockIdx.x * RPB + r_local;
  const bool row_ok = row < M;
  const int64_t nchunks = Kp / 8;
  const uint16_t* xr = x + row * K;

  uint4 v[CPT];
  float amax = 0.0f;
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int64_t ch = t + (int64_t)c * TPR;
    v[c] = (row_ok && ch * 8 < K) ? load_chunk<VEC>(xr, ch, K) : make_uint4(0, 0, 0, 0);
    amax = fmaxf(amax, absmax8(v[c]));
  }
  amax = wave_max_f32(amax);
  if constexpr (WPR > 1) {
    if (threadIdx.x % kWave == 0) smax[threadIdx.x / kWave] = amax;
    __syncthreads();
    const int w0 = r_local * WPR;
    amax = smax[w0];
#pragma unroll
    for (int j = 1; j < WPR; ++j) amax = fmaxf(amax, smax[w0 + j]);
  }
  const float s = fmaxf(amax, 1e-8f);
  if (row_ok && t == 0) s_out[row] = s;
  const float r127 = 127.0f / s;
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int64_t ch = t + (int64_t)c * TPR;
    if (row_ok && ch < nchunks)
      *reinterpret_cast<uint2*>(xq + row * Kp + ch * 8) = quant8(v[c], r127, s);
  }
}

// Rows longer than the register-resident variant allows: two passes over the
// row (the second read is served by the caches).
template <bool VEC>
__global__ __launch_bounds__(256) void act_quant_long_kernel(const uint16_t* __restrict__ x,
                                                             int64_t M, int64_t K, int64_t Kp,
                                                             int8_t* __restrict__ xq,
                                                             float* __restrict__ s_out) {
  __shared__ float smax[256 / kWave];
  const int64_t row = blockIdx.x;
  const uint16_t* xr = x + row * K;
  const int64_t nchunks = Kp / 8;
  float amax = 0.0f;
  for (int64_t ch = threadIdx.x; ch * 8 < K; ch += 256) amax = fmaxf(amax, absmax8(load_chunk<VEC>(xr, ch, K)));
  amax = wave_max_f32(amax);
  if (threadIdx.x % kWave == 0) smax[threadIdx.x / kWave] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(smax[0], smax[1]), fmaxf(smax[2], smax[3]));
  const float s = fmaxf(amax, 1e-8f);
  if (threadIdx.x == 0) s_out[row] = s;
  const float r127 = 127.0f / s;
  for (int64_t ch = threadIdx.x; ch < nchunks; ch += 256) {
    const uint4 v = (ch * 8 < K) ? load_chunk<VEC>(xr, ch, K) : make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint2*>(xq + row * Kp + ch * 8) = quant8(v, r127, s);
  }
}

template <int TPR, bool VEC>
static void launch_aq_tpr(int cpt, const uint16_t* x, int64_t M, int64_t K, int64_t Kp,
                          int8_t* xq, float* s, hipStream_t st) {
  const int grid = (int)((M + (256 / TPR) - 1) / (256 / TPR));
  switch (cpt) {
    case 1: act_quant_kernel<TPR, 1, VEC><<<grid, 256, 0, st>>>(x, M, K, Kp, xq, s); break;
    case 2: act_quant_kernel<TPR, 2, VEC><<<grid, 256, 0, st>>>(x, M, K, Kp, xq, s); break;
    case 3: act_quant_kernel<TPR, 3, VEC><<<grid, 256, 0, st>>>(x, M, K, Kp, xq, s); break;
    case 4: act_quant_kernel<TPR, 4, VEC><<<grid, 256, 0, st>>>(x, M, K, Kp, xq, s); break;
    case 5: act_quant_kernel<TPR, 5, VEC><<<grid, 256, 0, st>>>(x, M, K, Kp, xq, s); break;
    case 6: act_quant_kernel<TPR, 6, VEC><<<grid, 256, 0, st>>>(x, M, K, Kp, xq, s); break;
    case 7: act_quant_kernel<TPR, 7, VEC><<<grid, 256, 0, st>>>(x, M, K, Kp, xq, s); break;
    default: act_quant_kernel<TPR, 8, VEC><<<grid, 256, 0, st>>>(x, M, K, Kp, xq, s); break;
  }
}

template <bool VEC>
static void launch_aq(const uint16_t* x, int64_t M, int64_t K, int64_t Kp, int8_t* xq, float* s,
                      hipStream_t st) {
  const int64_t nchunks = Kp / 8;
  if (nchunks <= 64 * 8) {
    launch_aq_tpr<64, VEC>((int)((nchunks + 63) / 64), x, M, K, Kp, xq, s, st);
  } else if (nchunks <= 128 * 8) {
    launch_aq_tpr<128, VEC>((int)((nchunks + 127) / 128), x, M, K, Kp, xq, s, st);
  } else if (nchunks <= 256 * 8) {
    launch_aq_tpr<256, VEC>((int)((nchunks + 255) / 256), x, M, K, Kp, xq, s, st);
  } else {
    act_quant_long_kernel<VEC><<<(int)M, 256, 0, st>>>(x, M, K, Kp, xq, s);
  }
}

hipError_t launch_act_quant(const uint16_t* x, int64_t M, int64_t K, int8_t* x_q, float* s_x,
                            hipStream_t stream) {
  const int64_t Kp = k_pad(K);
  if (K % 8 == 0) launch_aq<true>(x, M, K, Kp, x_q, s_x, stream);
  else launch_aq<false>(x, M, K, Kp, x_q, s_x, stream);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Bias gradient ("bitlinear.py", BitLinear: the optional bias is added after
// the product, so its gradient is the token sum of dY): db[n] = sum_m dY[m][n]
// in fp32, in a fixed order. A block of 1024 threads owns 64 columns: thread
// (g = t / 8, c = t % 8) sums rows g, g + 128, ... of columns 8c .. 8c+7 in
// row order (16-byte loads; a wave covers 8 rows x 128 bytes), then the 128
// row groups' partial sums are added in group order.
// ---------------------------------------------------------------------------

constexpr int kBiasGroups = 128;

__global__ __launch_bounds__(1024) void bias_grad_kernel(const uint16_t* __restrict__ dY, int64_t M, int64_t N,
                                                         void* __restrict__ db, bool f32) {
  __shared__ float part[kBiasGroups][64 + 1];
  const int t = threadIdx.x, g = t >> 3, c = t & 7;
  const int64_t n0 = (int64_t)blockIdx.x * 64 + 8 * c;
  float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  if (N % 8 == 0) {
    if (n0 < N) {
#pragma unroll 8
      for (int64_t m = g; m < M; m += kBiasGroups) {
        const uint4 v = *reinterpret_cast<const uint4*>(dY + m * N + n0);
        acc[0] += bf16_lo(v.x); acc[1] += bf16_hi(v.x); acc[2] += bf16_lo(v.y); acc[3] += bf16_hi(v.y);
        acc[4] += bf16_lo(v.z); acc[5] += bf16_hi(v.z); acc[6] += bf16_lo(v.w); acc[7] += bf16_hi(v.w);
      }
    }
  } else {
    for (int64_t m = g; m < M; m += kBiasGroups)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (n0 + e < N) acc[e] += bf16_to_f32(dY[m * N + n0 + e]);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[g][8 * c + e] = acc[e];
  __syncthreads();
  if (t < 64) {
    float sum = 0.0f;
    for (int i = 0; i < kBiasGroups; ++i) sum += part[i][t];
    const int64_t n = (int64_t)blockIdx.x * 64 + t;
    if (n < N) {
      if (f32) static_cast<float*>(db)[n] = sum;
      else static_cast<uint16_t*>(db)[n] = f32_to_bf16_bits(sum);
    }
  }
}

hipError_t launch_bias_grad(const uint16_t* dY, int64_t M, int64_t N, void* db, bool db_is_f32,
                            hipStream_t stream) {
  bias_grad_kernel<<<(unsigned)((N + 63) / 64), 1024, 0, stream>>>(dY, M, N, db, db_is_f32);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// TTQ ("TTQ_VERIFICATION.md", Algorithm Summary): Eq. 1 takes +Wp where
// W > delta, -Wn where W < -delta and 0 elsewhere; the initialization (Eq. 2)
// sets delta = 0.7 E|W| and Wp = Wn = E|W|. params = {delta, Wp, Wn}, fp32,
// on the device.
// ---------------------------------------------------------------------------

// Initialization from the absmean partials: E is gamma's value (the same
// reduction in the same order, the same floor), delta = fl32(0.7f * E).
__global__ __launch_bounds__(kPackThreads) void ttq_init_kernel(const double* __restrict__ partials,
                                                                 int64_t count, float* __restrict__ params) {
  __shared__ double sred[kPackThreads / kWave];
  const double S = partials_total(partials, sred);
  if (threadIdx.x == 0) {
    const float e = fmaxf((float)(S / (double)count), 1e-8f);
    params[0] = 0.7f * e;
    params[1] = e;
    params[2] = e;
  }
}

hipError_t launch_ttq_init(const void* W, bool w_is_f32, int64_t N, int64_t K, float* params, double* partials,
                           hipStream_t stream) {
  const int64_t n = N * K;
  if (w_is_f32)
    absmean_partials_kernel<true><<<kAbsmeanBlocks, kAbsmeanThreads, 0, stream>>>(W, n, partials);
  else
    absmean_partials_kernel<false><<<kAbsmeanBlocks, kAbsmeanThreads, 0, stream>>>(W, n, partials);
  if (hipError_t e = hipGetLastError()) return e;
  ttq_init_kernel<<<1, kPackThreads, 0, stream>>>(partials, n, params);
  return hipGetLastError();
}

// Eq. 1 on one pass over W: per 16-weight word, the 2-bit codes (the BitNet
// format: +1 -> 01, -1 -> 11, 0 -> 00 at bit 8*(j%4) + 2*(j/4)) and the bf16
// values the products use, bf16(Wp), -bf16(Wn) or 0 (round half to even),
// into wt [N][Kp] (padding columns 0). Both comparisons are strict and exact
// (fp32 weights or bf16 weights widened exactly, fp32 delta).
template <bool F32, bool VEC>
__global__ __launch_bounds__(kPackThreads) void ttq_quantize_kernel(
    const void* __restrict__ w, int64_t N, int64_t K, int64_t words_per_row, const float* __restrict__ params,
    uint32_t* __restrict__ packed, uint16_t* __restrict__ wt) {
  const float d = params[0];
  const uint32_t vp = f32_to_bf16_bits(params[1]);
  const uint32_t vn = f32_to_bf16_bits(params[2]) ^ 0x8000u;  // -bf16(Wn)
  const int64_t total = N * words_per_row, Kp = 16 * words_per_row;
  for (int64_t wi = (int64_t)blockIdx.x * kPackThreads + threadIdx.x; wi < total;
       wi += (int64_t)gridDim.x * kPackThreads) {
    const int64_t n = wi / words_per_row;
    const int64_t k0 = (wi - n * words_per_row) * 16;
    float vals[16];
    load_word<F32, VEC>(w, n, K, k0, vals);
    uint32_t word = 0, o[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const bool pos = vals[j] > d, neg = vals[j] < -d;
      word |= (pos ? 1u : (neg ? 3u : 0u)) << (8 * (j & 3) + 2 * (j >> 2));
      o[j >> 1] |= (pos ? vp : (neg ? vn : 0u)) << (16 * (j & 1));
    }
    packed[wi] = word;
    uint4* dst = reinterpret_cast<uint4*>(wt + n * Kp + k0);
    dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
    dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
  }
}

// The bf16 values of Eq. 1 from stored codes (the exported state): wt
// [N][Kp] = bf16(Wp), -bf16(Wn) or 0 per code, as ttq_quantize writes them.
__global__ __launch_bounds__(kPackThreads) void ttq_expand_kernel(const uint32_t* __restrict__ packed, int64_t N,
                                                                   int64_t words_per_row,
                                                                   const float* __restrict__ params,
                                                                   uint16_t* __restrict__ wt) {
  const uint32_t vp = f32_to_bf16_bits(params[1]);
  const uint32_t vn = f32_to_bf16_bits(params[2]) ^ 0x8000u;
  const int64_t total = N * words_per_row, Kp = 16 * words_per_row;
  for (int64_t wi = (int64_t)blockIdx.x * kPackThreads + threadIdx.x; wi < total;
       wi += (int64_t)gridDim.x * kPackThreads) {
    const int64_t n = wi / words_per_row;
    const int64_t k0 = (wi - n * words_per_row) * 16;
    const uint32_t word = packed[wi];
    uint32_t o[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t c = (word >> (8 * (j & 3) + 2 * (j >> 2))) & 3u;
      o[j >> 1] |= (c == 1u ? vp : (c == 3u ? vn : 0u)) << (16 * (j & 1));
    }
    uint4* dst = reinterpret_cast<uint4*>(wt + n * Kp + k0);
    dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
    dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
  }
}

hipError_t launch_ttq_expand(const uint8_t* w_packed, int64_t N, int64_t K, const float* params, uint16_t* wt,
                             hipStream_t stream) {
  const int64_t wpr = k_pad(K) / 16;
  const int64_t want = (N * wpr + kPackThreads - 1) / kPackThreads;
  const int grid = (int)(want < 2048 ? want : 2048);
  ttq_expand_kernel<<<grid, kPackThreads, 0, stream>>>(reinterpret_cast<const uint32_t*>(w_packed), N, wpr, params,
                                                       wt);
  return hipGetLastError();
}

hipError_t launch_ttq_quantize(const void* W, bool w_is_f32, int64_t N, int64_t K, const float* params,
                               uint8_t* w_packed, uint16_t* wt, hipStream_t stream) {
  const int64_t wpr = k_pad(K) / 16;
  const int64_t want = (N * wpr + kPackThreads - 1) / kPackThreads;
  const int grid = (int)(want < 2048 ? want : 2048);
  uint32_t* pw = reinterpret_cast<uint32_t*>(w_packed);
  const bool vec = w_is_f32 ? (K % 4 == 0) : (K % 8 == 0);
  if (w_is_f32) {
    if (vec) ttq_quantize_kernel<true, true><<<grid, kPackThreads, 0, stream>>>(W, N, K, wpr, params, pw, wt);
    else ttq_quantize_kernel<true, false><<<grid, kPackThreads, 0, stream>>>(W, N, K, wpr, params, pw, wt);
  } else {
    if (vec) ttq_quantize_kernel<false, true><<<grid, kPackThreads, 0, stream>>>(W, N, K, wpr, params, pw, wt);
    else ttq_quantize_kernel<false, false><<<grid, kPackThreads, 0, stream>>>(W, N, K, wpr, params, pw, wt);
  }
  return hipGetLastError();
}

}  // namespace bitnet
