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

// Partial sum b of the fixed grid: thread t of the kAbsmeanThreads of block
// b reads the 16-byte vectors b * kAbsmeanThreads + t + j * stride (stride =
// kAbsmeanBlocks * kAbsmeanThreads, the whole grid), 8 loads in flight, and
// the block adds its threads' sums in a fixed tree. The order depends only
// on the grid constants, never on the launch, so every kernel that runs
// this body (alone or next to other work) gives gamma the same bits.
template <bool F32>
__device__ __forceinline__ double absmean_thread_sum(const void* __restrict__ w, int64_t n, int b) {
  constexpr int kVec = F32 ? 4 : 8;  // elements per 16 bytes
  constexpr int kUnroll = 8;
  const uint4* wv = static_cast<const uint4*>(w);
  const int64_t nvec = n / kVec;
  const int64_t tid = (int64_t)b * kAbsmeanThreads + threadIdx.x;
  constexpr int64_t stride = (int64_t)kAbsmeanBlocks * kAbsmeanThreads;

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
  return ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
}

// The block's thread sums -> its partial: a butterfly within each wave, then
// thread 0 adds the wave sums in wave order. The partial is returned in
// thread 0 (the other threads get 0). Called by all kAbsmeanThreads threads;
// a caller that runs it again in the same block separates the two calls
// with a barrier.
__device__ __forceinline__ double absmean_block_reduce(double v) {
  v = wave_sum_f64(v);
  __shared__ double sw[kAbsmeanThreads / kWave];
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  if (lane == 0) sw[wave] = v;
  __syncthreads();
  double t = 0.0;
  if (threadIdx.x == 0) {
#pragma unroll
    for (int j = 0; j < kAbsmeanThreads / kWave; ++j) t += sw[j];
  }
  return t;
}

template <bool F32>
__device__ __forceinline__ void absmean_block(const void* __restrict__ w, int64_t n, double* __restrict__ partials,
                                              int b) {
  const double t = absmean_block_reduce(absmean_thread_sum<F32>(w, n, b));
  if (threadIdx.x == 0) partials[b] = t;
}

template <bool F32>
__global__ __launch_bounds__(kAbsmeanThreads) void absmean_partials_kernel(
    const void* __restrict__ w, int64_t n, double* __restrict__ partials) {
  absmean_block<F32>(w, n, partials, blockIdx.x);
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
  const int64_t total = N * words_per_row;
  const int64_t stride = (int64_t)gridDim.x * kPackThreads;
  const int64_t wi0 = (int64_t)blockIdx.x * kPackThreads + threadIdx.x;
  // the thread's first word is requested before gamma is reduced, so that
  // its load latency overlaps the reduction of the partials
  float vals[16];
  if (wi0 < total) {
    const int64_t n = wi0 / words_per_row;
    load_word<F32, VEC>(w, n, K, (wi0 - n * words_per_row) * 16, vals);
  }
  const double S = partials_total(partials, sred);
  if (threadIdx.x == 0) {
    const double mean = S / (double)(N * K);
    const float g = fmaxf((float)mean, 1e-8f);
    s_half = g * 0.5f;  // exact
    if (blockIdx.x == 0) *gamma_out = g;
  }
  __syncthreads();
  const float h = s_half;

  for (int64_t wi = wi0; wi < total; wi += stride) {
    if (wi != wi0) {
      const int64_t n = wi / words_per_row;
      load_word<F32, VEC>(w, n, K, (wi - n * words_per_row) * 16, vals);
    }
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

// The pack pass (gamma from the partials, codes, packing).
hipError_t launch_pack(const void* W, bool w_is_f32, int64_t N, int64_t K, uint8_t* w_packed, float* gamma,
                       const double* partials, hipStream_t stream) {
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

hipError_t launch_ternarize_pack(const void* W, bool w_is_f32, int64_t N, int64_t K,
                                 uint8_t* w_packed, float* gamma, double* partials,
                                 hipStream_t stream) {
  if (onepass_ok(w_is_f32, N, K, false)) {
    launch_onepass(static_cast<const uint16_t*>(W), N, K, partials, reinterpret_cast<uint32_t*>(w_packed), gamma,
                   nullptr, 0, nullptr, nullptr, stream);
    return hipGetLastError();
  }
  const int64_t n = N * K;
  if (w_is_f32)
    absmean_partials_kernel<true><<<kAbsmeanBlocks, kAbsmeanThreads, 0, stream>>>(W, n, partials);
  else
    absmean_partials_kernel<false><<<kAbsmeanBlocks, kAbsmeanThreads, 0, stream>>>(W, n, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_pack(W, w_is_f32, N, K, w_packed, gamma, partials, stream);
}

// ---------------------------------------------------------------------------
// Code counts ("bitlinear.py", BitLinear.ternary_stats: the share of -1, 0
// and +1 in the current ternary weight). The two bits of each code are
// adjacent (bits 2i, 2i+1 of a word hold one code), so with lo = the even
// bits and hi = the odd bits of a word, +1 (01) is lo & ~hi and -1 (11) is
// lo & hi; padding codes are 0 and count for neither. One block, a fixed
// order: the counts are exact and repeatable.
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(1024) void code_counts_kernel(const uint32_t* __restrict__ packed, int64_t words,
                                                           unsigned long long* __restrict__ counts) {
  unsigned long long pos = 0, neg = 0;
  for (int64_t i = threadIdx.x; i < words; i += 1024) {
    const uint32_t w = packed[i];
    const uint32_t lo = w & 0x55555555u, hi = (w >> 1) & 0x55555555u;
    pos += __popc(lo & ~hi);
    neg += __popc(lo & hi);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    pos += __shfl_xor(pos, off, kWave);
    neg += __shfl_xor(neg, off, kWave);
  }
  __shared__ unsigned long long sp[16], sn[16];
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  if (lane == 0) {
    sp[wave] = pos;
    sn[wave] = neg;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long p = 0, n = 0;
    for (int j = 0; j < 16; ++j) {
      p += sp[j];
      n += sn[j];
    }
    counts[0] = n;
    counts[1] = p;
  }
}

hipError_t launch_code_counts(const uint8_t* w_packed, int64_t N, int64_t K, unsigned long long* counts,
                              hipStream_t stream) {
  code_counts_kernel<<<1, 1024, 0, stream>>>(reinterpret_cast<const uint32_t*>(w_packed), N * (k_pad(K) / 16),
                                             counts);
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
// in registers: one HBM read of x, one write of x_q. A block of BLOCK
// threads holds BLOCK / TPR rows; `b` is the block's index among the
// act-quant blocks of the launch.
// The chunks of one row for its TPR threads (K % 8 == 0), every load
// unconditional and all CPT in flight before the first use: a buffer
// resource over the row (none past M) returns zeros for chunks past K and
// for rows past M. (A load under a condition is waited for at the branch
// join, which turns the CPT loads into CPT dependent round trips.) Whole
// waves share a row, so the row index is uniform across the wave.
template <int TPR, int CPT>
__device__ __forceinline__ void aq_load(const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t row, int t,
                                        uint4 (&v)[CPT]) {
  const int row_w = __builtin_amdgcn_readfirstlane((int)row);
  const rsrc_t rx = make_rsrc(x + (int64_t)row_w * K, row_w < M ? (uint32_t)(K * 2) : 0u);
#pragma unroll
  for (int c = 0; c < CPT; ++c) v[c] = buf_load16(rx, (uint32_t)(t + c * TPR) * 16u);
}

// The rest of a row once its chunks are in registers: row absmax (wave
// max, then LDS across the row's waves), s, and x_q from the registers.
template <int BLOCK, int TPR, int CPT>
__device__ __forceinline__ void aq_finish(const uint4 (&v)[CPT], int64_t M, int64_t Kp, int8_t* __restrict__ xq,
                                          float* __restrict__ s_out, int64_t row, int t) {
  static_assert(TPR % kWave == 0 && BLOCK % TPR == 0, "whole waves per row");
  constexpr int WPR = TPR / kWave;
  __shared__ float smax[BLOCK / kWave];
  const int r_local = threadIdx.x / TPR;
  const bool row_ok = row < M;
  const int64_t nchunks = Kp / 8;
  float amax = 0.0f;
#pragma unroll
  for (int c = 0; c < CPT; ++c) amax = fmaxf(amax, absmax8(v[c]));
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

// TPR threads (whole waves) per row, CPT chunks of 8 values per thread kept
// in registers: one HBM read of x, one write of x_q. A block of BLOCK
// threads holds BLOCK / TPR rows; `b` is the block's index among the
// act-quant blocks of the launch.
template <int BLOCK, int TPR, int CPT, bool VEC>
__device__ __forceinline__ void act_quant_rows(const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t Kp,
                                               int8_t* __restrict__ xq, float* __restrict__ s_out, int b) {
  constexpr int RPB = BLOCK / TPR;
  const int t = threadIdx.x % TPR;
  const int64_t row = (int64_t)b * RPB + threadIdx.x / TPR;
  uint4 v[CPT];
  if constexpr (VEC) {
    aq_load<TPR, CPT>(x, M, K, row, t, v);
  } else {
    const bool row_ok = row < M;
    const uint16_t* xr = x + row * K;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int64_t ch = t + (int64_t)c * TPR;
      v[c] = (row_ok && ch * 8 < K) ? load_chunk<VEC>(xr, ch, K) : make_uint4(0, 0, 0, 0);
    }
  }
  aq_finish<BLOCK, TPR, CPT>(v, M, Kp, xq, s_out, row, t);
}

template <int TPR, int CPT, bool VEC>
__global__ __launch_bounds__(256) void act_quant_kernel(const uint16_t* __restrict__ x, int64_t M,
                                                        int64_t K, int64_t Kp,
                                                        int8_t* __restrict__ xq,
                                                        float* __restrict__ s_out) {
  act_quant_rows<256, TPR, CPT, VEC>(x, M, K, Kp, xq, s_out, blockIdx.x);
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

// Threads per row: as many as keep every thread busy with at least one
// chunk, up to 256. More threads per row (fewer chunks each) keep more loads
// in flight per CU and shorten each wave's dependent load -> max -> store
// chain (measured at 4096 x 2560: 64 threads per row 13.1 us, 256 12.1 us;
// at 4096 x 6912: 28.4 and 24.7 us).
static int aq_tpr(int64_t nchunks) { return nchunks >= 256 ? 256 : nchunks >= 128 ? 128 : 64; }

template <bool VEC>
static void launch_aq(const uint16_t* x, int64_t M, int64_t K, int64_t Kp, int8_t* xq, float* s,
                      hipStream_t st) {
  const int64_t nchunks = Kp / 8;
  if (nchunks > 256 * 8) {
    act_quant_long_kernel<VEC><<<(int)M, 256, 0, st>>>(x, M, K, Kp, xq, s);
    return;
  }
  switch (aq_tpr(nchunks)) {
    case 64: launch_aq_tpr<64, VEC>((int)((nchunks + 63) / 64), x, M, K, Kp, xq, s, st); break;
    case 128: launch_aq_tpr<128, VEC>((int)((nchunks + 127) / 128), x, M, K, Kp, xq, s, st); break;
    default: launch_aq_tpr<256, VEC>((int)((nchunks + 255) / 256), x, M, K, Kp, xq, s, st); break;
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
// One pass over W: the weight is read once. The grid is the absmean's fixed
// grid (kAbsmeanBlocks blocks of kAbsmeanThreads threads), and each thread
// keeps the 16-byte vectors it sums (those absmean_thread_sum reads) in
// registers instead of dropping them. Each block publishes its partial,
// quantizes its share of the activation rows (if any) while the other
// blocks finish theirs, then reads all kAbsmeanBlocks partials, forms gamma
// in the order ternarize_pack_kernel uses (so gamma, and every code, has the
// bits of the two-pass path) and writes the codes of the vectors it holds.
//
// A code word is 16 consecutive k of one row; with K a multiple of 64 (no
// row padding) word i / 2 is the pair of vectors i (codes 0..7) and i + 1
// (codes 8..15). Both sit in adjacent lanes of one wave (the vector index
// of a lane is b * kAbsmeanThreads + t + j * stride, stride even), so each
// lane builds its half of the word's bits and one lane exchange joins them.
//
// Publication: each block owns a 16-byte record in the workspace: its
// partial, then a publication word. It stores the partial, waits for the
// store to complete, then stores the word (device-coherent stores). The
// word is the launch's tag with a sequence number, so a word left by
// another launch, or by an earlier replay of a captured graph (same tag,
// smaller sequence), never matches: each block computes the expected word
// from its own record's previous one, and all records move in step because
// every launch rewrites each of them once. 256 threads of each block poll
// the records, one each (a 16-byte volatile load, which returns a published
// word together with its partial). No atomics and no counter to clear. No block ever waits on one that might not run: after `spin_limit`
// polls (another kernel holding CUs so that not every block of this launch
// is resident, or a test forcing the limit to 0) a block computes each
// partial still unpublished itself, with the same arithmetic on the same
// vectors, so the bits do not change. The wait also ends after 200 us
// (kOnePassWaitTicks) whatever `spin_limit` says.
// ---------------------------------------------------------------------------

// 16-byte vectors of W per thread, held in registers: 17 covers a 6912 x
// 2560 weight; 24 holds up to 25.1 M weights, used where the activation
// rows leave the registers for it (no spills: K <= 3072 with the rows, any
// K for the weight alone).
constexpr int kOnePassVecsSmall = 17;
constexpr int kOnePassVecsLarge = 24;
constexpr int64_t kOnePassStride = (int64_t)kAbsmeanBlocks * kAbsmeanThreads;

// The ternarize workspace: the partials first (the two-pass kernels use only
// them), then one 16-byte record per block of the one-pass launch: its
// partial and its publication word.
struct QuantSlot {
  uint64_t partial;  // fp64 bits
  uint64_t flag;     // tag << 16 | sequence
};
struct QuantSync {
  double partials[kAbsmeanBlocks];
  QuantSlot slots[kAbsmeanBlocks];
};

// The register count for a one-pass launch of this shape (0: none; the
// two-pass kernels run). with_rows: the activation rows share the launch
// (K <= 8192 then).
static int onepass_vecs(bool w_is_f32, int64_t N, int64_t K, bool with_rows) {
  if (w_is_f32 || K % 64 != 0) return 0;
  const int64_t nvec = N * K / 8;
  if (with_rows && K > 7168) return 0;  // 128 threads x 8 chunks per row would spill
  if (nvec <= kOnePassVecsSmall * kOnePassStride) return kOnePassVecsSmall;
  if (nvec <= kOnePassVecsLarge * kOnePassStride && (!with_rows || K <= 3072)) return kOnePassVecsLarge;
  return 0;
}

bool onepass_ok(bool w_is_f32, int64_t N, int64_t K, bool with_rows) {
  return onepass_vecs(w_is_f32, N, K, with_rows) != 0;
}

// The publication word a launch with this tag writes, from the word the
// block's record held: the sequence counts the launches with this tag
// (graph replays) in 1 .. 65535; a word of another tag restarts it at 1.
// Every launch rewrites every record, so all records hold the same word
// between launches and each block derives the same word from its own.
__device__ __forceinline__ uint64_t next_flag(uint64_t prev, uint64_t tag) {
  const uint64_t seq = (prev >> 16) == tag ? (prev & 0xFFFF) % 0xFFFF + 1 : 1;
  return (tag << 16) | seq;
}

// The longest a block waits for the others' records, in ticks of the
// 100 MHz real-time counter: 200 us, ten times the whole launch at the layer
// shapes. Blocks that are all resident publish within microseconds of each
// other; a longer wait means some block cannot start before others finish
// (another kernel holding CUs), and computing the missing partials is then
// far cheaper than waiting.
constexpr uint64_t kOnePassWaitTicks = 20000;

// One 16-byte volatile load: the records change under the polling loop
// (other blocks store them), so the compiler must issue the load on every
// iteration instead of keeping one result, and a volatile access bypasses
// the caches that are not coherent across the device.
__device__ __forceinline__ uint4 load16_polled(const QuantSlot* p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = *reinterpret_cast<const volatile u32x4*>(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Partials a one-pass block computed itself because their record was not
// published after the wait (read and cleared by bitnet_quantize_recomputes()).
__device__ unsigned int g_onepass_recomputes;

template <int V, bool AQ, int TPR, int CPT>
__global__ __launch_bounds__(kAbsmeanThreads) void quant_onepass_kernel(
    const uint16_t* __restrict__ w, int64_t N, int64_t K, QuantSync* __restrict__ sync, uint64_t tag,
    uint32_t spin_limit, uint32_t* __restrict__ packed, float* __restrict__ gamma_out,
    const uint16_t* __restrict__ x, int64_t M, int8_t* __restrict__ xq, float* __restrict__ s_out) {
  constexpr int64_t stride = kOnePassStride;
  const int b = blockIdx.x, t = threadIdx.x;
  const int64_t n = N * K, nvec = n / 8;
  const int64_t tid = (int64_t)b * kAbsmeanThreads + t;
  // the block's own record from the last launch, read by every thread (one
  // request per wave, no branch, so nothing waits for it until it is used)
  const uint64_t prev = __hip_atomic_load(&sync->slots[b].flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // unconditional buffer loads, all V in flight: offsets past W read zeros
  // (n * 2 bytes and every offset fit in 32 bits at these sizes)
  const rsrc_t rw = make_rsrc(w, (uint32_t)(n * 2));
  uint4 v[V];
#pragma unroll
  for (int j = 0; j < V; ++j) v[j] = buf_load16(rw, (uint32_t)((tid + j * stride) * 16));
  // the chunks of this block's first two groups of activation rows,
  // requested behind W's loads so that they are in flight while W is summed
  // and published (rows past M get an empty resource: zeros, no stores).
  // Requested before W's, they were quantized earlier but W's sum, and so
  // every block's publication, came later: 21.8 against 17.3 us to the
  // codes, cold, at 4096 x 2560 -> 6912.
  constexpr int RPB = kAbsmeanThreads / TPR;
  constexpr int64_t kGroupStride = kAbsmeanBlocks;  // groups b, b + 256, b + 512, ... are this block's
  uint4 xa[CPT], xb[CPT];
  if constexpr (AQ) {
    aq_load<TPR, CPT>(x, M, K, (int64_t)b * RPB + t / TPR, t % TPR, xa);
    aq_load<TPR, CPT>(x, M, K, ((int64_t)b + kGroupStride) * RPB + t / TPR, t % TPR, xb);
  }
  // W's vectors (the launch holds all of W: nvec <= V * stride) are
  // summed as absmean_thread_sum sums them: whole groups of 8 into the 8
  // accumulators, the rest into the first, in order (a zero vector adds
  // +0.0, which changes nothing). A group that extends past V is never
  // whole, since its last vector would lie past nvec.
  double acc[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) acc[u] = 0.0;
#pragma unroll
  for (int g = 0; g < (V + 7) / 8; ++g) {
    if (8 * g + 8 <= V && tid + (8 * g + 7) * stride < nvec) {
#pragma unroll
      for (int u = 0; u < 8; ++u) acc[u] += abs_sum16<false>(v[(8 * g + u) % V]);
    } else {
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (8 * g + u < V) acc[0] += abs_sum16<false>(v[8 * g + u]);
    }
  }
  const double mine =
      absmean_block_reduce(((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7])));
  const uint64_t want = next_flag(prev, tag);
  if (t == 0) {
    // the partial first, complete before the word that publishes it: a
    // reader that sees the word in a 16-byte load sees the partial with it
    __hip_atomic_store(&sync->slots[b].partial, (uint64_t)__double_as_longlong(mine), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    wait_vmem();
    __hip_atomic_store(&sync->slots[b].flag, want, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  if constexpr (AQ) {
    // this block's rows of the activation quantization, behind which the
    // other blocks' partials arrive: two groups at a time, each buffer
    // refilled with the group two ahead as soon as it is used, so that two
    // groups' loads stay in flight. The refills run in every block that
    // gets here (a group past M is all zeros and stores nothing): no load
    // sits under a condition, where it would be waited for at the join. A
    // block whose second group lies past M stops after the first (few
    // tokens: the blocks that hold rows would otherwise finish an empty
    // group and end the launch later than the others).
    const int64_t groups = (M + RPB - 1) / RPB;
    for (int64_t gi = b; gi < groups; gi += 2 * kGroupStride) {
      aq_finish<kAbsmeanThreads, TPR, CPT>(xa, M, K, xq, s_out, gi * RPB + t / TPR, t % TPR);
      aq_load<TPR, CPT>(x, M, K, (gi + 2 * kGroupStride) * RPB + t / TPR, t % TPR, xa);
      __syncthreads();  // the row maxima in LDS are reused by the next group
      if (gi + kGroupStride >= groups) break;  // the same in every thread of the block
      aq_finish<kAbsmeanThreads, TPR, CPT>(xb, M, K, xq, s_out, (gi + kGroupStride) * RPB + t / TPR, t % TPR);
      aq_load<TPR, CPT>(x, M, K, (gi + 3 * kGroupStride) * RPB + t / TPR, t % TPR, xb);
      __syncthreads();
    }
  }

  // every partial: each of the first 256 threads polls one record (a
  // 16-byte volatile load) until every record holds this launch's word or
  // `spin_limit` polls have passed; a record still unpublished then is
  // computed here
  __shared__ double sp[kAbsmeanBlocks];
  __shared__ int smiss[kAbsmeanBlocks];
  __shared__ int s_anymiss;
  __shared__ double sred[kAbsmeanBlocks / kWave];
  uint4 r = make_uint4(0u, 0u, 0u, 0u);
  bool ok = true;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  for (uint32_t i = 0;; ++i) {
    if (t < kAbsmeanBlocks) {
      r = load16_polled(&sync->slots[t]);
      ok = ((uint64_t)r.w << 32 | r.z) == want;
    }
    // thread 0's clock decides for the block, so every thread takes the
    // same branch
    const bool late = t == 0 && __builtin_amdgcn_s_memrealtime() - t0 > kOnePassWaitTicks;
    if (__syncthreads_and(ok) || __syncthreads_or(late) || i >= spin_limit) break;
    __builtin_amdgcn_s_sleep(4);
  }
  if (t == 0) s_anymiss = 0;
  __syncthreads();
  if (t < kAbsmeanBlocks) {
    sp[t] = ok ? __longlong_as_double((long long)((uint64_t)r.y << 32 | r.x)) : 0.0;
    smiss[t] = ok ? 0 : 1;
    if (!ok) s_anymiss = 1;
  }
  __syncthreads();
  if (s_anymiss) {  // the same value in every thread
    for (int q = 0; q < kAbsmeanBlocks; ++q) {
      if (smiss[q]) {
        const double p = absmean_block_reduce(absmean_thread_sum<false>(w, n, q));
        if (t == 0) {
          sp[q] = p;
          atomicAdd(&g_onepass_recomputes, 1u);
        }
        __syncthreads();
      }
    }
  }
  // gamma as ternarize_pack_kernel forms it (partials_total's order)
  if (t < kAbsmeanBlocks) {
    const double ws = wave_sum_f64(sp[t]);
    if (t % kWave == 0) sred[t / kWave] = ws;
  }
  __syncthreads();
  const double S = (sred[0] + sred[1]) + (sred[2] + sred[3]);
  const float g = fmaxf((float)(S / (double)n), 1e-8f);
  const float h = g * 0.5f;  // exact
  if (b == 0 && t == 0) *gamma_out = g;

  // the codes of the held vectors: code e of vector i goes to code 8 (i % 2)
  // + e of word i / 2, at bit 8 (c % 4) + 2 (c / 4) for code c of a word
  const uint32_t hsh = 4u * (uint32_t)(t & 1);
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const int64_t i = tid + j * stride;
    uint4 d = v[j];
    // keeps the unpacking here: hoisted above the exchange it would hold 8
    // floats per vector instead of 4 words across the whole wait
    asm volatile("" : "+v"(d.x), "+v"(d.y), "+v"(d.z), "+v"(d.w));
    const float e[8] = {bf16_lo(d.x), bf16_hi(d.x), bf16_lo(d.y), bf16_hi(d.y),
                        bf16_lo(d.z), bf16_hi(d.z), bf16_lo(d.w), bf16_hi(d.w)};
    uint32_t half = 0;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint32_t code = (e[c] > h) ? 1u : ((e[c] < -h) ? 3u : 0u);
      half |= code << (8 * (c & 3) + 2 * (c >> 2));
    }
    half <<= hsh;
    // the other half from the neighbouring lane: a DPP quad permute
    // [1, 0, 3, 2] (lane l reads lane l ^ 1), no LDS round trip
    const uint32_t other = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)half, 0xB1, 0xF, 0xF, false);
    const uint32_t word = half | other;
    if (i < nvec && (t & 1) == 0) packed[i >> 1] = word;
  }
}

// The (V, threads per row, chunks per thread) launches onepass_vecs admits
// (those that keep everything in registers); the others are not built.
constexpr bool onepass_variant(int V, int TPR, int C) {
  return V == kOnePassVecsSmall ? !(TPR == 128 && C == 8) : (TPR == 64 && C <= 6);
}

template <int V, int TPR>
static void launch_onepass_tpr(int cpt, const uint16_t* W, int64_t N, int64_t K, QuantSync* sync, uint64_t tag,
                               uint32_t spin, uint32_t* packed, float* gamma, const uint16_t* x, int64_t M,
                               int8_t* xq, float* s, hipStream_t st) {
  switch (cpt) {
#define BITNET_ONEPASS(C)                                                                                     \
    case C:                                                                                                 \
      if constexpr (onepass_variant(V, TPR, C))                                                             \
        quant_onepass_kernel<V, true, TPR, C><<<kAbsmeanBlocks, kAbsmeanThreads, 0, st>>>(                  \
            W, N, K, sync, tag, spin, packed, gamma, x, M, xq, s);                                          \
      break;
    BITNET_ONEPASS(1) BITNET_ONEPASS(2) BITNET_ONEPASS(3) BITNET_ONEPASS(4)
    BITNET_ONEPASS(5) BITNET_ONEPASS(6) BITNET_ONEPASS(7) BITNET_ONEPASS(8)
#undef BITNET_ONEPASS
  }
}

template <int V>
static void launch_onepass_v(const uint16_t* W, int64_t N, int64_t K, QuantSync* sync, uint64_t tag, uint32_t spin,
                             uint32_t* packed, float* gamma, const uint16_t* x, int64_t M, int8_t* xq, float* s,
                             hipStream_t st) {
  if (x == nullptr) {
    quant_onepass_kernel<V, false, 64, 1><<<kAbsmeanBlocks, kAbsmeanThreads, 0, st>>>(
        W, N, K, sync, tag, spin, packed, gamma, nullptr, 0, nullptr, nullptr);
    return;
  }
  // rows as in the shared two-pass launch: 64 threads up to 512 chunks, 128
  // above
  const int64_t nchunks = K / 8;
  if (nchunks <= 64 * 8)
    launch_onepass_tpr<V, 64>((int)((nchunks + 63) / 64), W, N, K, sync, tag, spin, packed, gamma, x, M, xq, s, st);
  else if constexpr (V == kOnePassVecsSmall)
    launch_onepass_tpr<V, 128>((int)((nchunks + 127) / 128), W, N, K, sync, tag, spin, packed, gamma, x, M, xq, s,
                               st);
}

// x == nullptr: the weight alone (bitnet_ternarize_pack). The caller checked
// onepass_ok. The launch's tag is fresh for every launch.
void launch_onepass(const uint16_t* W, int64_t N, int64_t K, void* ws, uint32_t* packed, float* gamma,
                    const uint16_t* x, int64_t M, int8_t* xq, float* s, hipStream_t st) {
  QuantSync* sync = static_cast<QuantSync*>(ws);
  const uint64_t tag = next_launch_tag();
  const uint32_t spin = test_knobs().spin_limit.load(std::memory_order_relaxed);
  if (onepass_vecs(false, N, K, x != nullptr) == kOnePassVecsSmall)
    launch_onepass_v<kOnePassVecsSmall>(W, N, K, sync, tag, spin, packed, gamma, x, M, xq, s, st);
  else
    launch_onepass_v<kOnePassVecsLarge>(W, N, K, sync, tag, spin, packed, gamma, x, M, xq, s, st);
}

size_t quant_workspace_bytes() { return sizeof(QuantSync); }

hipError_t take_onepass_recomputes(unsigned int* count) {
  unsigned int* d = nullptr;
  if (hipError_t e = hipGetSymbolAddress(reinterpret_cast<void**>(&d), HIP_SYMBOL(g_onepass_recomputes))) return e;
  if (hipError_t e = hipDeviceSynchronize()) return e;
  if (hipError_t e = hipMemcpy(count, d, sizeof(unsigned int), hipMemcpyDeviceToHost)) return e;
  const unsigned int zero = 0;
  return hipMemcpy(d, &zero, sizeof(unsigned int), hipMemcpyHostToDevice);
}

// ---------------------------------------------------------------------------
// Weight absmean partials and activation quantization in one launch. The
// two are independent HBM streams (W, and x -> x_q, s); sharing a launch
// lets each fill the CUs while the other ramps up or drains, and saves a
// launch. The first blocks quantize rows, kAbsmeanThreads / TPR per block
// (dispatched first: measured 1-3 us faster than the other order at the
// layer shapes); the last kAbsmeanBlocks compute the absmean partials
// exactly as absmean_partials_kernel does (same grid constants, so gamma
// gets the same bits). The codes are then packed by ternarize_pack_kernel,
// which needs every partial. Used when the rows fit the register-resident
// layout with 16-byte loads (K % 8 == 0, K <= 8192).
// ---------------------------------------------------------------------------

template <bool F32, int TPR, int CPT>
__global__ __launch_bounds__(kAbsmeanThreads) void quant_front_kernel(
    const void* __restrict__ w, int64_t n, double* __restrict__ partials, const uint16_t* __restrict__ x,
    int64_t M, int64_t K, int64_t Kp, int8_t* __restrict__ xq, float* __restrict__ s_out) {
  const int naq = (int)gridDim.x - kAbsmeanBlocks;
  if ((int)blockIdx.x < naq)
    act_quant_rows<kAbsmeanThreads, TPR, CPT, true>(x, M, K, Kp, xq, s_out, blockIdx.x);
  else
    absmean_block<F32>(w, n, partials, blockIdx.x - naq);
}

template <bool F32, int TPR>
static void launch_front_tpr(int cpt, const void* W, int64_t n, double* partials, const uint16_t* x, int64_t M,
                             int64_t K, int64_t Kp, int8_t* xq, float* s, hipStream_t st) {
  constexpr int RPB = kAbsmeanThreads / TPR;
  const int grid = kAbsmeanBlocks + (int)((M + RPB - 1) / RPB);
  switch (cpt) {
#define BITNET_FRONT(C) \
    case C: quant_front_kernel<F32, TPR, C><<<grid, kAbsmeanThreads, 0, st>>>(W, n, partials, x, M, K, Kp, xq, s); break;
    BITNET_FRONT(1) BITNET_FRONT(2) BITNET_FRONT(3) BITNET_FRONT(4)
    BITNET_FRONT(5) BITNET_FRONT(6) BITNET_FRONT(7)
    default: quant_front_kernel<F32, TPR, 8><<<grid, kAbsmeanThreads, 0, st>>>(W, n, partials, x, M, K, Kp, xq, s);
#undef BITNET_FRONT
  }
}

// In the shared launch rows take 64 threads up to 512 chunks and 128 up to
// 1024: the act-quant share then has few, large blocks (measured 2 us faster
// at 4096 x 2560 than 256 threads per row, whose 2048 small blocks
// the absmean blocks wait behind).
template <bool F32>
static void launch_front(const void* W, int64_t n, double* partials, const uint16_t* x, int64_t M, int64_t K,
                         int64_t Kp, int8_t* xq, float* s, hipStream_t st) {
  const int64_t nchunks = Kp / 8;
  if (nchunks <= 64 * 8)
    launch_front_tpr<F32, 64>((int)((nchunks + 63) / 64), W, n, partials, x, M, K, Kp, xq, s, st);
  else
    launch_front_tpr<F32, 128>((int)((nchunks + 127) / 128), W, n, partials, x, M, K, Kp, xq, s, st);
}

hipError_t launch_quantize(const void* W, bool w_is_f32, int64_t N, int64_t K, const uint16_t* x, int64_t M,
                           uint8_t* w_packed, float* gamma, int8_t* x_q, float* s_x, double* partials,
                           hipStream_t stream) {
  const int64_t Kp = k_pad(K), nchunks = Kp / 8;
  if (K % 8 != 0 || nchunks > 128 * 8) {
    if (hipError_t e = launch_act_quant(x, M, K, x_q, s_x, stream)) return e;
    return launch_ternarize_pack(W, w_is_f32, N, K, w_packed, gamma, partials, stream);
  }
  if (onepass_ok(w_is_f32, N, K, true)) {
    launch_onepass(static_cast<const uint16_t*>(W), N, K, partials, reinterpret_cast<uint32_t*>(w_packed), gamma,
                   x, M, x_q, s_x, stream);
    return hipGetLastError();
  }
  if (w_is_f32) launch_front<true>(W, N * K, partials, x, M, K, Kp, x_q, s_x, stream);
  else launch_front<false>(W, N * K, partials, x, M, K, Kp, x_q, s_x, stream);
  if (hipError_t e = hipGetLastError()) return e;
  return launch_pack(W, w_is_f32, N, K, w_packed, gamma, partials, stream);
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
