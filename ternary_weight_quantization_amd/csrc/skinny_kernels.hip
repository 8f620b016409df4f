// Products for few tokens (M <= 64): the decode-shaped GEMMs of an inference
// forward or a small training batch ("bitnet-qat-train", Semantics):
//  - the INT8 forward, acc = sum_k x_q * q (INT32), y = bf16(acc * (s/127) *
//    gamma [+ bias]);
//  - the STE backward dX = dY * W_hat, W_hat = q * bf16(gamma), products
//    exact in fp32 and sums in fp32.
// At these sizes the cost is reading the codes once and the token operand
// (x_q or dY) from L2; the 256 x 256 tiles of the large-M GEMMs would leave
// most of each MFMA tile empty and split the few tiles into many pieces.
//
// Both are C[i][m] = sum_r A[i][r] * B[m][r] with A a code operand (rows i)
// and B the token operand (rows m), and move the same bytes per lane: the
// reduction runs in super-steps of 32 code bytes per row (128 k of 2-bit
// codes for the forward, 64 n of the fp4 transposed codes for dX) and 128
// token-operand bytes per row (128 k of int8, 64 n of bf16).
//
// One workgroup of W waves (16 for up to 32 tokens, 8 for up to 64) owns 32
// code rows i0 .. i0+31 and every token. The reduction runs in chunks of W
// super-steps, one per wave. The token operand's columns of a chunk are
// loaded with coalesced 16-byte loads (8W threads per token row) and written
// to an LDS tile of 128W + 16-byte rows (the pad makes the fragment reads
// conflict-free); P chunks are in flight. In wave w's super-step of a chunk,
// lane half h takes code bytes 32w + 16h .. +15 of its row (read straight
// from memory) and bytes 128w + 64h .. +63 of its token's LDS row; step j
// (0..3) multiplies dword j of the codes, expanded to MFMA operand form,
// with token bytes 16j .. 16j+15 of those in one MFMA per 32 tokens (rows:
// code row i0 + l % 32; columns: token 32mt + l % 32). The waves' partial
// tiles are added in LDS in wave order (exact for the forward's int32), then
// the epilogue rescales. The forward's y and acc are bit-identical to the
// large-M GEMM's. Rows past the operands and columns past their valid bytes
// read as zeros through the buffer range checks.

#include "device_common.h"
#include "internal.h"

namespace bitnet {

// Forward: A = 2-bit codes [N][Kp/4] (rows i = n), B = x_q [M][Kp].
struct SkFwd {
  typedef i32x16_t Acc;
  typedef int Elem;
  static constexpr int kCodeB = 32;  // code bytes per row per super-step
  static __device__ __forceinline__ Acc mma(uint32_t code_word, uint4 b, Acc acc) {
    i32x4_t a;
#pragma unroll
    for (int t = 0; t < 4; ++t) a[t] = (int)codes4_to_i8((code_word >> (2 * t)) & 0x03030303u);
    const i32x4_t bx = {(int)b.x, (int)b.y, (int)b.z, (int)b.w};
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, bx, acc, 0, 0, 0);
  }
};

// dX: A = fp4 transposed codes [Kp][Np/2] (rows i = k; +1 = 0x2, -1 = 0xA,
// 0 = 0x0, n even in the low nibble), B = dY [M][N] bf16.
struct SkDx {
  typedef f32x16_t Acc;
  typedef float Elem;
  static constexpr int kCodeB = 32;
  static __device__ __forceinline__ Acc mma(uint32_t code_word, uint4 b, Acc acc) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    // byte t of the word: two fp4 values -> two bf16 (scale 1: exact +-1, 0)
    const u32x4 a = {__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(code_word, 1.0f, 0)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(code_word, 1.0f, 1)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(code_word, 1.0f, 2)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(code_word, 1.0f, 3))};
    const u32x4 bx = {b.x, b.y, b.z, b.w};
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, bx),
                                                   acc, 0, 0, 0);
  }
};

// TTQ forward ("TTQ_VERIFICATION.md", Eq. 1): A = the same 2-bit codes
// [N][Kp/4] (rows i = n), B = x [M][K] bf16, unquantized. 16 code bytes
// (64 k) per row per super-step match the 128 bytes (64 k) of bf16 tokens.
// Lane half h's 8 code bytes are two words of 16 codes (k = 32h .. 32h+31
// of the super-step); step j takes codes 8j .. 8j+7, i.e. word j/2 shifted
// by 4(j%2), whose bytes hold codes b and b+4 at bits 0 and 2 (code j of a
// word at bit 8(j%4) + 2(j/4)). Each code becomes its bf16 value through a
// byte permute of the table {0, bf16(Wp), 0, -bf16(Wn)} (2 bytes per entry,
// entry c at bytes 2c, 2c+1): selector bytes 2c, 2c+1 are built from the
// codes with one more permute.
struct SkTtq {
  typedef f32x16_t Acc;
  typedef float Elem;
  static constexpr int kCodeB = 16;
  // two bf16 values (codes in bytes b0, b0+1 of d = 2 * codes) -> one dword
  static __device__ __forceinline__ uint32_t pair(uint32_t d, uint32_t sel, uint32_t tlo, uint32_t thi) {
    return perm(thi, tlo, perm(d + 0x01010101u, d, sel));
  }
  static __device__ __forceinline__ Acc mma(uint32_t w, uint4 b, Acc acc, uint32_t tlo, uint32_t thi) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const uint32_t d0 = (w & 0x03030303u) << 1;         // codes 0..3, doubled
    const uint32_t d1 = ((w >> 2) & 0x03030303u) << 1;  // codes 4..7, doubled
    // selector bytes [d.b0, d.b0 + 1, d.b1, d.b1 + 1] and [d.b2, .., d.b3 + 1]
    const u32x4 a = {pair(d0, 0x05010400u, tlo, thi), pair(d0, 0x07030602u, tlo, thi),
                     pair(d1, 0x05010400u, tlo, thi), pair(d1, 0x07030602u, tlo, thi)};
    const u32x4 bx = {b.x, b.y, b.z, b.w};
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, bx),
                                                   acc, 0, 0, 0);
  }
};

// The code operand: `rows` rows of `pitch` bytes, the first `bytes` of
// each in use; the token operand: M rows of `tpitch` bytes, the first
// `tbytes` of each valid (both multiples of 16). tlo, thi: SkTtq's value
// table (unused by the other policies).
struct SkArgs {
  const uint8_t* codes;
  int64_t rows, pitch, bytes;
  const void* tok;
  int64_t tpitch, tbytes;
  int M;
  uint32_t tlo, thi;
};

template <int MT>  // token tiles of 32: 1 for M <= 32, 2 for M <= 64
struct SkChunk {
  uint4 x[4 * MT];  // this thread's 16-byte pieces of the chunk's token columns (32 MT rows x 128 W bytes)
  uint4 codes;      // this lane's code bytes for its wave's super-step
};

// The partial tiles of the W waves of a workgroup, summed in wave order for
// the 4 values of rows i0 + 8g + 4h + 0..3 and token 32mt + l % 32 held by
// this lane (g = wave % 4, mt = wave / 4; nothing when mt >= MT).
template <class SK, int MT, int W, int P>
__device__ __forceinline__ void skinny_body(const SkArgs& a, char* smem, typename SK::Elem (&out)[4], int& mt_out,
                                            int& g_out) {
  typedef typename SK::Elem E;
  constexpr int kThreads = kWave * W;
  constexpr int kChunkB = 128 * W;           // token-operand bytes per row per chunk
  constexpr int kPitch = kChunkB + 16;       // LDS bytes per token row
  constexpr int kRowPieces = kChunkB / 16;   // 16-byte pieces per token row of a chunk
  static_assert(32 * MT * kRowPieces / kThreads == 4 * MT, "32 MT rows x 128 W bytes over 64 W threads");
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int h = lane >> 5, r32 = lane & 31;
  const int64_t i0 = (int64_t)blockIdx.x * 32;
  constexpr int kCB = SK::kCodeB;
  const int nchunks = (int)((a.bytes + kCB * W - 1) / (kCB * W));

  const rsrc_t rc = make_rsrc(a.codes, (uint32_t)(a.rows * a.pitch));
  const uint32_t coff = i0 + r32 < a.rows ? (uint32_t)((i0 + r32) * a.pitch) : kOob;  // the lane's code row
  const rsrc_t rx = make_rsrc(a.tok, (uint32_t)(a.M * a.tpitch));
  // piece p of a chunk: token row (p * kThreads + tid) / kRowPieces, 16-byte
  // column (p * kThreads + tid) % kRowPieces of the chunk
  const auto load = [&](SkChunk<MT>& b, int c) {
#pragma unroll
    for (int p = 0; p < 4 * MT; ++p) {
      const int e = p * kThreads + tid, row = e / kRowPieces, col = 16 * (e % kRowPieces);
      const int64_t x = (int64_t)c * kChunkB + col;
      b.x[p] = buf_load16(rx, row < a.M && x < a.tbytes ? (uint32_t)(row * a.tpitch + x) : kOob);
    }
    const int64_t cb = (int64_t)c * (kCB * W) + kCB * wave + (kCB / 2) * h;
    const uint32_t off = cb < a.bytes ? coff + (uint32_t)cb : kOob;
    if constexpr (kCB == 32) {
      b.codes = buf_load16(rc, off);
    } else {
      const uint2 c8 = buf_load8(rc, off);
      b.codes = make_uint4(c8.x, c8.y, 0u, 0u);
    }
  };
  const auto stage = [&](const SkChunk<MT>& b) {
#pragma unroll
    for (int p = 0; p < 4 * MT; ++p) {
      const int e = p * kThreads + tid;
      *reinterpret_cast<uint4*>(smem + (e / kRowPieces) * kPitch + 16 * (e % kRowPieces)) = b.x[p];
    }
  };

  typename SK::Acc acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[mt][e] = 0;
  const auto compute = [&](const SkChunk<MT>& b) {
    const uint32_t w4[4] = {b.codes.x, b.codes.y, b.codes.z, b.codes.w};
    const char* xr = smem + r32 * kPitch + 128 * wave + 64 * h;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const uint4 tok = *reinterpret_cast<const uint4*>(xr + 32 * mt * kPitch + 16 * j);
        if constexpr (kCB == 32)
          acc[mt] = SK::mma(w4[j], tok, acc[mt]);
        else
          acc[mt] = SK::mma(w4[j >> 1] >> (4 * (j & 1)), tok, acc[mt], a.tlo, a.thi);
      }
  };

  SkChunk<MT> buf[P];
#pragma unroll
  for (int d = 0; d < P; ++d) load(buf[d], d);
  for (int i = 0; i < nchunks; i += P) {
#pragma unroll
    for (int d = 0; d < P; ++d) {
      if (i + d < nchunks) {
        __syncthreads();  // the previous chunk's fragment reads are done
        stage(buf[d]);
        __syncthreads();
        compute(buf[d]);
        load(buf[d], i + d + P);  // past the last chunk: zeros, never staged
      }
    }
  }

  __syncthreads();
  E* red = reinterpret_cast<E*>(smem);  // [wave][mt][16][lane]
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int e = 0; e < 16; ++e) red[((wave * MT + mt) * 16 + e) * kWave + lane] = acc[mt][e];
  __syncthreads();
  const int g = wave % 4, mt = wave / 4;
  mt_out = mt;
  g_out = g;
  if (mt >= MT) return;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    E sum = 0;
#pragma unroll
    for (int w = 0; w < W; ++w) sum += red[((w * MT + mt) * 16 + 4 * g + e) * kWave + lane];
    out[e] = sum;
  }
}

// LDS bytes: the token tile of a chunk, reused for the partial tiles.
template <int MT, int W>
constexpr int skinny_lds() {
  return 32 * MT * (128 * W + 16) > W * MT * 16 * kWave * 4 ? 32 * MT * (128 * W + 16) : W * MT * 16 * kWave * 4;
}

// Forward: code rows n, tokens m; y [M][N] bf16, acc_out [M][N] int32 or NULL.
template <int MT, int W, int P>
__global__ __launch_bounds__(kWave * W) void fwd_skinny_kernel(SkArgs a, const float* __restrict__ s,
                                                               const float* __restrict__ gamma,
                                                               const uint16_t* __restrict__ bias, int64_t N,
                                                               uint16_t* __restrict__ y,
                                                               int32_t* __restrict__ acc_out) {
  __shared__ __attribute__((aligned(16))) char smem[skinny_lds<MT, W>()];
  int v[4], mt, g;
  skinny_body<SkFwd, MT, W, P>(a, smem, v, mt, g);
  const int lane = threadIdx.x % kWave, h = lane >> 5;
  const int64_t m = 32 * mt + (lane & 31);
  if (mt >= MT || m >= a.M) return;
  const float c = s[m] * *gamma / 127.0f;  // the large-M epilogue's expression
  const int64_t nb = (int64_t)blockIdx.x * 32 + 8 * g + 4 * h;
  float f[4] = {(float)v[0] * c, (float)v[1] * c, (float)v[2] * c, (float)v[3] * c};
  if (bias != nullptr) {
    const float4 b = bias4(bias, N, nb);
    f[0] += b.x; f[1] += b.y; f[2] += b.z; f[3] += b.w;
  }
  uint16_t* yr = y + m * N;
  if (N % 4 == 0 && nb + 4 <= N) {
    *reinterpret_cast<uint2*>(yr + nb) = make_uint2(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]));
    if (acc_out != nullptr) *reinterpret_cast<int4*>(acc_out + m * N + nb) = make_int4(v[0], v[1], v[2], v[3]);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (nb + e >= N) break;
      yr[nb + e] = f32_to_bf16_bits(f[e]);
      if (acc_out != nullptr) acc_out[m * N + nb + e] = v[e];
    }
  }
}

// dX: code rows k, tokens m; dX [M][K] bf16 = bf16(sum * bf16(gamma)).
template <int MT, int W, int P>
__global__ __launch_bounds__(kWave * W) void dx_skinny_kernel(SkArgs a, const float* __restrict__ gamma, int64_t K,
                                                              uint16_t* __restrict__ dX) {
  __shared__ __attribute__((aligned(16))) char smem[skinny_lds<MT, W>()];
  float v[4];
  int mt, g;
  skinny_body<SkDx, MT, W, P>(a, smem, v, mt, g);
  const int lane = threadIdx.x % kWave, h = lane >> 5;
  const int64_t m = 32 * mt + (lane & 31);
  if (mt >= MT || m >= a.M) return;
  const float sc = bf16_to_f32(f32_to_bf16_bits(*gamma));  // bf16(gamma), exact in fp32
  const int64_t kb = (int64_t)blockIdx.x * 32 + 8 * g + 4 * h;
  uint16_t* dr = dX + m * K;
  if (K % 4 == 0 && kb + 4 <= K) {
    *reinterpret_cast<uint2*>(dr + kb) = make_uint2(pack_bf16x2(v[0] * sc, v[1] * sc), pack_bf16x2(v[2] * sc, v[3] * sc));
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (kb + e >= K) break;
      dr[kb + e] = f32_to_bf16_bits(v[e] * sc);
    }
  }
}

// TTQ forward from the codes: code rows n, tokens m; y [M][N] bf16 = the fp32
// sum rounded once.
template <int MT, int W, int P>
__global__ __launch_bounds__(kWave * W) void ttq_fwd_skinny_kernel(SkArgs a, const float* __restrict__ params,
                                                                   int64_t N, uint16_t* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) char smem[skinny_lds<MT, W>()];
  a.tlo = (uint32_t)f32_to_bf16_bits(params[1]) << 16;               // codes 0, 1: 0, bf16(Wp)
  a.thi = (uint32_t)(f32_to_bf16_bits(params[2]) ^ 0x8000u) << 16;   // codes 2, 3: 0, -bf16(Wn)
  float v[4];
  int mt, g;
  skinny_body<SkTtq, MT, W, P>(a, smem, v, mt, g);
  const int lane = threadIdx.x % kWave, h = lane >> 5;
  const int64_t m = 32 * mt + (lane & 31);
  if (mt >= MT || m >= a.M) return;
  const int64_t nb = (int64_t)blockIdx.x * 32 + 8 * g + 4 * h;
  uint16_t* yr = y + m * N;
  if (N % 4 == 0 && nb + 4 <= N) {
    *reinterpret_cast<uint2*>(yr + nb) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (nb + e >= N) break;
      yr[nb + e] = f32_to_bf16_bits(v[e]);
    }
  }
}

hipError_t launch_ttq_fwd_skinny(const uint16_t* x, const uint8_t* w_packed, const float* params, int64_t M,
                                 int64_t N, int64_t K, uint16_t* y, hipStream_t stream) {
  if (M < 1 || M > kSkinnyMaxM || K % 8 != 0) return hipErrorInvalidValue;
  const int64_t Kp = k_pad(K);
  const SkArgs a{w_packed, N, Kp / 4, Kp / 4, x, 2 * K, 2 * K, (int)M, 0u, 0u};
  const unsigned grid = (unsigned)((N + 31) / 32);
  if (M <= 32)
    ttq_fwd_skinny_kernel<1, 16, 3><<<grid, kWave * 16, 0, stream>>>(a, params, N, y);
  else
    ttq_fwd_skinny_kernel<2, 8, 3><<<grid, kWave * 8, 0, stream>>>(a, params, N, y);
  return hipGetLastError();
}

hipError_t launch_fwd_skinny(const int8_t* x_q, const float* s_x, const uint8_t* w_packed, const float* gamma,
                             const uint16_t* bias, int64_t M, int64_t N, int64_t K, uint16_t* y, int32_t* acc_out,
                             hipStream_t stream) {
  if (M < 1 || M > kSkinnyMaxM) return hipErrorInvalidValue;
  const int64_t Kp = k_pad(K);
  const SkArgs a{w_packed, N, Kp / 4, Kp / 4, x_q, Kp, Kp, (int)M, 0u, 0u};
  const unsigned grid = (unsigned)((N + 31) / 32);
  if (M <= 32)
    fwd_skinny_kernel<1, 16, 3><<<grid, kWave * 16, 0, stream>>>(a, s_x, gamma, bias, N, y, acc_out);
  else
    fwd_skinny_kernel<2, 8, 3><<<grid, kWave * 8, 0, stream>>>(a, s_x, gamma, bias, N, y, acc_out);
  return hipGetLastError();
}

hipError_t launch_dx_skinny(const uint8_t* wt, const uint16_t* dY, const float* gamma, int64_t M, int64_t N,
                            int64_t K, uint16_t* dX, hipStream_t stream) {
  if (M < 1 || M > kSkinnyMaxM || N % 8 != 0) return hipErrorInvalidValue;
  const int64_t Kp = k_pad(K), Np = (N + 63) / 64 * 64;
  const SkArgs a{wt, Kp, Np / 2, Np / 2, dY, 2 * N, 2 * N, (int)M, 0u, 0u};
  const unsigned grid = (unsigned)(Kp / 32);
  if (M <= 32)
    dx_skinny_kernel<1, 16, 3><<<grid, kWave * 16, 0, stream>>>(a, gamma, K, dX);
  else
    dx_skinny_kernel<2, 8, 3><<<grid, kWave * 8, 0, stream>>>(a, gamma, K, dX);
  return hipGetLastError();
}

}  // namespace bitnet
