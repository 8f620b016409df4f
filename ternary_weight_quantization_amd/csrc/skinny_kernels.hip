// Forward GEMM for few tokens (M <= 64): the decode-shaped product of an
// inference forward or a small training batch ("bitnet-qat-train",
// Semantics: acc = sum_k x_q * q in INT32, y = bf16(acc * (s/127) * gamma)).
// At these sizes the cost is reading the 2-bit codes once (N * Kp/4 bytes)
// and the int8 activations from L2; the 256 x 256 tiles of the large-M GEMM
// would leave most of each MFMA tile empty and split the few tiles into many
// pieces.
//
// One workgroup of W waves (16 for up to 32 tokens, 8 for up to 64) owns 32
// weight rows n0 .. n0+31 and every token. The reduction runs in chunks of
// 128W k, each W super-steps of 128 k (32 bytes of codes per row), one per
// wave. The x_q columns of a chunk are loaded with coalesced 16-byte loads
// (8W threads per token row) and written to an LDS tile of 128W + 16-byte
// rows (the pad makes the fragment reads conflict-free); P chunks are in
// flight. In wave w's
// super-step of a chunk, lane half h takes the codes of k = 128w + 64h ..
// +63 of the chunk (16 bytes read straight from the codes' row) and the
// same 64 bytes of its token's LDS row; k-step j (0..3) multiplies word j of
// the codes, expanded to int8, with bytes 16j .. 16j+15 of those in one
// v_mfma_i32_32x32x32_i8 per 32 tokens (rows: weight row n0 + l % 32;
// columns: token 32mt + l % 32). The waves' int32 partial tiles are added in
// LDS (exact), then rescaled with the same fp32 expression as the large-M
// epilogue, so y and acc are bit-identical to it. Rows past N or M and
// columns at or past Kp read as zeros through the buffer range checks.

#include "device_common.h"
#include "internal.h"

namespace bitnet {

template <int MT>  // token tiles of 32: 1 for M <= 32, 2 for M <= 64
struct SkChunk {
  uint4 x[4 * MT];  // this thread's 16-byte pieces of the chunk's x_q columns (32 MT rows x 128 W bytes)
  uint4 codes;      // this lane's codes for its wave's super-step
};

// MT token tiles, W waves (a chunk is W super-steps), P chunks in flight.
template <int MT, int W, int P>
__global__ __launch_bounds__(kWave * W) void fwd_skinny_kernel(const int8_t* __restrict__ xq,
                                                                const float* __restrict__ s,
                                                                const uint8_t* __restrict__ wp,
                                                                const float* __restrict__ gamma, int M, int64_t N,
                                                                int64_t Kp, uint16_t* __restrict__ y,
                                                                int32_t* __restrict__ acc_out) {
  constexpr int kSkWaves = W, kSkThreads = kWave * W;
  constexpr int kSkChunk = 128 * W;           // k per chunk
  constexpr int kSkPitch = kSkChunk + 16;     // LDS bytes per token row
  constexpr int kRowPieces = kSkChunk / 16;   // 16-byte pieces per token row of a chunk
  constexpr int kPieces = 32 * MT * kRowPieces / kSkThreads;  // per thread
  constexpr int kTileB = 32 * MT * kSkPitch;
  constexpr int kRedB = kSkWaves * MT * 16 * kWave * 4;
  __shared__ __attribute__((aligned(16))) char smem[kTileB > kRedB ? kTileB : kRedB];
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int h = lane >> 5, r32 = lane & 31;
  const int64_t n0 = (int64_t)blockIdx.x * 32;
  const int nchunks = (int)((Kp + kSkChunk - 1) / kSkChunk);

  const rsrc_t rc = make_rsrc(wp, (uint32_t)(N * (Kp / 4)));
  const uint32_t coff = n0 + r32 < N ? (uint32_t)((n0 + r32) * (Kp / 4)) : kOob;  // the lane's codes row
  const rsrc_t rx = make_rsrc(xq, (uint32_t)(M * Kp));
  // piece p of a chunk: token row (p * kSkThreads + tid) / kRowPieces,
  // 16-byte column (p * kSkThreads + tid) % kRowPieces of the chunk
  static_assert(kPieces == 4 * MT, "32 MT rows x 128 W bytes in 16-byte pieces over 64 W threads");
  const auto load = [&](SkChunk<MT>& b, int c) {
#pragma unroll
    for (int p = 0; p < kPieces; ++p) {
      const int e = p * kSkThreads + tid, row = e / kRowPieces, col = 16 * (e % kRowPieces);
      const int64_t k = (int64_t)c * kSkChunk + col;
      b.x[p] = buf_load16(rx, row < M && k < Kp ? (uint32_t)(row * Kp + k) : kOob);
    }
    const int64_t k = (int64_t)c * kSkChunk + 128 * wave + 64 * h;
    b.codes = buf_load16(rc, k < Kp ? coff + (uint32_t)(k / 4) : kOob);
  };
  const auto stage = [&](const SkChunk<MT>& b) {
#pragma unroll
    for (int p = 0; p < kPieces; ++p) {
      const int e = p * kSkThreads + tid;
      *reinterpret_cast<uint4*>(smem + (e / kRowPieces) * kSkPitch + 16 * (e % kRowPieces)) = b.x[p];
    }
  };

  i32x16_t acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[mt][e] = 0;
  const auto compute = [&](const SkChunk<MT>& b) {
    const uint32_t w4[4] = {b.codes.x, b.codes.y, b.codes.z, b.codes.w};
    const char* xr = smem + r32 * kSkPitch + 128 * wave + 64 * h;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      i32x4_t a;
#pragma unroll
      for (int t = 0; t < 4; ++t) a[t] = (int)codes4_to_i8((w4[j] >> (2 * t)) & 0x03030303u);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const uint4 v = *reinterpret_cast<const uint4*>(xr + 32 * mt * kSkPitch + 16 * j);
        const i32x4_t bx = {(int)v.x, (int)v.y, (int)v.z, (int)v.w};
        acc[mt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, bx, acc[mt], 0, 0, 0);
      }
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
  int* red = reinterpret_cast<int*>(smem);  // [wave][mt][16][lane]
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int e = 0; e < 16; ++e) red[((wave * MT + mt) * 16 + e) * kWave + lane] = acc[mt][e];
  __syncthreads();

  // wave w finishes rows group g = w % 4 (n = n0 + 8g + 4h + 0..3) of token
  // tile w / 4: the sum over the waves (exact), then the rescale
  const int g = wave % 4, mt = wave / 4;
  if (mt >= MT) return;
  const int64_t m = 32 * mt + r32;
  if (m >= M) return;
  int v[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    int sum = 0;
#pragma unroll
    for (int w = 0; w < kSkWaves; ++w) sum += red[((w * MT + mt) * 16 + 4 * g + e) * kWave + lane];
    v[e] = sum;
  }
  const float c = s[m] * *gamma / 127.0f;
  const int64_t nb = n0 + 8 * g + 4 * h;
  uint16_t* yr = y + m * N;
  if (N % 4 == 0 && nb + 4 <= N) {
    *reinterpret_cast<uint2*>(yr + nb) =
        make_uint2(pack_bf16x2((float)v[0] * c, (float)v[1] * c), pack_bf16x2((float)v[2] * c, (float)v[3] * c));
    if (acc_out != nullptr) *reinterpret_cast<int4*>(acc_out + m * N + nb) = make_int4(v[0], v[1], v[2], v[3]);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (nb + e >= N) break;
      yr[nb + e] = f32_to_bf16_bits((float)v[e] * c);
      if (acc_out != nullptr) acc_out[m * N + nb + e] = v[e];
    }
  }
}

hipError_t launch_fwd_skinny(const int8_t* x_q, const float* s_x, const uint8_t* w_packed, const float* gamma,
                             int64_t M, int64_t N, int64_t K, uint16_t* y, int32_t* acc_out, hipStream_t stream) {
  if (M < 1 || M > kSkinnyMaxM) return hipErrorInvalidValue;
  const int64_t Kp = k_pad(K);
  const unsigned grid = (unsigned)((N + 31) / 32);
  if (M <= 32)
    fwd_skinny_kernel<1, 16, 3><<<grid, kWave * 16, 0, stream>>>(x_q, s_x, w_packed, gamma, (int)M, N, Kp, y, acc_out);
  else
    fwd_skinny_kernel<2, 8, 3><<<grid, kWave * 8, 0, stream>>>(x_q, s_x, w_packed, gamma, (int)M, N, Kp, y, acc_out);
  return hipGetLastError();
}

}  // namespace bitnet
