// MFMA GEMMs of the BitLinear layer for gfx950 (CDNA4, wave64).
//
// All three products are computed by one kernel template
//
//     C[i][j] = sum_r P[i][r] * Q[j][r],      output O[j][i] (i contiguous)
//
// with both operand tiles staged in LDS as [row][r] (reduction contiguous,
// 64 bytes of reduction per row per stage, rows padded to 80 bytes so that
// 16-byte fragment reads of 8 consecutive rows hit distinct banks). The
// staging step converts each operand from its stored form into MFMA-ready
// values once per block:
//
//   forward  y[m][n]  = sum_k x_q[m][k] q[n][k]        i = n, j = m, r = k
//            P = 2-bit codes unpacked to int8, Q = x_q copied;
//            v_mfma_i32_32x32x32_i8, exact int32 accumulation
//   dX       dX[m][k] = sum_n dY[m][n] W_hat[n][k]     i = k, j = m, r = n
//            P = codes transposed and unpacked to bf16 (+-1, 0), Q = dY
//            copied; v_mfma_f32_32x32x16_bf16; bf16(gamma) applied in the
//            epilogue (exact: q * bf16(gamma) is exact in bf16)
//   dW       dW[n][k] = sum_m dY[m][n] x_hat[m][k]     i = k, j = n, r = m
//            P = x_q transposed and rescaled to bf16 x_hat, Q = dY
//            transposed; v_mfma_f32_32x32x16_bf16
//
// ("bitnet-qat-train": opening bullets - INT8 forward, backward operands
// rebuilt transiently from the 2-bit / INT8 state; Semantics - forward
// formula and STE backward dX = dY W_hat, dW = dY^T x_hat.)
//
// Block tile 256 x 256, 8 waves in a 2 (i) x 4 (j) grid, wave tile 128 x 64
// = 4 x 2 fragments of 32 x 32. Two LDS stages (one barrier per stage) with
// the next stage's global loads held in registers while the current stage's
// MFMAs run.
//
// MFMA 32x32 output layout (both instructions): lane l, accumulator element
// v holds row i = 8*(v/4) + 4*(l/32) + (v%4), column j = l%32. Operand
// fragments: lane l supplies 16 bytes of row (l%32) of its operand at
// reduction chunk (l/32) of the step; the same slot-to-reduction-index map is
// used for P and Q, so the hardware's internal order of the reduction index
// within a step does not matter.

#include "device_common.h"
#include "internal.h"

namespace bitnet {

constexpr int kBI = 256, kBJ = 256;
constexpr int kThreads = 512;
constexpr int kWavesI = 2, kWavesJ = 4;
constexpr int kWTI = kBI / kWavesI;  // 128
constexpr int kWTJ = kBJ / kWavesJ;  // 64
constexpr int kFI = kWTI / 32;       // 4
constexpr int kFJ = kWTJ / 32;       // 2
constexpr int kStageBytes = 64;
constexpr int kPitch = kStageBytes + 16;
constexpr int kTileBytes = 256 * kPitch;

// ---------------------------------------------------------------------------
// MFMA flavours
// ---------------------------------------------------------------------------

struct MfmaI8 {
  typedef i32x4_t Frag;
  typedef i32x16_t Acc;
  static __device__ __forceinline__ Acc mma(Frag a, Frag b, Acc c) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
  }
};

struct MfmaBf16 {
  typedef bf16x8_t Frag;
  typedef f32x16_t Acc;
  static __device__ __forceinline__ Acc mma(Frag a, Frag b, Acc c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

// ---------------------------------------------------------------------------
// Operand loaders. load(): global -> registers for one stage (rows row0..+255
// of the operand, reduction stage s); store(): registers -> LDS tile.
// ---------------------------------------------------------------------------

// Row-major source already in MFMA element form with the reduction axis
// contiguous (x_q for the forward, dY for dX). 2 x 16 bytes per thread.
template <int kElem, bool VEC>
struct CopyLoader {
  const char* base;
  int64_t pitch;      // bytes between rows
  int64_t rows;       // valid rows
  int64_t red_bytes;  // valid reduction bytes per row
  struct Regs { uint4 v[2]; };

  __device__ __forceinline__ void load(Regs& r, int row0, int s, float*) const {
    const int tid = threadIdx.x;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = tid + h * kThreads;
      const int64_t row = row0 + (c >> 2);
      const int64_t kb = (int64_t)s * kStageBytes + (c & 3) * 16;
      const char* src = base + row * pitch + kb;
      if (row < rows && VEC && kb + 16 <= red_bytes) {
        r.v[h] = *reinterpret_cast<const uint4*>(src);
      } else if (row < rows && kb < red_bytes) {
        uint32_t d[4] = {0, 0, 0, 0};
        if constexpr (kElem == 1) {
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (kb + e < red_bytes) d[e >> 2] |= uint32_t(uint8_t(src[e])) << (8 * (e & 3));
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (kb + 2 * e < red_bytes)
              d[e >> 1] |= uint32_t(*reinterpret_cast<const uint16_t*>(src + 2 * e)) << (16 * (e & 1));
        }
        r.v[h] = make_uint4(d[0], d[1], d[2], d[3]);
      } else {
        r.v[h] = make_uint4(0, 0, 0, 0);
      }
    }
  }
  __device__ __forceinline__ void store(const Regs& r, char* lds, const float*) const {
    const int tid = threadIdx.x;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = tid + h * kThreads;
      *reinterpret_cast<uint4*>(lds + (c >> 2) * kPitch + (c & 3) * 16) = r.v[h];
    }
  }
};

// 4 codes of one packed byte -> 4 int8 in one word (byte p = code p).
__device__ __forceinline__ uint32_t unpack4_i8(uint32_t b) {
  uint32_t s = b | (b << 6) | (b << 12) | (b << 18);
  s &= 0x03030303u;
  // table: code 0 -> 0x00, 1 -> 0x01, 3 -> 0xFF (code 2 never written)
  return perm(0u, 0xFF000100u, s);
}

// Forward P: packed codes [N][Kp/4], rows n, reduction k contiguous.
// 8 packed bytes (32 codes) per thread -> 32 int8.
struct PackedRowLoader {
  const uint8_t* packed;
  int64_t pitch;  // Kp/4
  int64_t rows;   // N
  struct Regs { uint2 v; };

  __device__ __forceinline__ void load(Regs& r, int row0, int s, float*) const {
    const int tid = threadIdx.x;
    const int64_t row = row0 + (tid >> 1);
    if (row < rows)
      r.v = *reinterpret_cast<const uint2*>(packed + row * pitch + (int64_t)s * 16 + (tid & 1) * 8);
    else
      r.v = make_uint2(0, 0);
  }
  __device__ __forceinline__ void store(const Regs& r, char* lds, const float*) const {
    const int tid = threadIdx.x;
    char* dst = lds + (tid >> 1) * kPitch + (tid & 1) * 32;
    uint4 a, b;
    a.x = unpack4_i8(r.v.x & 0xFF); a.y = unpack4_i8((r.v.x >> 8) & 0xFF);
    a.z = unpack4_i8((r.v.x >> 16) & 0xFF); a.w = unpack4_i8(r.v.x >> 24);
    b.x = unpack4_i8(r.v.y & 0xFF); b.y = unpack4_i8((r.v.y >> 8) & 0xFF);
    b.z = unpack4_i8((r.v.y >> 16) & 0xFF); b.w = unpack4_i8(r.v.y >> 24);
    reinterpret_cast<uint4*>(dst)[0] = a;
    reinterpret_cast<uint4*>(dst)[1] = b;
  }
};

// dX P: W_hat^T from packed codes [N][Kp/4]: rows k, reduction n (strided).
// Thread (ng = tid/64, kq = tid%64) reads one packed byte (codes of k =
// 4kq..4kq+3) from each of the rows n = 4ng..4ng+3 and writes, for each of
// its 4 k, the 4 codes as bf16 (+1 = 0x3F80, -1 = 0xBF80, 0 = 0).
struct PackedTransposeLoader {
  const uint8_t* packed;
  int64_t pitch;  // Kp/4 bytes per n row
  int64_t nred;   // N (valid reduction rows)
  struct Regs { uint32_t b; };

  __device__ __forceinline__ void load(Regs& r, int row0, int s, float*) const {
    const int tid = threadIdx.x;
    const int64_t n = (int64_t)s * 32 + 4 * (tid >> 6);
    const int64_t col = (row0 >> 2) + (tid & 63);  // byte within the row
    uint32_t b = 0;
    if (col < pitch) {
      const uint8_t* src = packed + n * pitch + col;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (n + e < nred) b |= uint32_t(src[e * pitch]) << (8 * e);
    }
    r.b = b;
  }
  __device__ __forceinline__ void store(const Regs& r, char* lds, const float*) const {
    const int tid = threadIdx.x;
    const int kq = tid & 63, ng = tid >> 6;
    constexpr uint32_t kLo = 0x80008000u;  // low bytes of bf16(code) for codes 0..3
    constexpr uint32_t kHi = 0xBF003F00u;  // high bytes
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t c = (r.b >> (2 * p)) & 0x03030303u;  // codes of n0..n3 for k = 4kq+p
      const uint32_t s0 = perm(c, c, 0x01010000u) + 0x04000400u;
      const uint32_t s1 = perm(c, c, 0x03030202u) + 0x04000400u;
      uint2 o;
      o.x = perm(kHi, kLo, s0);
      o.y = perm(kHi, kLo, s1);
      *reinterpret_cast<uint2*>(lds + (4 * kq + p) * kPitch + 8 * ng) = o;
    }
  }
};

// dW Q: dY^T: rows n, reduction m (strided). Thread (mg = tid/64, nq =
// tid%64) reads 4 bf16 (n = 4nq..4nq+3) from each of the rows m = 4mg..+3
// and writes a 4x4 transpose.
template <bool VEC>
struct RowTransposeBf16Loader {
  const uint16_t* dy;
  int64_t ld;    // N
  int64_t mred;  // M (valid reduction rows)
  int64_t rows;  // N (valid rows)
  struct Regs { uint2 v[4]; };

  __device__ __forceinline__ void load(Regs& r, int row0, int s, float*) const {
    const int tid = threadIdx.x;
    const int64_t m = (int64_t)s * 32 + 4 * (tid >> 6);
    const int64_t n = row0 + 4 * (tid & 63);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint16_t* src = dy + (m + e) * ld + n;
      if (m + e < mred && VEC && n + 4 <= rows) {
        r.v[e] = *reinterpret_cast<const uint2*>(src);
      } else if (m + e < mred && n < rows) {
        uint32_t d[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) d[q] = (n + q < rows) ? src[q] : 0u;
        r.v[e] = make_uint2(d[0] | (d[1] << 16), d[2] | (d[3] << 16));
      } else {
        r.v[e] = make_uint2(0, 0);
      }
    }
  }
  __device__ __forceinline__ void store(const Regs& r, char* lds, const float*) const {
    const int tid = threadIdx.x;
    const int nq = tid & 63, mg = tid >> 6;
    char* dst = lds + (4 * nq) * kPitch + 8 * mg;
    // column q of the 4x4 block: (m0, m1) from halves of v[0], v[1]; (m2, m3) from v[2], v[3]
    uint2 o;
    o.x = perm(r.v[1].x, r.v[0].x, 0x05040100u);
    o.y = perm(r.v[3].x, r.v[2].x, 0x05040100u);
    *reinterpret_cast<uint2*>(dst + 0 * kPitch) = o;
    o.x = perm(r.v[1].x, r.v[0].x, 0x07060302u);
    o.y = perm(r.v[3].x, r.v[2].x, 0x07060302u);
    *reinterpret_cast<uint2*>(dst + 1 * kPitch) = o;
    o.x = perm(r.v[1].y, r.v[0].y, 0x05040100u);
    o.y = perm(r.v[3].y, r.v[2].y, 0x05040100u);
    *reinterpret_cast<uint2*>(dst + 2 * kPitch) = o;
    o.x = perm(r.v[1].y, r.v[0].y, 0x07060302u);
    o.y = perm(r.v[3].y, r.v[2].y, 0x07060302u);
    *reinterpret_cast<uint2*>(dst + 3 * kPitch) = o;
  }
};

// dW P: x_hat^T from x_q [M][Kp] and s[M]: rows k, reduction m (strided).
// x_hat = bf16(fl32(x_q * fl32(s/127))); for bf16 scales this equals the
// exactly rounded bf16(x_q * s / 127). Thread (mg, kq) reads 4 int8 (k =
// 4kq..+3) from rows m = 4mg..+3. The 32 scales of a stage are computed by
// the first 32 threads when the stage is loaded and published in LDS.
struct Int8TransposeScaleLoader {
  const int8_t* xq;
  const float* s;
  int64_t pitch;  // Kp
  int64_t mred;   // M
  struct Regs { uint32_t d[4]; };

  __device__ __forceinline__ void load(Regs& r, int row0, int st, float* scale_out) const {
    const int tid = threadIdx.x;
    const int64_t m = (int64_t)st * 32 + 4 * (tid >> 6);
    const int64_t k = row0 + 4 * (tid & 63);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      r.d[e] = (m + e < mred && k < pitch) ? *reinterpret_cast<const uint32_t*>(xq + (m + e) * pitch + k) : 0u;
    if (tid < 32) {
      const int64_t mm = (int64_t)st * 32 + tid;
      scale_out[tid] = (mm < mred) ? s[mm] / 127.0f : 0.0f;
    }
  }
  __device__ __forceinline__ void store(const Regs& r, char* lds, const float* scale_in) const {
    const int tid = threadIdx.x;
    const int kq = tid & 63, mg = tid >> 6;
    float rs[4], off[4];
    uint32_t u[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      rs[e] = scale_in[4 * mg + e];
      off[e] = -128.0f * rs[e];       // exact
      u[e] = r.d[e] ^ 0x80808080u;    // bytes x_q + 128 in [1, 255]
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float f = (float)((u[e] >> (8 * p)) & 0xFFu);
        v[e] = fmaf(f, rs[e], off[e]);  // = fl32(x_q * r): single rounding of the exact value
      }
      uint2 o;
      o.x = pack_bf16x2(v[0], v[1]);
      o.y = pack_bf16x2(v[2], v[3]);
      *reinterpret_cast<uint2*>(lds + (4 * kq + p) * kPitch + 8 * mg) = o;
    }
  }
};

// ---------------------------------------------------------------------------
// Epilogues: acc (wave tile origin i0, j0) -> memory. Lane l holds, for each
// fragment (fi, fj) and group g, the 4 consecutive i = i0 + 32fi + 8g +
// 4(l/32) + 0..3 at j = j0 + 32fj + l%32.
// ---------------------------------------------------------------------------

struct FwdEpilogue {
  uint16_t* y;
  int32_t* acc_out;
  const float* s;
  const float* gamma;
  int64_t I, J;  // N, M
  bool vec;      // N % 4 == 0

  __device__ __forceinline__ void store(MfmaI8::Acc (&acc)[kFI][kFJ], int i0, int j0, int lane) const {
    const float g = *gamma;
#pragma unroll
    for (int fj = 0; fj < kFJ; ++fj) {
      const int64_t j = j0 + 32 * fj + (lane & 31);
      if (j >= J) continue;
      const float c = s[j] * g / 127.0f;
#pragma unroll
      for (int fi = 0; fi < kFI; ++fi) {
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
          const int64_t i = i0 + 32 * fi + 8 * gi + 4 * (lane >> 5);
          if (i >= I) continue;
          const int a0 = acc[fi][fj][4 * gi + 0], a1 = acc[fi][fj][4 * gi + 1];
          const int a2 = acc[fi][fj][4 * gi + 2], a3 = acc[fi][fj][4 * gi + 3];
          const float v0 = (float)a0 * c, v1 = (float)a1 * c, v2 = (float)a2 * c, v3 = (float)a3 * c;
          uint16_t* dst = y + j * I + i;
          if (vec && i + 4 <= I) {
            *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
            if (acc_out) *reinterpret_cast<int4*>(acc_out + j * I + i) = make_int4(a0, a1, a2, a3);
          } else {
            const float vv[4] = {v0, v1, v2, v3};
            const int aa[4] = {a0, a1, a2, a3};
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (i + q < I) {
                dst[q] = f32_to_bf16_bits(vv[q]);
                if (acc_out) acc_out[j * I + i + q] = aa[q];
              }
          }
        }
      }
    }
  }
};

// dX (bf16 out, scaled by bf16(gamma)) and dW (bf16 or f32 out, unscaled).
template <bool OUT_F32>
struct Bf16Epilogue {
  void* out;
  const float* gamma;  // NULL: no scale
  int64_t I, J;        // output [J][I]
  bool vec;            // I % 4 == 0

  __device__ __forceinline__ void store(MfmaBf16::Acc (&acc)[kFI][kFJ], int i0, int j0, int lane) const {
    float sc = 1.0f;
    if (gamma) sc = bf16_to_f32(f32_to_bf16_bits(*gamma));  // bf16(gamma), exact in fp32
#pragma unroll
    for (int fj = 0; fj < kFJ; ++fj) {
      const int64_t j = j0 + 32 * fj + (lane & 31);
      if (j >= J) continue;
#pragma unroll
      for (int fi = 0; fi < kFI; ++fi) {
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
          const int64_t i = i0 + 32 * fi + 8 * gi + 4 * (lane >> 5);
          if (i >= I) continue;
          float v[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = acc[fi][fj][4 * gi + q] * sc;
          if constexpr (OUT_F32) {
            float* dst = static_cast<float*>(out) + j * I + i;
            if (vec && i + 4 <= I) {
              *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
            } else {
#pragma unroll
              for (int q = 0; q < 4; ++q)
                if (i + q < I) dst[q] = v[q];
            }
          } else {
            uint16_t* dst = static_cast<uint16_t*>(out) + j * I + i;
            if (vec && i + 4 <= I) {
              *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
            } else {
#pragma unroll
              for (int q = 0; q < 4; ++q)
                if (i + q < I) dst[q] = f32_to_bf16_bits(v[q]);
            }
          }
        }
      }
    }
  }
};

// ---------------------------------------------------------------------------
// Block -> tile. Workgroups are dispatched round-robin over the 8 XCDs
// (block b on XCD b % 8); each XCD gets a contiguous range of tiles so that
// the blocks sharing an L2 share operand panels. Within the range, i varies
// fastest.
// ---------------------------------------------------------------------------

__device__ __forceinline__ void map_tile(int b, int tiles_i, int tiles_j, int& ti, int& tj) {
  const int T = tiles_i * tiles_j;
  const int q = T / 8, r = T % 8;
  const int x = b % 8, k = b / 8;
  const int v = (x < r) ? x * (q + 1) + k : r * (q + 1) + (x - r) * q + k;
  ti = v % tiles_i;
  tj = v / tiles_i;
}

template <class Acc>
__device__ __forceinline__ void zero_acc(Acc& a) {
#pragma unroll
  for (int e = 0; e < 16; ++e) a[e] = 0;
}

template <class MT, class PL, class QL, class EP>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(PL pl, QL ql, EP ep, int tiles_i,
                                                          int tiles_j, int nstages) {
  __shared__ __attribute__((aligned(16))) char smem[2][2][kTileBytes];
  __shared__ float sscale[2][32];

  int ti, tj;
  map_tile(blockIdx.x, tiles_i, tiles_j, ti, tj);
  const int i0 = ti * kBI, j0 = tj * kBJ;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wi = wave % kWavesI, wj = wave / kWavesI;

  typename MT::Acc acc[kFI][kFJ];
#pragma unroll
  for (int fi = 0; fi < kFI; ++fi)
#pragma unroll
    for (int fj = 0; fj < kFJ; ++fj) zero_acc(acc[fi][fj]);

  typename PL::Regs pr;
  typename QL::Regs qr;
  pl.load(pr, i0, 0, sscale[0]);
  ql.load(qr, j0, 0, sscale[0]);
  __syncthreads();  // per-stage scales published by load()
  pl.store(pr, smem[0][0], sscale[0]);
  ql.store(qr, smem[0][1], sscale[0]);
  if (nstages > 1) {
    pl.load(pr, i0, 1, sscale[1]);
    ql.load(qr, j0, 1, sscale[1]);
  }
  __syncthreads();

  const int prow = wi * kWTI + (lane & 31);
  const int qrow = wj * kWTJ + (lane & 31);
  for (int s = 0; s < nstages; ++s) {
    const char* Pt = smem[s & 1][0];
    const char* Qt = smem[s & 1][1];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int chunk = 2 * ks + (lane >> 5);
      typename MT::Frag a[kFI], b[kFJ];
#pragma unroll
      for (int fi = 0; fi < kFI; ++fi)
        a[fi] = *reinterpret_cast<const typename MT::Frag*>(Pt + (prow + 32 * fi) * kPitch + chunk * 16);
#pragma unroll
      for (int fj = 0; fj < kFJ; ++fj)
        b[fj] = *reinterpret_cast<const typename MT::Frag*>(Qt + (qrow + 32 * fj) * kPitch + chunk * 16);
#pragma unroll
      for (int fi = 0; fi < kFI; ++fi)
#pragma unroll
        for (int fj = 0; fj < kFJ; ++fj) acc[fi][fj] = MT::mma(a[fi], b[fj], acc[fi][fj]);
    }
    if (s + 1 < nstages) {
      pl.store(pr, smem[(s + 1) & 1][0], sscale[(s + 1) & 1]);
      ql.store(qr, smem[(s + 1) & 1][1], sscale[(s + 1) & 1]);
    }
    if (s + 2 < nstages) {
      pl.load(pr, i0, s + 2, sscale[s & 1]);
      ql.load(qr, j0, s + 2, sscale[s & 1]);
    }
    __syncthreads();
  }
  ep.store(acc, i0 + wi * kWTI, j0 + wj * kWTJ, lane);
}

template <class MT, class PL, class QL, class EP>
static hipError_t run_gemm(const PL& pl, const QL& ql, const EP& ep, int64_t I, int64_t J,
                           int64_t nstages, hipStream_t stream) {
  const int tiles_i = (int)((I + kBI - 1) / kBI);
  const int tiles_j = (int)((J + kBJ - 1) / kBJ);
  gemm_kernel<MT, PL, QL, EP><<<tiles_i * tiles_j, kThreads, 0, stream>>>(pl, ql, ep, tiles_i, tiles_j,
                                                                         (int)nstages);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

hipError_t launch_fwd(const int8_t* x_q, const float* s_x, const uint8_t* w_packed,
                      const float* gamma, int64_t M, int64_t N, int64_t K, uint16_t* y,
                      int32_t* acc_out, hipStream_t stream) {
  const int64_t Kp = k_pad(K);
  PackedRowLoader pl{w_packed, Kp / 4, N};
  CopyLoader<1, true> ql{reinterpret_cast<const char*>(x_q), Kp, M, Kp};
  FwdEpilogue ep{y, acc_out, s_x, gamma, N, M, N % 4 == 0};
  return run_gemm<MfmaI8>(pl, ql, ep, N, M, Kp / 64, stream);
}

hipError_t launch_bwd_dx(const uint16_t* dY, const uint8_t* w_packed, const float* gamma,
                         int64_t M, int64_t N, int64_t K, uint16_t* dX, hipStream_t stream) {
  const int64_t Kp = k_pad(K);
  PackedTransposeLoader pl{w_packed, Kp / 4, N};
  Bf16Epilogue<false> ep{dX, gamma, K, M, K % 4 == 0};
  const int64_t nst = (N + 31) / 32;
  if (N % 8 == 0) {
    CopyLoader<2, true> ql{reinterpret_cast<const char*>(dY), 2 * N, M, 2 * N};
    return run_gemm<MfmaBf16>(pl, ql, ep, K, M, nst, stream);
  }
  CopyLoader<2, false> ql{reinterpret_cast<const char*>(dY), 2 * N, M, 2 * N};
  return run_gemm<MfmaBf16>(pl, ql, ep, K, M, nst, stream);
}

hipError_t launch_bwd_dw(const uint16_t* dY, const int8_t* x_q, const float* s_x, int64_t M,
                         int64_t N, int64_t K, void* dW, bool dw_is_f32, hipStream_t stream) {
  const int64_t Kp = k_pad(K);
  Int8TransposeScaleLoader pl{x_q, s_x, Kp, M};
  const int64_t nst = (M + 31) / 32;
  const bool vec = (N % 4 == 0);
  if (dw_is_f32) {
    Bf16Epilogue<true> ep{dW, nullptr, K, N, K % 4 == 0};
    if (vec) return run_gemm<MfmaBf16>(pl, RowTransposeBf16Loader<true>{dY, N, M, N}, ep, K, N, nst, stream);
    return run_gemm<MfmaBf16>(pl, RowTransposeBf16Loader<false>{dY, N, M, N}, ep, K, N, nst, stream);
  }
  Bf16Epilogue<false> ep{dW, nullptr, K, N, K % 4 == 0};
  if (vec) return run_gemm<MfmaBf16>(pl, RowTransposeBf16Loader<true>{dY, N, M, N}, ep, K, N, nst, stream);
  return run_gemm<MfmaBf16>(pl, RowTransposeBf16Loader<false>{dY, N, M, N}, ep, K, N, nst, stream);
}

}  // namespace bitnet
