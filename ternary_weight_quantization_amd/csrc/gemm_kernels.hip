// MFMA GEMMs of the BitLinear layer for gfx950 (CDNA4, wave64).
//
// All three products are computed by one kernel template
//
//     C[i][j] = sum_r P[i][r] * Q[j][r],      output O[j][i] (i contiguous)
//
// with both operand tiles staged in LDS, 64 bf16 or 128 int8 reduction
// values per row per stage:
//
//   forward  y[m][n]  = sum_k x_q[m][k] q[n][k]        i = n, j = m, r = k
//            P = the 2-bit codes as stored (expanded to int8 after the
//            fragment read), Q = x_q copied; v_mfma_i32_32x32x32_i8, exact
//            int32 accumulation
//   dX       dX[m][k] = sum_n dY[m][n] W_hat[n][k]     i = k, j = m, r = n
//            P = the codes transposed to fp4 [k][n] by a pre-pass (expanded
//            to bf16 +-1, 0 after the fragment read), Q = dY copied;
//            v_mfma_f32_32x32x16_bf16; bf16(gamma) applied in the epilogue
//            (exact: q * bf16(gamma) is exact in bf16)
//   dW       dW[n][k] = sum_m dY[m][n] x_hat[m][k]     i = k, j = n, r = m
//            P = bf16 x_hat built by a pre-pass, Q = dY, both staged in
//            their [m][.] orientation and read transposed from LDS
//            (ds_read_b64_tr_b16); v_mfma_f32_32x32x16_bf16
//
// ("bitnet-qat-train": opening bullets - INT8 forward, backward operands
// rebuilt transiently from the 2-bit / INT8 state; Semantics - forward
// formula and STE backward dX = dY W_hat, dW = dY^T x_hat.)
//
// The LDS traffic, not the MFMA rate, bounds these kernels on gfx950 (about
// 128 B/clk/CU of 16-byte reads and 64 B/clk/CU of 16-byte writes), so the
// ternary operand stays 2-bit in LDS and is expanded in registers.
//
// Block tile 256 x 256, 4 waves (one per SIMD) in a 2 x 2 grid, wave tile
// 128 x 128 = 4 x 4 fragments of 32 x 32 (256 accumulator registers per
// lane, held in AGPRs). Two LDS stages (one barrier per stage); while the
// MFMAs of stage s run, the registers holding stage s+1 are converted and
// stored into the other LDS buffer and stage s+2 is fetched into them, one
// quarter per k-step.
//
// MFMA 32x32 output layout (both instructions): lane l, accumulator element
// v holds row i = 8*(v/4) + 4*(l/32) + (v%4), column j = l%32. Operand
// fragments: lane l supplies 16 bytes of row (l%32) of its operand for lane
// half h = l/32 of the k-step; which reduction values those are (red_chunk)
// is the same for P and Q of a GEMM, so the hardware's internal order of the
// reduction index within a step does not matter.

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdlib>
#include <mutex>
#include <random>
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace bitnet {

constexpr int kBI = 256, kBJ = 256;
constexpr int kThreads = 256;        // 4 waves, one per SIMD
constexpr int kWavesI = 2, kWavesJ = 2;
constexpr int kWTI = kBI / kWavesI;  // 128
constexpr int kWTJ = kBJ / kWavesJ;  // 128
constexpr int kFI = kWTI / 32;       // 4
constexpr int kFJ = kWTJ / 32;       // 4
constexpr int kStageBytes = 128;     // operand bytes per row per stage (bf16 or int8)
constexpr int kKSteps = kStageBytes / 32;
constexpr int kPitch = kStageBytes + 16;  // plain tiles: 9 chunks of 16 bytes
constexpr int kRed16 = kStageBytes / 2;   // bf16 reduction elements per stage

// Byte offset of 16-byte chunk c (0..7) of a plain LDS tile row r. Tiles
// written by the transposing loaders (one chunk of many rows at a time)
// XOR-swizzle the chunk index with bits 4..6 of the row so those stores
// spread over the banks; the other tiles are stored plainly.
template <bool SWZ>
__device__ __forceinline__ int lds_off(int r, int c) {
  return r * kPitch + ((SWZ ? (c ^ ((r >> 4) & 7)) : c) << 4);
}

// 16-byte reduction chunk (8 bf16 or 16 int8 values) that lane half h
// supplies at k-step ks. MAP 0: chunk 2ks + h; MAP 1: chunk 4h + ks.
template <int MAP>
__device__ __forceinline__ constexpr int red_chunk(int ks, int h) {
  return MAP == 0 ? 2 * ks + h : 4 * h + ks;
}

// ---------------------------------------------------------------------------
// MFMA flavours
// ---------------------------------------------------------------------------

struct MfmaI8 {
  typedef i32x4_t Frag;
  typedef i32x16_t Acc;
  typedef int Elem;
  static constexpr uint32_t kPoisonBits = 0x80000000u;  // INT32_MIN
  static __device__ __forceinline__ Elem from_bits(uint32_t b) { return (int)b; }
  static __device__ __forceinline__ uint32_t to_bits(Elem e) { return (uint32_t)e; }
  static __device__ __forceinline__ Acc mma(Frag a, Frag b, Acc c) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
  }
};

struct MfmaBf16 {
  typedef bf16x8_t Frag;
  typedef f32x16_t Acc;
  typedef float Elem;
  static constexpr uint32_t kPoisonBits = 0x7FC00000u;  // quiet NaN
  static __device__ __forceinline__ Elem from_bits(uint32_t b) { return __uint_as_float(b); }
  static __device__ __forceinline__ uint32_t to_bits(Elem e) { return __float_as_uint(e); }
  static __device__ __forceinline__ Acc mma(Frag a, Frag b, Acc c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Fragment readers: the kFI (or kFJ) fragments of a wave for each k-step.
// A k-step is 16 MFMA slots (see gemm_slot); slot<KS, U>() runs after the
// MFMA of slot U and issues this reader's share of the work for later
// slots: the LDS reads of the next k-step's fragments and, for code
// operands, the expansion of fragment f + 1 during the slots of fragment f
// (and of the next k-step's fragment 0 during the last four). k-step 0 of a
// stage is prepared during the last k-step of the previous stage, by the
// reader of the other LDS buffer: ahead<U>() is the share of slot U (after
// the stage's barrier) of the LDS reads and expansion k-step 0 needs.
// frag<KS>(f) is fragment f of k-step KS, ready by the first slot that uses
// it. init() points the reader at the tile of one LDS buffer.
// ---------------------------------------------------------------------------

// The end-of-stage barrier sits in slot kBarrierSlot of the last k-step:
// by then every LDS store of the staged next stage has been issued (each
// loader's kLastStoreSlot is earlier) and the last k-step reads no LDS, so
// the next stage's k-step 0 reads can start right after it and overlap the
// remaining MFMAs of this stage.
constexpr int kBarrierSlot = 8;
static_assert(kBarrierSlot + 7 == 15, "ahead<U> covers the slots after the barrier");

// When the plain (LDS-read) fragments are read. Slot U of k-step KS uses P
// fragment U/4 and Q fragment U%4, so the Q fragments of a k-step are all
// needed in its first four slots and the P fragments in slots 0, 4, 8, 12.
// The next k-step's fragments are read in the first half of the current
// one, Q first, so that each is requested at least 9 slots before its use:
// P fragment f in slot next_read_slot<false>(f), Q fragment f in
// next_read_slot<true>(f); the next stage's k-step 0 fragments are read
// after the stage barrier in the same order (ahead_slot).
template <bool Q>
__device__ __forceinline__ constexpr int next_read_slot(int f) { return Q ? f : (f == 0 ? 0 : 3 + f); }
template <bool Q>
__device__ __forceinline__ constexpr int ahead_slot(int f) {
  return kBarrierSlot + 1 + (Q ? f / 2 : (f == 0 ? 0 : 1 + f));
}
static_assert(ahead_slot<false>(3) < 16, "");

// 16-byte fragments read directly from a plain tile (pitch kPitch).
template <class MT, bool SWZ, int MAP>
struct PlainFrags {
  typename MT::Frag buf[2][4];
  const char* base;
  __device__ __forceinline__ void init(const char* tile, int row0, int lane) {
    // row0 is a multiple of 128, so the swizzle of row row0 + 32f + (l%32)
    // is 2f + bit 4 of l (fragment offsets below)
    const int h = lane >> 5;
    if constexpr (SWZ) {
      static_assert(MAP == 0, "swizzled tiles use chunk map 0");
      base = tile + (row0 + (lane & 31)) * kPitch + 16 * (h ^ ((lane >> 4) & 1));
    } else {
      base = tile + (row0 + (lane & 31)) * kPitch + 16 * red_chunk<MAP>(0, h);
    }
  }
  template <int KS>
  static __device__ __forceinline__ constexpr int off(int f) {
    return SWZ ? f * 32 * kPitch + 32 * (KS ^ f) : f * 32 * kPitch + 16 * (MAP == 0 ? 2 * KS : KS);
  }
  template <int KS>
  __device__ __forceinline__ void read(int f) {
    buf[KS & 1][f] = *reinterpret_cast<const typename MT::Frag*>(base + off<KS>(f));
  }
  template <int U, bool Q>
  __device__ __forceinline__ void ahead() {
    if constexpr (U == ahead_slot<Q>(0)) read<0>(0);
    if constexpr (U == ahead_slot<Q>(1)) read<0>(1);
    if constexpr (U == ahead_slot<Q>(2)) read<0>(2);
    if constexpr (U == ahead_slot<Q>(3)) read<0>(3);
  }
  template <int KS, int U, bool Q>
  __device__ __forceinline__ void slot() {
    if constexpr (KS + 1 < kKSteps) {
      if constexpr (U == next_read_slot<Q>(0)) read<KS + 1>(0);
      if constexpr (U == next_read_slot<Q>(1)) read<KS + 1>(1);
      if constexpr (U == next_read_slot<Q>(2)) read<KS + 1>(2);
      if constexpr (U == next_read_slot<Q>(3)) read<KS + 1>(3);
    }
  }
  template <int KS>
  __device__ __forceinline__ typename MT::Frag frag(int f) const { return buf[KS & 1][f]; }
};

// Forward P: rows of 2-bit codes in the stored layout (tile pitch 48 bytes,
// 32 bytes = 8 words = 128 codes per row per stage). Lane half h of k-step
// ks takes word 4h + ks (codes k = 16(4h+ks)..+15, chunk map 1); one 16-byte
// read per fragment per stage, expanded word by word with
// (w >> 2t) & 0x03030303.
struct CodesI8Frags {
  static constexpr int kPitchB = 48;
  uint4 raw[4];
  MfmaI8::Frag cur[2][4];
  const char* base;
  __device__ __forceinline__ void init(const char* tile, int row0, int lane) {
    base = tile + (row0 + (lane & 31)) * kPitchB + 16 * (lane >> 5);
  }
  template <int KS, int F, int T>
  __device__ __forceinline__ void expand() {
    const uint32_t w = KS == 0 ? raw[F].x : KS == 1 ? raw[F].y : KS == 2 ? raw[F].z : raw[F].w;
    cur[KS & 1][F][T] = (int)codes4_to_i8((w >> (2 * T)) & 0x03030303u);
  }
  template <int U, bool Q>
  __device__ __forceinline__ void ahead() {
    static_assert(kBarrierSlot + 2 < 12, "raw words must be read before slot 12");
    if constexpr (U == kBarrierSlot + 1 || U == kBarrierSlot + 2) {
      constexpr int f0 = 2 * (U - kBarrierSlot - 1);
      raw[f0] = *reinterpret_cast<const uint4*>(base + f0 * 32 * kPitchB);
      raw[f0 + 1] = *reinterpret_cast<const uint4*>(base + (f0 + 1) * 32 * kPitchB);
    }
    if constexpr (U >= 12) expand<0, 0, U - 12>();
  }
  template <int KS, int U, bool Q>
  __device__ __forceinline__ void slot() {
    if constexpr (U / 4 < 3) expand<KS, U / 4 + 1, U % 4>();
    else if constexpr (KS + 1 < kKSteps) expand<KS + 1, 0, U % 4>();
  }
  template <int KS>
  __device__ __forceinline__ MfmaI8::Frag frag(int f) const { return cur[KS & 1][f]; }
};

// dX P: the ternary codes transposed to [k][n] as fp4 (E2M1) nibbles in n
// order (tile pitch 48 bytes, 32 bytes = 64 n per row per stage): +1 = 0x2,
// -1 = 0xA, 0 = 0x0, n even in the low nibble. Lane half h of k-step ks
// takes n = 32h + 8ks..+7 (chunk map 1), dword ks of the 16 bytes at 16h:
// one 16-byte read per fragment per stage. A fragment is expanded by four
// v_cvt_scalef32_pk_bf16_fp4 (scale 1: exact +-1, 0), one per slot.
struct CodesFp4Frags {
  static constexpr int kPitchB = 48;
  uint4 raw[4];
  u32x4_t cur[2][4];
  const char* base;
  __device__ __forceinline__ void init(const char* tile, int row0, int lane) {
    base = tile + (row0 + (lane & 31)) * kPitchB + 16 * (lane >> 5);
  }
  template <int KS, int F, int T>
  __device__ __forceinline__ void expand() {
    const uint32_t w = KS == 0 ? raw[F].x : KS == 1 ? raw[F].y : KS == 2 ? raw[F].z : raw[F].w;
    cur[KS & 1][F][T] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, T));
  }
  template <int U, bool Q>
  __device__ __forceinline__ void ahead() {
    static_assert(kBarrierSlot + 2 < 12, "raw words must be read before slot 12");
    if constexpr (U == kBarrierSlot + 1 || U == kBarrierSlot + 2) {
      constexpr int f0 = 2 * (U - kBarrierSlot - 1);
      raw[f0] = *reinterpret_cast<const uint4*>(base + f0 * 32 * kPitchB);
      raw[f0 + 1] = *reinterpret_cast<const uint4*>(base + (f0 + 1) * 32 * kPitchB);
    }
    if constexpr (U >= 12) expand<0, 0, U - 12>();
  }
  template <int KS, int U, bool Q>
  __device__ __forceinline__ void slot() {
    if constexpr (U / 4 < 3) expand<KS, U / 4 + 1, U % 4>();
    else if constexpr (KS + 1 < kKSteps) expand<KS + 1, 0, U % 4>();
  }
  template <int KS>
  __device__ __forceinline__ MfmaBf16::Frag frag(int f) const {
    return __builtin_bit_cast(MfmaBf16::Frag, cur[KS & 1][f]);
  }
};

// ---------------------------------------------------------------------------
// Operand loaders. load(): global -> registers for one stage (rows row0..+255
// of the operand, reduction stage s); store(): registers -> LDS tile (used
// for the first stage); slot<KS, U>(): the share of MFMA slot U of k-step KS
// in staging the next stage from registers into LDS and fetching the stage
// after it.
// Out-of-range data (rows past the operand, reduction past its end, stages
// past the last) reads as zeros through the buffer resource range check or
// an out-of-range offset, so the loads of a stage are issued without
// branches. Each thread's addresses are a per-thread base plus offsets that
// are uniform or compile-time.
// ---------------------------------------------------------------------------

// Row-major source already in MFMA element form with the reduction axis
// contiguous (x_q for the forward, dY for dX). Thread t handles chunk t%8 of
// rows 8(t/8)+h, h < 8; a wave instruction covers 8 rows x 128 bytes.
// FULL: the valid reduction extent is a multiple of 16 bytes. S0: first
// staging slot (1, or 5 when the other operand is a CopyLoader too).
template <int kElem, bool FULL, int S0 = 1>
struct CopyLoader {
  static constexpr bool kSwz = false;
  static constexpr int kTileB = 256 * kPitch;
  template <class MT, int MAP>
  using Frags = PlainFrags<MT, false, MAP>;
  const char* base;
  int64_t pitch;      // bytes between rows
  int64_t rows;       // valid rows
  int64_t red_bytes;  // valid reduction bytes per row
  // lane_off: byte offset of the thread's chunk of its first row in stage 0
  // (below 2^31: every operand read this way satisfies
  // (rows + 256) * pitch <= 2^31)
  struct Regs { uint4 v[8]; uint32_t lane_off; };

  // Offset of row h of the thread's 8 in stage s, or an out-of-range offset
  // for a chunk past the reduction (and every chunk of a stage past the
  // last): 32-bit arithmetic on a per-lane base and uniform terms, so that
  // the main loop keeps no 64-bit per-lane values.
  __device__ __forceinline__ uint32_t stage_off(const Regs& r, int s, int h) const {
    const int lim = (int)red_bytes - s * kStageBytes;
    return (int)(threadIdx.x & 7) * 16 < lim ? r.lane_off + (uint32_t)(s * kStageBytes) + (uint32_t)(h * pitch) : kOob;
  }

  __device__ __forceinline__ void load(Regs& r, int row0, int s) const {
    const int tid = threadIdx.x;
    const int64_t rowb = row0 + 8 * (tid >> 3);
    if constexpr (FULL) {
      // rows past the end fall outside the resource; chunks past the
      // reduction (and stages past the last) get an out-of-range offset
      const rsrc_t rs = make_rsrc(base, (uint32_t)(rows * pitch));
      r.lane_off = (uint32_t)(rowb * pitch) + (uint32_t)((tid & 7) * 16);
#pragma unroll
      for (int h = 0; h < 8; ++h) r.v[h] = buf_load16(rs, stage_off(r, s, h));
    } else {
      const int64_t kb = (int64_t)s * kStageBytes + (tid & 7) * 16;
      const char* p = base + rowb * pitch + kb;
#pragma unroll
      for (int h = 0; h < 8; ++h) {
        uint32_t d[4] = {0, 0, 0, 0};
        if (kb < red_bytes && rowb + h < rows) {
          const char* src = p + h * pitch;
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
        }
        r.v[h] = make_uint4(d[0], d[1], d[2], d[3]);
      }
    }
  }
  __device__ __forceinline__ void store(const Regs& r, char* lds) const {
    const int tid = threadIdx.x;
    char* dst = lds + lds_off<kSwz>(8 * (tid >> 3), tid & 7);
#pragma unroll
    for (int h = 0; h < 8; ++h) *reinterpret_cast<uint4*>(dst + h * kPitch) = r.v[h];
  }

  // Staging of the next stage, spread over the slots of k-step KS: rows
  // 2KS, 2KS+1 of the thread's block are stored (slots S0, S0+2), then
  // refilled with stage s+2 (slots S0+8, S0+10).
  struct Tmp {};
  static constexpr int kLastStoreSlot = S0 + 2;
  static_assert(S0 + 10 < 16, "the refills fit the k-step");
  template <int KS, int U>
  __device__ __forceinline__ void slot(Regs& r, Tmp&, char* lds, int row0, int s2) const {
    const int tid = threadIdx.x;
    if constexpr (U == S0 || U == S0 + 2) {
      constexpr int h = 2 * KS + (U == S0 + 2);
      *reinterpret_cast<uint4*>(lds + lds_off<kSwz>(8 * (tid >> 3), tid & 7) + h * kPitch) = r.v[h];
    }
    if constexpr (FULL && (U == S0 + 8 || U == S0 + 10)) {
      constexpr int h = 2 * KS + (U == S0 + 10);
      const rsrc_t rs = make_rsrc(base, (uint32_t)(rows * pitch));
      r.v[h] = buf_load16(rs, stage_off(r, s2, h));
    }
    if constexpr (!FULL && KS == kKSteps - 1 && U == S0 + 8) load(r, row0, s2);
  }
};

// A narrow code operand copied as stored, 32 bytes per row per stage: the
// forward's 2-bit codes [N][Kp/4] (rows n; F = CodesI8Frags) or dX's fp4
// transposed codes [Kp][Np/2] (rows k; F = CodesFp4Frags). Thread t handles
// row t: two 16-byte loads.
template <class F>
struct RowCodesLoader {
  static constexpr bool kSwz = false;
  static constexpr int kTileB = 256 * F::kPitchB;
  template <class MT, int MAP>
  using Frags = F;
  const uint8_t* packed;
  int64_t pitch;  // bytes per row (a multiple of 16)
  int64_t rows;   // valid rows
  // lane_off: byte offset of the thread's row (below 2^31, as every operand
  // read through a buffer resource)
  struct Regs { uint4 v[2]; uint32_t lane_off; };
  struct Tmp {};

  // Half h of the thread's row in stage s; a column past the row (a stage
  // past the last) gets an out-of-range offset. The column test is uniform.
  __device__ __forceinline__ uint32_t offset(const Regs& r, int s, int h) const {
    const int col = s * (kStageBytes / 4) + 16 * h;
    return col < (int)pitch ? r.lane_off + (uint32_t)col : kOob;
  }
  __device__ __forceinline__ void load(Regs& r, int row0, int s) const {
    const rsrc_t rs = make_rsrc(packed, (uint32_t)(rows * pitch));
    r.lane_off = (uint32_t)((row0 + threadIdx.x) * pitch);
#pragma unroll
    for (int h = 0; h < 2; ++h) r.v[h] = buf_load16(rs, offset(r, s, h));
  }
  __device__ __forceinline__ void store(const Regs& r, char* lds) const {
    char* dst = lds + threadIdx.x * F::kPitchB;
    *reinterpret_cast<uint4*>(dst) = r.v[0];
    *reinterpret_cast<uint4*>(dst + 16) = r.v[1];
  }
  // K-steps 0 and 1 store one half of the row (slot 5) and refill it with
  // stage s+2 (slot 13).
  static constexpr int kLastStoreSlot = -1;
  template <int KS, int U>
  __device__ __forceinline__ void slot(Regs& r, Tmp&, char* lds, int row0, int s2) const {
    if constexpr (KS < 2 && U == 5)
      *reinterpret_cast<uint4*>(lds + threadIdx.x * F::kPitchB + 16 * KS) = r.v[KS];
    if constexpr (KS < 2 && U == 13) {
      const rsrc_t rs = make_rsrc(packed, (uint32_t)(rows * pitch));
      r.v[KS] = buf_load16(rs, offset(r, s2, KS));
    }
  }
};
using PackedCodesLoader = RowCodesLoader<CodesI8Frags>;

// dW operands from a bf16 [rows m][ld] matrix read transposed: rows j
// (n of dY for Q, k of x_hat for P), reduction m (strided). Thread
// (mg = wave, nq = lane) reads 4 bf16 (columns 4nq..4nq+3) from each of the
// rows m = 16mg..16mg+15 and writes the 16 x 4 transpose as 4 rows of 16 m
// values.
template <bool VEC, int W0>
struct RowTransposeBf16Loader {
  static constexpr bool kSwz = true;
  static constexpr int kTileB = 256 * kPitch;
  template <class MT, int MAP>
  using Frags = PlainFrags<MT, true, MAP>;
  const uint16_t* dy;
  int64_t ld;    // elements per source row (N, or Kp for x_hat)
  int64_t mred;  // M (valid reduction rows)
  int64_t rows;  // valid operand rows (N, or Kp)
  // lane_off: byte offset of the thread's first element in stage 0, or an
  // out-of-range offset for columns past the operand (adding a stage's
  // offset, below 2^31, keeps it out of range)
  struct Regs { uint2 v[16]; uint32_t lane_off; };

  // Byte offset of row e of the thread's 16 in stage s (uniform part).
  __device__ __forceinline__ uint32_t stage_off(int s, int e) const {
    return (uint32_t)(((int64_t)s * kRed16 + e) * ld * 2);
  }
  __device__ __forceinline__ void load(Regs& r, int row0, int s) const {
    const int tid = threadIdx.x;
    const int64_t m = (int64_t)s * kRed16 + 16 * (tid >> 6);
    const int64_t n = row0 + 4 * (tid & 63);
    if constexpr (VEC) {
      const rsrc_t rs = make_rsrc(dy, (uint32_t)(mred * ld * 2));
      r.lane_off = n < rows ? (uint32_t)((16 * (tid >> 6) * ld + n) * 2) : kOob;
#pragma unroll
      for (int e = 0; e < 16; ++e) r.v[e] = buf_load8(rs, r.lane_off + stage_off(s, e));
    } else {
      const uint16_t* p = dy + m * ld + n;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        uint32_t q[4] = {0, 0, 0, 0};
        if (m + e < mred) {
          const uint16_t* src = p + e * ld;
#pragma unroll
          for (int j = 0; j < 4; ++j) q[j] = (n + j < rows) ? src[j] : 0u;
        }
        r.v[e] = make_uint2(q[0] | (q[1] << 16), q[2] | (q[3] << 16));
      }
    }
  }
  __device__ __forceinline__ void store(const Regs& r, char* lds) const {
    const int tid = threadIdx.x;
    const int nq = tid & 63, mg = tid >> 6;
    // element (m = e, n = q) is half (q & 1) of word (q >> 1) of v[e]
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      char* dst = lds + lds_off<kSwz>(4 * nq, 2 * mg + hh);  // rows 4nq..4nq+3 share the swizzle
      const uint2* v = r.v + 8 * hh;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t sel = (q & 1) ? 0x07060302u : 0x05040100u;
        uint4 o;
        o.x = perm((q >> 1) ? v[1].y : v[1].x, (q >> 1) ? v[0].y : v[0].x, sel);
        o.y = perm((q >> 1) ? v[3].y : v[3].x, (q >> 1) ? v[2].y : v[2].x, sel);
        o.z = perm((q >> 1) ? v[5].y : v[5].x, (q >> 1) ? v[4].y : v[4].x, sel);
        o.w = perm((q >> 1) ? v[7].y : v[7].x, (q >> 1) ? v[6].y : v[6].x, sel);
        *reinterpret_cast<uint4*>(dst + q * kPitch) = o;
      }
    }
  }

  // Staging in the slots of k-step KS: half hh = KS/2 (m rows 8hh..8hh+7 of
  // the thread's 16), n columns q = 2(KS&1), +1 (slots W0, W0+1; each uses
  // all 8 rows); odd k-steps then refill that half's 8 rows with stage s+2,
  // one row per slot (slots W0+2 .. W0+9) so that the loads of the two
  // operands do not arrive at the memory pipeline in bursts. W0 = 3 for the
  // P operand and 5 for Q.
  struct Tmp {};
  static constexpr int kLastStoreSlot = W0 + 1;
  __device__ __forceinline__ void write_q(const Regs& r, char* lds, int hh, int q) const {
    const int tid = threadIdx.x;
    const int nq = tid & 63, mg = tid >> 6;
    char* dst = lds + lds_off<kSwz>(4 * nq, 2 * mg + hh);
    const uint2* v = r.v + 8 * hh;
    const uint32_t sel = (q & 1) ? 0x07060302u : 0x05040100u;
    uint4 o;
    o.x = perm((q >> 1) ? v[1].y : v[1].x, (q >> 1) ? v[0].y : v[0].x, sel);
    o.y = perm((q >> 1) ? v[3].y : v[3].x, (q >> 1) ? v[2].y : v[2].x, sel);
    o.z = perm((q >> 1) ? v[5].y : v[5].x, (q >> 1) ? v[4].y : v[4].x, sel);
    o.w = perm((q >> 1) ? v[7].y : v[7].x, (q >> 1) ? v[6].y : v[6].x, sel);
    *reinterpret_cast<uint4*>(dst + q * kPitch) = o;
  }
  template <int KS, int U>
  __device__ __forceinline__ void slot(Regs& r, Tmp&, char* lds, int row0, int s2) const {
    constexpr int hh = KS >> 1;
    if constexpr (U == W0 || U == W0 + 1) write_q(r, lds, hh, 2 * (KS & 1) + (U == W0 + 1));
    if constexpr ((KS & 1) && U >= W0 + 2 && U < W0 + 10) {
      if constexpr (VEC) {
        const rsrc_t rs = make_rsrc(dy, (uint32_t)(mred * ld * 2));
        constexpr int e = 8 * hh + (U - W0 - 2);
        r.v[e] = buf_load8(rs, r.lane_off + stage_off(s2, e));
      } else if constexpr (KS == kKSteps - 1 && U == W0 + 9) {
        load(r, row0, s2);
      }
    }
  }
};

// dW operands kept in their memory orientation. The tile of a stage is 64
// reduction rows m x 256 operand rows (columns of the source), copied as
// stored into LDS rows of kTrPitch bytes, and the fragments are read with
// ds_read_b64_tr_b16, which transposes 4 x 16 blocks of 16-bit values on
// the way out: in each 16-lane group, lane 4e + q addresses LDS row e,
// columns 4q..4q+3, and lane 4q + p receives column 4q + p of rows 0..3.
// A 32 x 16 MFMA fragment is two such reads per lane (reduction rows
// 16KS + 8h + 0..3 and + 4..7 for lane half h). The 64-byte row padding puts
// the 4 rows a 32-lane half reads 16 banks apart, so a read is free of bank
// conflicts, and a staging store (one 512-byte row per half-wave) is too.
constexpr int kTrPitch = 512 + 64;

typedef short v4i16_t __attribute__((ext_vector_type(4)));

template <int PITCH>
struct TrFragsP {
  MfmaBf16::Frag buf[2][4];
  const char* base;
  __device__ __forceinline__ void init(const char* tile, int row0, int lane) {
    const int g = lane >> 4, e = (lane >> 2) & 3, q = lane & 3;
    base = tile + (8 * (g >> 1) + e) * PITCH + 2 * (row0 + 16 * (g & 1) + 4 * q);
  }
  static __device__ __forceinline__ v4i16_t tr(const char* p) {
    typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(__attribute__((address_space(3))) char*)p);
  }
  template <int KS>
  __device__ __forceinline__ void read(int f) {
    const char* a = base + 16 * KS * PITCH + 64 * f;
    const v4i16_t lo = tr(a), hi = tr(a + 4 * PITCH);
    typedef short v8i16_t __attribute__((ext_vector_type(8)));
    const v8i16_t v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    buf[KS & 1][f] = __builtin_bit_cast(MfmaBf16::Frag, v);
  }
  template <int U, bool Q>
  __device__ __forceinline__ void ahead() {
    if constexpr (U == ahead_slot<Q>(0)) read<0>(0);
    if constexpr (U == ahead_slot<Q>(1)) read<0>(1);
    if constexpr (U == ahead_slot<Q>(2)) read<0>(2);
    if constexpr (U == ahead_slot<Q>(3)) read<0>(3);
  }
  template <int KS, int U, bool Q>
  __device__ __forceinline__ void slot() {
    if constexpr (KS + 1 < kKSteps) {
      if constexpr (U == next_read_slot<Q>(0)) read<KS + 1>(0);
      if constexpr (U == next_read_slot<Q>(1)) read<KS + 1>(1);
      if constexpr (U == next_read_slot<Q>(2)) read<KS + 1>(2);
      if constexpr (U == next_read_slot<Q>(3)) read<KS + 1>(3);
    }
  }
  template <int KS>
  __device__ __forceinline__ MfmaBf16::Frag frag(int f) const { return buf[KS & 1][f]; }
};

using TrFrags = TrFragsP<kTrPitch>;

// Copy loader for TrFrags tiles from a bf16 [m][ld] matrix whose first
// `cols` columns are the operand rows (x_hat: ld = cols = Kp; dY: ld = cols
// = N), ld a multiple of 8 so that 16-byte pieces never straddle a row end.
// Thread t handles 16-byte chunk t % 32 of reduction rows t / 32 + 8h,
// h < 8 (a wave instruction covers 2 rows x 512 bytes). Staging in k-step
// KS: rows h = 2KS, 2KS + 1 are stored (slots S0, S0 + 2) and refilled with
// stage s+2 (slots S0 + 8, S0 + 10). S0 = 1 for P and 5 for Q.
template <int S0>
struct RowCopyBf16Loader {
  static constexpr bool kSwz = false;
  static constexpr int kTileB = 64 * kTrPitch;
  static constexpr int kLastStoreSlot = S0 + 2;
  template <class MT, int MAP>
  using Frags = TrFrags;
  const uint16_t* src;
  int64_t ld;    // elements per source row
  int64_t mred;  // valid reduction rows (M)
  int64_t cols;  // valid operand rows (columns of the source)
  // lane_off: byte offset of the thread's chunk in stage 0, row t/32, or an
  // out-of-range offset for chunks past `cols`
  struct Regs { uint4 v[8]; uint32_t lane_off; };
  struct Tmp {};

  __device__ __forceinline__ uint32_t stage_off(int s, int h) const {
    return (uint32_t)(((int64_t)s * kRed16 + 8 * h) * ld * 2);
  }
  __device__ __forceinline__ void load(Regs& r, int row0, int s) const {
    const int tid = threadIdx.x;
    const int64_t col = row0 + 8 * (tid & 31);
    r.lane_off = col < cols ? (uint32_t)(((tid >> 5) * ld + col) * 2) : kOob;
    const rsrc_t rs = make_rsrc(src, (uint32_t)(mred * ld * 2));
#pragma unroll
    for (int h = 0; h < 8; ++h) r.v[h] = buf_load16(rs, r.lane_off + stage_off(s, h));
  }
  __device__ __forceinline__ void store(const Regs& r, char* lds) const {
    const int tid = threadIdx.x;
    char* dst = lds + (tid >> 5) * kTrPitch + 16 * (tid & 31);
#pragma unroll
    for (int h = 0; h < 8; ++h) *reinterpret_cast<uint4*>(dst + 8 * h * kTrPitch) = r.v[h];
  }
  template <int KS, int U>
  __device__ __forceinline__ void slot(Regs& r, Tmp&, char* lds, int, int s2) const {
    const int tid = threadIdx.x;
    if constexpr (U == S0 || U == S0 + 2) {
      constexpr int h = 2 * KS + (U == S0 + 2);
      *reinterpret_cast<uint4*>(lds + ((tid >> 5) + 8 * h) * kTrPitch + 16 * (tid & 31)) = r.v[h];
    }
    if constexpr (U == S0 + 8 || U == S0 + 10) {
      constexpr int h = 2 * KS + (U == S0 + 10);
      const rsrc_t rs = make_rsrc(src, (uint32_t)(mred * ld * 2));
      r.v[h] = buf_load16(rs, r.lane_off + stage_off(s2, h));
    }
  }
};

// dW P: x_hat = bf16(fl32(x_q * fl32(s/127))) is built once per backward
// call into the workspace ([M][Kp] bf16; for the scales act-quant produces
// it equals the exactly rounded bf16(x_q * s / 127)) and then staged like dY
// (RowTransposeBf16Loader). Each element is converted once instead of once
// per output tile column. Thread t converts 16 int8 of row m: each byte is
// biased to [1, 255] so that u*r - 128r = x_q*r exactly before the single
// rounding of the fma.
// 16 int8 of a row with scale factor r = s / 127 -> 16 bf16 (lo: values
// 0..7, hi: 8..15). The one definition of x_hat's arithmetic: the pre-pass
// and the few-token dW kernel, which converts its own slice, both call it.
__device__ __forceinline__ void xhat16(uint4 v, float r, uint4& lo, uint4& hi) {
  const float bias = -128.0f * r;
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t o[8];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t u = w[d] ^ 0x80808080u;
    o[2 * d] = pack_bf16x2(fmaf((float)(u & 0xFFu), r, bias), fmaf((float)((u >> 8) & 0xFFu), r, bias));
    o[2 * d + 1] = pack_bf16x2(fmaf((float)((u >> 16) & 0xFFu), r, bias), fmaf((float)(u >> 24), r, bias));
  }
  lo = make_uint4(o[0], o[1], o[2], o[3]);
  hi = make_uint4(o[4], o[5], o[6], o[7]);
}

__device__ __forceinline__ void xhat_blocks(const int8_t* __restrict__ xq, const float* __restrict__ s, int64_t M,
                                            int64_t Kp, uint16_t* __restrict__ xhat, int b, int nb) {
  const int64_t cpr = Kp / 16;  // 16-byte chunks per row
  const int64_t total = M * cpr;
  for (int64_t c = (int64_t)b * 256 + threadIdx.x; c < total; c += (int64_t)nb * 256) {
    const int64_t m = c / cpr;
    uint4* dst = reinterpret_cast<uint4*>(xhat) + 2 * c;
    xhat16(reinterpret_cast<const uint4*>(xq)[c], s[m] / 127.0f, dst[0], dst[1]);
  }
}

__global__ __launch_bounds__(256) void xhat_kernel(const int8_t* __restrict__ xq, const float* __restrict__ s,
                                                   int64_t M, int64_t Kp, uint16_t* __restrict__ xhat) {
  xhat_blocks(xq, s, M, Kp, xhat, blockIdx.x, gridDim.x);
}

// dX P: the ternary codes transposed to [k][n] as fp4 nibbles (the layout
// CodesFp4Frags reads: n even in the low nibble, +1 = 0x2, -1 = 0xA, 0 =
// 0x0), rows of Np/2 bytes with Np = N rounded up to 64 (zero nibbles past
// N), built once per backward call into the workspace and then copied stage
// by stage like the forward's codes (RowCodesLoader). A block covers 64 k x
// 256 n: thread t loads the 64 codes k0..k0+63 of row n0 + t (16 bytes, 4
// planar words; code j of a word sits at bit 8(j%4) + 2(j/4)), then writes
// the 64 nibbles n0 + 64(t%4) + 0..63 of row k0 + t/4 (32 bytes).
__device__ __forceinline__ void wt_fp4_block(const uint8_t* __restrict__ packed, int64_t N, int64_t Kp, int64_t Np,
                                             uint8_t* __restrict__ wt, int bx, int by) {
  // tile[word][n]: the 4 words of each row, word-major so that the words
  // of 4 consecutive rows are one 16-byte read
  __shared__ __attribute__((aligned(16))) uint32_t tile[4][256 + 4];
  const int t = threadIdx.x;
  const int64_t k0 = (int64_t)bx * 64, n0 = (int64_t)by * 256;
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (n0 + t < N) v = *reinterpret_cast<const uint4*>(packed + (n0 + t) * (Kp / 4) + k0 / 4);
  tile[0][t] = v.x;
  tile[1][t] = v.y;
  tile[2][t] = v.z;
  tile[3][t] = v.w;
  __syncthreads();
  // code j of a word: byte j % 4, bits 2(j / 4)
  const int kl = t >> 2, w = kl >> 4, j = kl & 15;
  const uint32_t byte = j & 3, sh = 2 * (j >> 2);
  const uint32_t gsel = byte | ((byte + 4) << 8);
  const int nb = 64 * (t & 3);
  if (n0 + nb >= Np) return;
  // nibbles of rows n..n+3 (4 words) -> bytes 0 and 2 of the result
  const auto quad = [&](uint4 a) {
    const uint32_t g = perm(perm(a.w, a.z, gsel), perm(a.y, a.x, gsel), 0x05040100u);  // byte e: row n+e
    const uint32_t f = perm(0u, 0x0A000200u, (g >> sh) & 0x03030303u);                 // code 0, 1, 3 -> fp4 0, 2, A
    return f | (f >> 4);
  };
  const uint4* src = reinterpret_cast<const uint4*>(&tile[w][nb]);
  uint32_t o[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) o[q] = perm(quad(src[2 * q + 1]), quad(src[2 * q]), 0x06040200u);
  uint4* dst = reinterpret_cast<uint4*>(wt + (k0 + kl) * (Np / 2) + (n0 + nb) / 2);
  dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
  dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
}

// Transpose blocks in XCD-major order. Blocks are dispatched round-robin
// over the 8 XCDs (block b on XCD b % 8), and the 8 k-blocks that read one
// 128-byte line of a code row are neighbours; numbered as they come, each
// line was fetched once per XCD into 8 private L2s. Here the blocks of one
// XCD take consecutive indices (k fastest), so the line's readers share one
// L2. The first 8 * floor(nb / 8) indices are permuted; the rest keep
// theirs.
__device__ __forceinline__ int xcd_major(int b, int nb) {
  const int per = nb / 8;
  return b < per * 8 ? (b % 8) * per + b / 8 : b;
}

__device__ __forceinline__ void wt_fp4_xcd(const uint8_t* __restrict__ packed, int64_t N, int64_t Kp, int64_t Np,
                                           uint8_t* __restrict__ wt, int b, int wt_bx, int wt_by) {
  const int v = xcd_major(b, wt_bx * wt_by);
  wt_fp4_block(packed, N, Kp, Np, wt, v % wt_bx, v / wt_bx);
}

__global__ __launch_bounds__(256) void wt_fp4_kernel(const uint8_t* __restrict__ packed, int64_t N, int64_t Kp,
                                                     int64_t Np, uint8_t* __restrict__ wt, int wt_bx, int wt_by) {
  wt_fp4_xcd(packed, N, Kp, Np, wt, blockIdx.x, wt_bx, wt_by);
}

// Both backward pre-passes in one launch: the first wt_bx * wt_by blocks
// transpose the codes, the other xhat_nb blocks build x_hat (the two are
// independent, and the transpose is ALU-heavy while x_hat is HBM-heavy).
__global__ __launch_bounds__(256) void bwd_prep_kernel(const uint8_t* __restrict__ packed, int64_t N, int64_t Kp,
                                                       int64_t Np, uint8_t* __restrict__ wt, int wt_bx, int wt_by,
                                                       const int8_t* __restrict__ xq, const float* __restrict__ s,
                                                       int64_t M, uint16_t* __restrict__ xhat, int xhat_nb) {
  const int b = blockIdx.x, nwt = wt_bx * wt_by;
  if (b < nwt)
    wt_fp4_xcd(packed, N, Kp, Np, wt, b, wt_bx, wt_by);
  else
    xhat_blocks(xq, s, M, Kp, xhat, b - nwt, xhat_nb);
}

// ---------------------------------------------------------------------------
// Epilogues: acc (wave tile origin i0, j0) -> memory. Lane l holds, for each
// fragment (fi, fj) and group g, the 4 consecutive i = i0 + 32fi + 8g +
// 4(l/32) + 0..3 at j = j0 + 32fj + l%32.
//
// Stored from the accumulator layout, one instruction would write 16-byte
// pieces of 32 output rows, which runs at about half the HBM write rate of
// whole-row stores. The block goes through LDS instead (EpStage): in four
// passes of 32 rows j (one fragment column fj), each lane puts its 4-value
// pieces into a per-wave LDS buffer of 32 rows, and every store instruction
// then writes whole 128-value row segments (4 rows of bf16 or 2 of 32-bit
// values). LDS rows are padded by 16 bytes: the 16 rows a half-wave puts to
// start 4 banks apart, and a row read by 16 or 32 lanes covers every bank
// once; all LDS offsets are a per-lane base plus a constant. LDS is free
// when the epilogue runs: the last stage's reads and staging stores all
// precede its barrier.
// ---------------------------------------------------------------------------

template <int EB>  // bytes per output element: 2 (bf16) or 4 (f32, int32)
struct EpStage {
  static constexpr int kRowB = 128 * EB;
  static constexpr int kPitch = kRowB + 16;
  static constexpr int kChunks = kRowB / 16;
  static constexpr int kWaveBytes = 32 * kPitch;
  static constexpr int kRowsPerGet = 1024 / kRowB;  // rows per wave instruction
  static constexpr int kGets = 32 / kRowsPerGet;
  // The lane's piece of (fi, g): 4 values of row l%32 at i = 32fi + 8g + 4(l/32).
  template <class V>
  static __device__ __forceinline__ void put(char* w, int lane, int fi, int g, V v) {
    char* base = w + (lane & 31) * kPitch + 4 * EB * (lane >> 5);
    *reinterpret_cast<V*>(base + (32 * fi + 8 * g) * EB) = v;
  }
  // Row-wise read-out of the 32 rows into out[j][i] (rows of I elements):
  // get k is the 16 bytes of row k * kRowsPerGet + lane / kChunks, chunk
  // lane % kChunks, i.e. out[j0 + row][i0 + chunk * 16 / EB ..]. All gets
  // are issued first. When I is a multiple of 16 / EB (a chunk then lies
  // all inside or all outside a row), each get is one 16-byte store through
  // a buffer resource based at the pass's first row (a streaming store: the
  // output is not read again by the launch), with the row offset as the
  // uniform soffset and an out-of-range voffset for rows at or past J
  // and chunks at or past I (32 * I * EB < 2^31, checked by the C ABI);
  // otherwise rows are not 16-byte aligned and the valid elements are
  // stored one by one. i0, j0 are uniform in the wave.
  static __device__ __forceinline__ void drain(const char* w, char* out, int64_t I, int64_t J, int i0, int j0,
                                               int lane) {
    i0 = __builtin_amdgcn_readfirstlane(i0);
    j0 = __builtin_amdgcn_readfirstlane(j0);
    int c = lane % kChunks, rl = lane / kChunks;
    // opaque to the optimizer: keeps the per-get row terms from being
    // computed once per kernel and spilled across the main loop
    asm volatile("" : "+v"(c), "+v"(rl));
    const char* src = w + rl * kPitch + 16 * c;
    uint4 v[kGets];
#pragma unroll
    for (int k = 0; k < kGets; ++k) v[k] = *reinterpret_cast<const uint4*>(src + k * kRowsPerGet * kPitch);
    const int rows_in = J - j0 < 32 ? (int)(J - j0) : 32;
    if ((I & (16 / EB - 1)) == 0) {
      const uint32_t row_b = (uint32_t)I * EB;
      const rsrc_t rs = make_rsrc(out + ((int64_t)j0 * I + i0) * EB, 32u * row_b);
      const uint32_t lane_off = i0 + c * (16 / EB) < I ? rl * row_b + 16 * c : kOob;
#pragma unroll
      for (int k = 0; k < kGets; ++k)
        buf_store16_stream(rs, rl < rows_in - k * kRowsPerGet ? lane_off : kOob,
                           (uint32_t)(k * kRowsPerGet) * row_b, v[k]);
    } else {
      const int64_t i = i0 + c * (16 / EB);
#pragma unroll
      for (int k = 0; k < kGets; ++k) {
        if (k * kRowsPerGet + rl >= rows_in) continue;
        char* row = out + (int64_t)(j0 + k * kRowsPerGet + rl) * I * EB;
        const uint32_t wv[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
        for (int e = 0; e < 16 / EB; ++e) {
          if (i + e >= I) continue;
          if constexpr (EB == 2)
            reinterpret_cast<uint16_t*>(row)[i + e] = (uint16_t)(wv[e >> 1] >> (16 * (e & 1)));
          else
            reinterpret_cast<uint32_t*>(row)[i + e] = wv[e];
        }
      }
    }
  }
};

// The bias values of the output tile being computed (FwdEpilogue<true>),
// staged once per tile before its main loop so that the epilogue reads
// them from LDS: each lane needs 16 groups of 4 per tile and reads each of
// them in all four column passes.
__shared__ __attribute__((aligned(16))) uint16_t s_tile_bias[kBI];

// BIAS: a bf16 bias [N] is added before the rounding (a separate
// instantiation, so that the plain epilogue keeps its registers).
template <bool BIAS>
struct FwdEpilogue {
  uint16_t* y;
  int32_t* acc_out;  // NULL: not written
  const float* s;
  const float* gamma;
  int64_t I, J;          // N, M
  const uint16_t* bias;  // [N] bf16 (BIAS only)

  // The scales this lane's columns need, loaded before the main loop so
  // that their latency is hidden (raw values; combined in store()).
  struct Pre { float g; float sj[kFJ]; };
  __device__ __forceinline__ Pre prefetch(int j0, int lane) const {
    Pre pre;
    pre.g = *gamma;
#pragma unroll
    for (int fj = 0; fj < kFJ; ++fj) {
      const int64_t j = j0 + 32 * fj + (lane & 31);
      pre.sj[fj] = j < J ? s[j] : 0.0f;
    }
    return pre;
  }
  static constexpr int kWaveLds = EpStage<4>::kWaveBytes;  // the int32 pass needs the larger buffer
  static constexpr bool kStagesBias = BIAS;
  // bias[ti0 .. ti0 + kBI) into s_tile_bias (zeros past I); called by every
  // thread of the block, after a barrier that ends the previous tile's
  // epilogue and before the main loop's barriers that order it before this
  // tile's epilogue
  __device__ __forceinline__ void stage_bias(int ti0) const {
    const int t = threadIdx.x;
    if (t < kBI / 8) {
      const int64_t n = (int64_t)ti0 + 8 * t;
      uint4 v;
      if (n + 8 <= I) {
        v = *reinterpret_cast<const uint4*>(bias + n);
      } else {
        uint32_t d[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t lo = n + 2 * e < I ? bias[n + 2 * e] : 0u;
          const uint32_t hi = n + 2 * e + 1 < I ? bias[n + 2 * e + 1] : 0u;
          d[e] = lo | (hi << 16);
        }
        v = make_uint4(d[0], d[1], d[2], d[3]);
      }
      *reinterpret_cast<uint4*>(s_tile_bias + 8 * t) = v;
    }
  }
  __device__ __forceinline__ void store(MfmaI8::Acc (&acc)[kFI][kFJ], const Pre& pre, int i0, int j0,
                                        int lane, char* wlds) const {
    const float g = pre.g;
#pragma unroll
    for (int fj = 0; fj < kFJ; ++fj) {
      const float c = pre.sj[fj] * g / 127.0f;
#pragma unroll
      for (int fi = 0; fi < kFI; ++fi)
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
          float v0 = (float)acc[fi][fj][4 * gi] * c, v1 = (float)acc[fi][fj][4 * gi + 1] * c;
          float v2 = (float)acc[fi][fj][4 * gi + 2] * c, v3 = (float)acc[fi][fj][4 * gi + 3] * c;
          if constexpr (BIAS) {  // n = i0 + 32fi + 8gi + 4h + 0..3 (EpStage::put); tiles start at multiples of kBI
            const uint2 b = *reinterpret_cast<const uint2*>(s_tile_bias + (i0 % kBI) + 32 * fi + 8 * gi +
                                                           4 * (lane >> 5));
            v0 += bf16_lo(b.x); v1 += bf16_hi(b.x); v2 += bf16_lo(b.y); v3 += bf16_hi(b.y);
          }
          EpStage<2>::put(wlds, lane, fi, gi, make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)));
        }
      EpStage<2>::drain(wlds, reinterpret_cast<char*>(y), I, J, i0, j0 + 32 * fj, lane);
      if (acc_out != nullptr) {
#pragma unroll
        for (int fi = 0; fi < kFI; ++fi)
#pragma unroll
          for (int gi = 0; gi < 4; ++gi)
            EpStage<4>::put(wlds, lane, fi, gi,
                            make_uint4((uint32_t)acc[fi][fj][4 * gi], (uint32_t)acc[fi][fj][4 * gi + 1],
                                       (uint32_t)acc[fi][fj][4 * gi + 2], (uint32_t)acc[fi][fj][4 * gi + 3]));
        EpStage<4>::drain(wlds, reinterpret_cast<char*>(acc_out), I, J, i0, j0 + 32 * fj, lane);
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

  struct Pre { float g; };
  static constexpr int kEB = OUT_F32 ? 4 : 2;
  static constexpr int kWaveLds = EpStage<kEB>::kWaveBytes;
  __device__ __forceinline__ Pre prefetch(int, int) const { return Pre{gamma ? *gamma : 1.0f}; }
  __device__ __forceinline__ void store(MfmaBf16::Acc (&acc)[kFI][kFJ], const Pre& pre, int i0, int j0,
                                        int lane, char* wlds) const {
    float sc = 1.0f;
    if (gamma) sc = bf16_to_f32(f32_to_bf16_bits(pre.g));  // bf16(gamma), exact in fp32
#pragma unroll
    for (int fj = 0; fj < kFJ; ++fj) {
#pragma unroll
      for (int fi = 0; fi < kFI; ++fi)
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
          const float v0 = acc[fi][fj][4 * gi] * sc, v1 = acc[fi][fj][4 * gi + 1] * sc;
          const float v2 = acc[fi][fj][4 * gi + 2] * sc, v3 = acc[fi][fj][4 * gi + 3] * sc;
          if constexpr (OUT_F32)
            EpStage<4>::put(wlds, lane, fi, gi, make_uint4(__float_as_uint(v0), __float_as_uint(v1),
                                                           __float_as_uint(v2), __float_as_uint(v3)));
          else
            EpStage<2>::put(wlds, lane, fi, gi, make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)));
        }
      EpStage<kEB>::drain(wlds, static_cast<char*>(out), I, J, i0, j0 + 32 * fj, lane);
    }
  }
};

// dW as 1-bit signs for sign-based optimisers ("1BitTraining.md", closing
// paragraphs: the identity-STE gradient has the sign of the gradient with
// respect to the quantised weight, so a sign optimiser needs only 1 bit per
// weight). out [J][Ip/8] bytes (Ip = Kp): bit b of byte c of row j is set
// iff the fp32 sum for element (j, 8c + b) is negative (zero sums, and the
// zero sums of the padding columns, give 0). Nothing is staged: the lane of
// row j = l % 32 holds, per fragment fi and group g, the sums of
// i = 32fi + 8g + 4h + 0..3 (h = l / 32). Their flags form a nibble, and the
// nibbles of lanes l and l ^ 32 make the bytes of i = 32fi + 8g .. +7; lane
// half h then stores the 8 bytes of i = 64h .. 64h + 63 of the wave tile.
struct Sign1Epilogue {
  uint8_t* out;
  int64_t Ip, J;  // Kp, N

  struct Pre {};
  static constexpr int kWaveLds = 0;
  __device__ __forceinline__ Pre prefetch(int, int) const { return Pre{}; }
  __device__ __forceinline__ void store(MfmaBf16::Acc (&acc)[kFI][kFJ], const Pre&, int i0, int j0, int lane,
                                        char*) const {
    const int h = lane >> 5;
#pragma unroll
    for (int fj = 0; fj < kFJ; ++fj) {
      uint32_t word[kFI];
#pragma unroll
      for (int fi = 0; fi < kFI; ++fi) {
        uint32_t mine = 0;  // flag of i = 32fi + 8g + 4h + e at bit 4g + e
#pragma unroll
        for (int r = 0; r < 16; ++r) mine |= (acc[fi][fj][r] < 0.0f ? 1u : 0u) << r;
        const uint32_t other = (uint32_t)__shfl_xor((int)mine, 32, kWave);
        const uint32_t lo = h ? other : mine, hi = h ? mine : other;
        uint32_t w = 0;
#pragma unroll
        for (int g = 0; g < 4; ++g) w |= (((lo >> (4 * g)) & 0xFu) | (((hi >> (4 * g)) & 0xFu) << 4)) << (8 * g);
        word[fi] = w;
      }
      const int64_t j = j0 + 32 * fj + (lane & 31);
      const int64_t i = i0 + 64 * h;
      if (j < J && i < Ip)
        *reinterpret_cast<uint2*>(out + j * (Ip / 8) + i / 8) =
            h ? make_uint2(word[2], word[3]) : make_uint2(word[0], word[1]);
    }
  }
};

// TTQ dW ("TTQ_VERIFICATION.md": Backward Pass, a straight-through
// estimator, and Bugs Fixed item 5, the gradient of Wp as a masked sum).
// dW = dY^T x is written as Bf16Epilogue writes it (the latent weight gets
// the quantized weight's gradient unchanged). With partials set, each wave
// also adds up its fp32 sums, before any rounding, over the positions whose
// code is +1 and over those whose code is -1, and writes the two totals to
// partials[wave tile] (one float2 per 128 x 128 wave tile, row-major over
// the wave-tile grid; every entry is written once per call, so nothing
// needs clearing). ttq_grads_kernel adds them up in a fixed order.
//
// Lane l holds k = i0 + 32fi + 8g + 4h + e (h = l/32, e < 4) of row
// n = j0 + 32fj + l%32. i0 + 32fi is a multiple of 32, so the codes of those
// 32 k are the two 32-bit words at byte (i0 + 32fi)/4 of row n (8 bytes,
// one load), and code k sits in word g/2 at bit 8e + 2(2(g%2) + h) (code j
// of a word at bit 8(j%4) + 2(j/4), j = k % 16).
template <bool OUT_F32>
struct TtqDwEpilogue {
  Bf16Epilogue<OUT_F32> out;  // dW [J][I], unscaled
  const uint8_t* codes;       // [J][code_pitch]
  uint32_t code_pitch;        // Kp / 4 bytes
  float2* partials;           // NULL: no sums
  int wtiles_i;               // wave tiles along i

  typedef typename Bf16Epilogue<OUT_F32>::Pre Pre;
  static constexpr int kWaveLds = Bf16Epilogue<OUT_F32>::kWaveLds;
  __device__ __forceinline__ Pre prefetch(int j0, int lane) const { return out.prefetch(j0, lane); }
  __device__ __forceinline__ void store(MfmaBf16::Acc (&acc)[kFI][kFJ], const Pre& pre, int i0, int j0, int lane,
                                        char* wlds) const {
    if (partials == nullptr) {
      out.store(acc, pre, i0, j0, lane, wlds);
      return;
    }
    const int h = lane >> 5;
    // rows past J fall outside the resource; words past the row's end get an
    // out-of-range offset (zeros: no code)
    const rsrc_t rs = make_rsrc(codes, (uint32_t)out.J * code_pitch);
    uint2 c[kFI][kFJ];
#pragma unroll
    for (int fj = 0; fj < kFJ; ++fj) {
      const uint32_t n = (uint32_t)(j0 + 32 * fj + (lane & 31));
#pragma unroll
      for (int fi = 0; fi < kFI; ++fi) {
        const uint32_t col = (uint32_t)(i0 + 32 * fi) / 4;
        c[fi][fj] = buf_load8(rs, col < code_pitch ? n * code_pitch + col : kOob);
      }
    }
    out.store(acc, pre, i0, j0, lane, wlds);
    float sp = 0.0f, sn = 0.0f;
#pragma unroll
    for (int fi = 0; fi < kFI; ++fi)
#pragma unroll
      for (int fj = 0; fj < kFJ; ++fj)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const uint32_t w = (g < 2 ? c[fi][fj].x : c[fi][fj].y) >> (4 * (g & 1) + 2 * h);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t code = (w >> (8 * e)) & 3u;
            const float v = acc[fi][fj][4 * g + e];
            sp += code == 1u ? v : 0.0f;
            sn += code == 3u ? v : 0.0f;
          }
        }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      sp += __shfl_xor(sp, off, kWave);
      sn += __shfl_xor(sn, off, kWave);
    }
    if (lane == 0) partials[(j0 / kWTJ) * wtiles_i + i0 / kWTI] = make_float2(sp, sn);
  }
};

// The two scale gradients from the wave-tile partials: grads[0] = sum of the
// +1 sums (dL/dWp), grads[1] = -(sum of the -1 sums) (dL/dWn: the weight
// there is -Wn). Thread t adds partials t, t + 256, ... in fp64, then the
// block adds the thread sums in a fixed order; rounded once to fp32.
__global__ __launch_bounds__(256) void ttq_grads_kernel(const float2* __restrict__ partials, int count,
                                                        float* __restrict__ grads) {
  double p = 0.0, n = 0.0;
  for (int i = threadIdx.x; i < count; i += 256) {
    const float2 v = partials[i];
    p += (double)v.x;
    n += (double)v.y;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    p += __shfl_xor(p, off, kWave);
    n += __shfl_xor(n, off, kWave);
  }
  __shared__ double sp[4], sn[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    sp[wave] = p;
    sn[wave] = n;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    grads[0] = (float)((sp[0] + sp[1]) + (sp[2] + sp[3]));
    grads[1] = (float)(-((sn[0] + sn[1]) + (sn[2] + sn[3])));
  }
}

// dW for few tokens (M <= 64, N % 8 == 0): dW[n][k] = sum_{m < M} dY[m][n] *
// x_hat[m][k] ("bitnet-qat-train", Semantics). The reduction is at most 4
// MFMA steps of 16 tokens, so the cost is writing dW: small output tiles
// (64 n x 256 k per workgroup) keep every CU busy with several tiles whose
// loads and stores overlap. The tile's slice of x_hat is converted from
// x_q and s on the way into LDS (xhat16, the pre-pass's arithmetic), so no
// pre-pass runs and the tiles can share a launch with the code transpose
// that the few-token dX needs. Both operands are staged as stored, rows m
// in LDS (rows m >= M as zeros), and read transposed with
// ds_read_b64_tr_b16 (TrFrags): A = x_hat columns k (wave k half 128wk +
// 32f, f < 4), B = dY columns n (wave n half 32wn). D[k][n] goes back
// through LDS as rows n and is written as 16-byte row pieces (element by
// element when K does not keep them aligned). Products are exact in fp32
// and each sum runs in token order. Tile b of ktiles x ceil(N / 64), 256
// threads.
template <bool OUT_F32>
__device__ __forceinline__ void dw_skinny_tile(const int8_t* __restrict__ xq, const float* __restrict__ sx,
                                               const uint16_t* __restrict__ dY, int M, int64_t N, int64_t Kp,
                                               int64_t K, int ktiles, void* __restrict__ dW, int b) {
  constexpr int kEB = OUT_F32 ? 4 : 2;
  constexpr int kOutPitch = 256 * kEB + 16;
  constexpr int kYPitch = 64 * 2 + 16;     // dY rows: 64 n, padded
  constexpr int kXB = 64 * kTrPitch;       // 64 token rows of x_hat
  constexpr int kInB = kXB + 64 * kYPitch;
  constexpr int kOutB = 64 * kOutPitch;
  __shared__ __attribute__((aligned(16))) char smem[kInB > kOutB ? kInB : kOutB];
  char* xs = smem;        // x_hat [m][256 k]
  char* ys = smem + kXB;  // dY [m][64 n]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t k0 = (int64_t)(b % ktiles) * 256, n0 = (int64_t)(b / ktiles) * 64;
  const int ms = (M + 15) / 16;  // MFMA steps of 16 tokens

  const rsrc_t rxq = make_rsrc(xq, (uint32_t)(M * Kp));
  const rsrc_t rdy = make_rsrc(dY, (uint32_t)(M * N * 2));
  uint4 vq[4], vy[2];
  float rq[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {  // x_q: rows m < 64, 16 pieces of 16 bytes per row
    const int e = tid + 256 * i, m = e >> 4;
    const int64_t k = k0 + 16 * (e & 15);
    vq[i] = buf_load16(rxq, m < M && k < Kp ? (uint32_t)(m * Kp + k) : kOob);
    rq[i] = m < M ? sx[m] / 127.0f : 0.0f;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {  // dY: rows m < 64, 8 pieces per row
    const int e = tid + 256 * i, m = e >> 3;
    const int64_t n = n0 + 8 * (e & 7);
    vy[i] = buf_load16(rdy, m < M && n < N ? (uint32_t)((m * N + n) * 2) : kOob);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {  // zeros past M (and past Kp) convert to 0
    const int e = tid + 256 * i;
    if ((e >> 4) < 16 * ms) {
      uint4 lo, hi;
      xhat16(vq[i], rq[i], lo, hi);
      char* dst = xs + (e >> 4) * kTrPitch + 32 * (e & 15);
      *reinterpret_cast<uint4*>(dst) = lo;
      *reinterpret_cast<uint4*>(dst + 16) = hi;
    }
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int e = tid + 256 * i;
    if ((e >> 3) < 16 * ms) *reinterpret_cast<uint4*>(ys + (e >> 3) * kYPitch + 16 * (e & 7)) = vy[i];
  }
  __syncthreads();

  const int wn = wave & 1, wk = wave >> 1;
  TrFrags fa;
  TrFragsP<kYPitch> fb;
  fa.init(xs, 128 * wk, lane);
  fb.init(ys, 32 * wn, lane);
  MfmaBf16::Acc acc[4];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[f][e] = 0.0f;
  const auto step = [&](auto ks) {
    constexpr int KS = decltype(ks)::value;
    fb.template read<KS>(0);
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      fa.template read<KS>(f);
      acc[f] = MfmaBf16::mma(fa.template frag<KS>(f), fb.template frag<KS>(0), acc[f]);
    }
  };
  step(std::integral_constant<int, 0>());
  if (ms > 1) step(std::integral_constant<int, 1>());
  if (ms > 2) step(std::integral_constant<int, 2>());
  if (ms > 3) step(std::integral_constant<int, 3>());
  __syncthreads();

  // D[k][n]: lane column n = 32wn + l % 32, rows k = 128wk + 32f + 8g + 4h + 0..3
  const int nl = 32 * wn + (lane & 31), h = lane >> 5;
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      char* dst = smem + nl * kOutPitch + (128 * wk + 32 * f + 8 * g + 4 * h) * kEB;
      const float v0 = acc[f][4 * g], v1 = acc[f][4 * g + 1], v2 = acc[f][4 * g + 2], v3 = acc[f][4 * g + 3];
      if constexpr (OUT_F32)
        *reinterpret_cast<uint4*>(dst) = make_uint4(__float_as_uint(v0), __float_as_uint(v1), __float_as_uint(v2),
                                                    __float_as_uint(v3));
      else
        *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
    }
  __syncthreads();
  constexpr int kPieces = 256 * kEB / 16;  // 16-byte pieces per output row of the tile
  constexpr int kPer = 16 / kEB;           // elements per piece
  char* out = static_cast<char*>(dW);
#pragma unroll
  for (int i = 0; i < 64 * kPieces / 256; ++i) {
    const int e = tid + 256 * i, r = e / kPieces, c = e % kPieces;
    const int64_t n = n0 + r, k = k0 + kPer * c;
    if (n >= N || k >= K) continue;
    const char* src = smem + r * kOutPitch + 16 * c;
    if (K % kPer == 0) {
      *reinterpret_cast<uint4*>(out + (n * K + k) * kEB) = *reinterpret_cast<const uint4*>(src);
    } else {
      for (int j = 0; j < kPer && k + j < K; ++j) {
        if constexpr (OUT_F32)
          reinterpret_cast<uint32_t*>(out)[n * K + k + j] = reinterpret_cast<const uint32_t*>(src)[j];
        else
          reinterpret_cast<uint16_t*>(out)[n * K + k + j] = reinterpret_cast<const uint16_t*>(src)[j];
      }
    }
  }
}

template <bool OUT_F32>
__global__ __launch_bounds__(256) void dw_skinny_kernel(const int8_t* __restrict__ xq, const float* __restrict__ sx,
                                                        const uint16_t* __restrict__ dY, int M, int64_t N,
                                                        int64_t Kp, int64_t K, int ktiles, void* __restrict__ dW) {
  dw_skinny_tile<OUT_F32>(xq, sx, dY, M, N, Kp, K, ktiles, dW, blockIdx.x);
}

// Few tokens with both outputs, first launch: the first wt_bx * wt_by blocks
// transpose the codes to fp4 for the few-token dX (which runs next), the
// others compute dW tiles (independent of the transpose: ALU- and
// latency-bound work next to the HBM writes of dW).
template <bool OUT_F32>
__global__ __launch_bounds__(256) void bwd_skinny_front_kernel(const uint8_t* __restrict__ packed, int64_t Np,
                                                               uint8_t* __restrict__ wt, int wt_bx, int wt_by,
                                                               const int8_t* __restrict__ xq,
                                                               const float* __restrict__ sx,
                                                               const uint16_t* __restrict__ dY, int M, int64_t N,
                                                               int64_t Kp, int64_t K, int ktiles,
                                                               void* __restrict__ dW) {
  const int b = blockIdx.x, nwt = wt_bx * wt_by;
  if (b < nwt)
    wt_fp4_xcd(packed, N, Kp, Np, wt, b, wt_bx, wt_by);
  else
    dw_skinny_tile<OUT_F32>(xq, sx, dY, M, N, Kp, K, ktiles, dW, b - nwt);
}

// ---------------------------------------------------------------------------
// Work split. The T output tiles of a product, each of S reduction stages,
// are T*S iterations in tile-major order (tile t = (ti, tj) with ti fastest).
// A grid of G workgroups shares them out: virtual workgroup v takes
// iterations [lo(v), lo(v+1)), lo(v) = floor(v * T * S / G). With G = T each
// workgroup gets one whole tile. With G below T (or not dividing it) a tile
// can be split between consecutive workgroups (stream-K): each piece
// accumulates its stages, and the last piece to arrive adds the partial
// tiles of the others in piece order, so the sum does not depend on the
// arrival order, and runs the epilogue.
//
// Workgroups are dispatched round-robin over the 8 XCDs (block b on XCD
// b % 8); virtual indices are numbered XCD by XCD, so an XCD owns a
// contiguous range of iterations and its blocks share operand panels in its
// L2 (and the pieces of a split tile are usually on one XCD).
// ---------------------------------------------------------------------------

struct SplitPlan {
  int64_t total;       // T * S
  int grid;            // G
  int tiles_i;
  int nstages;         // S
  uint32_t spin_limit; // polls before a wait for published partials gives up
  uint64_t gen;        // tag of this launch in the counters (0 < gen < 2^48)
  int nslots;          // partial-tile slots: min(2G, G + T - 1)
  uint64_t* counters;  // [T][2] tagged counters (pieces arrived, partials
                       // published); NULL when no tile is split
  uint4* partials;     // [nslots][64][kThreads] 16-byte chunks of partial tiles
};

__host__ __device__ __forceinline__ int cta_order(int b, int G) {
  const int q = G / 8, r = G % 8;
  const int x = b % 8, k = b / 8;
  return (x < r) ? x * (q + 1) + k : r * (q + 1) + (x - r) * q + k;
}

__host__ __device__ __forceinline__ int64_t split_lo(const SplitPlan& p, int v) {
  return (int64_t)v * p.total / p.grid;
}

// The virtual workgroup whose range holds iteration it.
__host__ __device__ __forceinline__ int split_owner(const SplitPlan& p, int64_t it) {
  return (int)(((it + 1) * p.grid - 1) / p.total);
}

// Partial-tile slot of workgroup v's piece of tile t. Two numberings, each
// giving every piece its own slot; the plan takes the one with fewer slots:
//  - 2v for the tile v's range starts in, 2v + 1 for the tile it ends in
//    (a range holds at most two split pieces: any tile strictly inside it
//    is whole), 2G slots;
//  - v + t: along the iteration order the next piece has the next
//    workgroup, the next tile, or both, so v + t strictly increases,
//    G + T - 1 slots (fewer when G > T).
__host__ __device__ __forceinline__ int partial_slots(int64_t tiles, int grid) {
  const int64_t a = 2 * (int64_t)grid, b = (int64_t)grid + tiles - 1;
  return (int)(a < b ? a : b);
}
__host__ __device__ __forceinline__ int64_t piece_slot(const SplitPlan& p, int v, int t) {
  if (p.nslots < 2 * p.grid) return (int64_t)v + t;
  return 2 * (int64_t)v + ((int64_t)t == split_lo(p, v) / p.nstages ? 0 : 1);
}

// The piece that starts at iteration it of a range ending at hi: tile t,
// stages [s0, s1).
__host__ __device__ __forceinline__ void split_piece(const SplitPlan& p, int64_t it, int64_t hi, int* t, int* s0,
                                                     int* s1) {
  *t = (int)(it / p.nstages);
  *s0 = (int)(it - (int64_t)*t * p.nstages);
  *s1 = (int)((int64_t)p.nstages < *s0 + (hi - it) ? (int64_t)p.nstages : *s0 + (hi - it));
}

// The workgroups that hold pieces of tile t: va .. va + n - 1, in stage order.
__host__ __device__ __forceinline__ void split_tile_owners(const SplitPlan& p, int t, int* va, int* n) {
  const int64_t S = p.nstages;
  *va = split_owner(p, (int64_t)t * S);
  *n = split_owner(p, (int64_t)t * S + S - 1) - *va + 1;
}

// Waits for published partials that ran out of polls (a piece that never
// published: it cannot happen while every workgroup makes progress). The
// tile is then written as NaN (int32 accumulators: INT32_MIN) instead of a
// sum of unpublished data, and this counter is raised; the host reads and
// clears it with bitnet_split_timeouts().
__device__ unsigned int g_split_timeouts;

// Tagged counters: a 64-bit word gen << 16 | count. A word written by
// another launch (another tag) counts as zero, so the counters never need
// clearing before a launch; the last piece of a tile clears its two words
// once they are no longer used, so that a launch repeated with the same tag
// (a captured graph replayed) also starts from zero. The counters only
// order the exchange of partial tiles, whose stores and loads are
// device-coherent and complete (wait_vmem) before the counter moves, so
// relaxed device-scope atomics suffice and no cache-wide fence is needed.
constexpr uint64_t kCountMask = 0xFFFF;

__device__ __forceinline__ uint32_t tagged_arrive(uint64_t* c, uint64_t gen) {
  uint64_t old = __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (;;) {
    const bool same = (old >> 16) == gen;
    const uint64_t nw = same ? old + 1 : ((gen << 16) | 1u);
    if (__hip_atomic_compare_exchange_strong(c, &old, nw, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT))
      return same ? (uint32_t)(old & kCountMask) : 0u;
  }
}

__device__ __forceinline__ uint32_t tagged_count(const uint64_t* c, uint64_t gen) {
  const uint64_t v = __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return (v >> 16) == gen ? (uint32_t)(v & kCountMask) : 0u;
}

// Wait until `want` partials of a tile are published. Only pieces that have
// already arrived (so are running and only have their stores left) are
// waited for, so the wait ends; the bound (about a second at the default
// limit) is a safety net. Returns false when it gave up.
__device__ __forceinline__ bool wait_published(const uint64_t* c, uint64_t gen, uint32_t want, uint32_t limit) {
  for (uint32_t i = 0; i < limit; ++i) {
    if (tagged_count(c, gen) >= want) return true;
    __builtin_amdgcn_s_sleep(2);
  }
  return tagged_count(c, gen) >= want;
}

template <class Acc>
__device__ __forceinline__ void zero_acc(Acc& a) {
#pragma unroll
  for (int e = 0; e < 16; ++e) a[e] = 0;
}

// All of ahead<U>() of a reader at once (the first stage of a run).
template <bool Q, class F>
__device__ __forceinline__ void prime(F& f) {
  f.template ahead<kBarrierSlot + 1, Q>(); f.template ahead<kBarrierSlot + 2, Q>();
  f.template ahead<kBarrierSlot + 3, Q>(); f.template ahead<kBarrierSlot + 4, Q>();
  f.template ahead<kBarrierSlot + 5, Q>(); f.template ahead<kBarrierSlot + 6, Q>();
  f.template ahead<kBarrierSlot + 7, Q>();
}

// One MFMA slot of a k-step: MFMA (U / 4, U % 4), then each reader's and
// loader's share of the work for U (issued behind the MFMA so that it
// overlaps its 32 cycles), fenced from the next slot so that the compiler
// keeps this interleave. fpn/fqn read the other LDS buffer (the next
// stage); `more` says whether there is a next stage.
template <int KS, int U, class MT, class PL, class QL, class FP, class FQ>
__device__ __forceinline__ void gemm_slot(const PL& pl, const QL& ql, typename PL::Regs& pr,
                                          typename QL::Regs& qr, typename PL::Tmp& pt,
                                          typename QL::Tmp& qt, FP& fp, FQ& fq, FP& fpn, FQ& fqn,
                                          char* Pn, char* Qn, typename MT::Acc (&acc)[kFI][kFJ],
                                          int i0, int j0, int s2, bool more) {
  acc[U / 4][U % 4] = MT::mma(fp.template frag<KS>(U / 4), fq.template frag<KS>(U % 4), acc[U / 4][U % 4]);
  fp.template slot<KS, U, false>();
  fq.template slot<KS, U, true>();
  pl.template slot<KS, U>(pr, pt, Pn, i0, s2);
  ql.template slot<KS, U>(qr, qt, Qn, j0, s2);
  if constexpr (KS == kKSteps - 1) {
    if constexpr (U == kBarrierSlot) __syncthreads();
    if constexpr (U > kBarrierSlot) {
      if (more) {
        fpn.template ahead<U, false>();
        fqn.template ahead<U, true>();
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (U + 1 < kFI * kFJ)
    gemm_slot<KS, U + 1, MT>(pl, ql, pr, qr, pt, qt, fp, fq, fpn, fqn, Pn, Qn, acc, i0, j0, s2, more);
}

// LDS: two stages, each a P tile followed by a Q tile.
template <class PL, class QL>
struct SmemLayout {
  static constexpr int kStage = PL::kTileB + QL::kTileB;
  static constexpr int kBytes = 2 * kStage;
};

// One pipeline stage: MFMAs on LDS buffer CUR (readers fp, fq) for
// reduction stage s, while staging stage s+1 from registers into buffer
// CUR^1 and fetching stage s+2 into those registers, one quarter per
// k-step, and, when `more`, preparing k-step 0 of stage s+1 (readers fpn,
// fqn of buffer CUR^1). Past the last stage the staging runs on zeros and
// is never read.
template <int CUR, class MT, class PL, class QL, class FP, class FQ>
__device__ __forceinline__ void gemm_stage(const PL& pl, const QL& ql, typename PL::Regs& pr,
                                           typename QL::Regs& qr, char* smem, FP& fp, FQ& fq,
                                           FP& fpn, FQ& fqn, typename MT::Acc (&acc)[kFI][kFJ],
                                           int i0, int j0, int s, bool more) {
  typedef SmemLayout<PL, QL> L;
  char* Pn = smem + (CUR ^ 1) * L::kStage;
  char* Qn = Pn + PL::kTileB;
  typename PL::Tmp pt;
  typename QL::Tmp qt;
  gemm_slot<0, 0, MT>(pl, ql, pr, qr, pt, qt, fp, fq, fpn, fqn, Pn, Qn, acc, i0, j0, s + 2, more);
  gemm_slot<1, 0, MT>(pl, ql, pr, qr, pt, qt, fp, fq, fpn, fqn, Pn, Qn, acc, i0, j0, s + 2, more);
  gemm_slot<2, 0, MT>(pl, ql, pr, qr, pt, qt, fp, fq, fpn, fqn, Pn, Qn, acc, i0, j0, s + 2, more);
  gemm_slot<3, 0, MT>(pl, ql, pr, qr, pt, qt, fp, fq, fpn, fqn, Pn, Qn, acc, i0, j0, s + 2, more);
}

// The stages [s0, s1) of tile (i0, j0), accumulated into acc. LDS is free
// on entry and on return. `arrive`, when not NULL, is the published-partials
// counter of this workgroup's previous piece, whose partial stores were
// issued but not waited for: it is incremented (tag gen) once every wave
// has waited for its first stage's loads, which were issued after those
// stores, so the stores are complete by then.
template <class MT, int MAP, class PL, class QL>
__device__ __forceinline__ void run_stages(const PL& pl, const QL& ql, char* smem,
                                           typename MT::Acc (&acc)[kFI][kFJ], int i0, int j0, int s0,
                                           int s1, int prow0, int qrow0, int lane, uint64_t* arrive,
                                           uint64_t gen) {
  static_assert(PL::kLastStoreSlot < kBarrierSlot && QL::kLastStoreSlot < kBarrierSlot,
                "staging stores must precede the end-of-stage barrier");
  typedef SmemLayout<PL, QL> L;
  typename PL::Regs pr;
  typename QL::Regs qr;
  pl.load(pr, i0, s0);
  ql.load(qr, j0, s0);
  __syncthreads();
  pl.store(pr, smem);
  ql.store(qr, smem + PL::kTileB);
  pl.load(pr, i0, s0 + 1);
  ql.load(qr, j0, s0 + 1);
  __syncthreads();
  if (arrive != nullptr && threadIdx.x == 0) tagged_arrive(arrive, gen);
  typename PL::template Frags<MT, MAP> fp0, fp1;
  typename QL::template Frags<MT, MAP> fq0, fq1;
  fp0.init(smem, prow0, lane);
  fq0.init(smem + PL::kTileB, qrow0, lane);
  fp1.init(smem + L::kStage, prow0, lane);
  fq1.init(smem + L::kStage + PL::kTileB, qrow0, lane);
  prime<false>(fp0);
  prime<true>(fq0);
  __builtin_amdgcn_sched_barrier(0);
  int s = s0;
  for (; s + 1 < s1; s += 2) {
    gemm_stage<0, MT>(pl, ql, pr, qr, smem, fp0, fq0, fp1, fq1, acc, i0, j0, s, true);
    gemm_stage<1, MT>(pl, ql, pr, qr, smem, fp1, fq1, fp0, fq0, acc, i0, j0, s + 1, s + 2 < s1);
  }
  if (s < s1) gemm_stage<0, MT>(pl, ql, pr, qr, smem, fp0, fq0, fp1, fq1, acc, i0, j0, s, false);
}

// Element e (0..3) of 16-byte chunk c (0..63) of a thread's accumulators:
// chunk c = 4 * (kFJ * fi + fj) + q holds acc[fi][fj][4q .. 4q + 3].
template <class MT>
__device__ __forceinline__ uint4 acc_chunk(const typename MT::Acc (&acc)[kFI][kFJ], int c) {
  const int fi = c / (4 * kFJ), fj = (c / 4) % kFJ, q = c % 4;
  return make_uint4(MT::to_bits(acc[fi][fj][4 * q]), MT::to_bits(acc[fi][fj][4 * q + 1]),
                    MT::to_bits(acc[fi][fj][4 * q + 2]), MT::to_bits(acc[fi][fj][4 * q + 3]));
}

template <class MT>
__device__ __forceinline__ void acc_chunk_add(typename MT::Acc (&acc)[kFI][kFJ], int c, uint4 v) {
  const int fi = c / (4 * kFJ), fj = (c / 4) % kFJ, q = c % 4;
  acc[fi][fj][4 * q] += MT::from_bits(v.x);
  acc[fi][fj][4 * q + 1] += MT::from_bits(v.y);
  acc[fi][fj][4 * q + 2] += MT::from_bits(v.z);
  acc[fi][fj][4 * q + 3] += MT::from_bits(v.w);
}

__device__ __forceinline__ uint4 chunk_add_f32(uint4 a, uint4 b) {
  return make_uint4(__float_as_uint(__uint_as_float(a.x) + __uint_as_float(b.x)),
                    __float_as_uint(__uint_as_float(a.y) + __uint_as_float(b.y)),
                    __float_as_uint(__uint_as_float(a.z) + __uint_as_float(b.z)),
                    __float_as_uint(__uint_as_float(a.w) + __uint_as_float(b.w)));
}

template <class MT>
__device__ __forceinline__ uint4 chunk_add(uint4 a, uint4 b) {
  if constexpr (std::is_same<typename MT::Elem, float>::value) {
    return chunk_add_f32(a, b);
  } else {
    return make_uint4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
  }
}

// End of a piece of a split tile. Arrive; a piece that is not the last
// issues the stores of its partial tile and returns false (the caller
// signals them published once they are complete); the last one waits for
// the others' partials, adds them in piece order into acc and returns true
// (the caller then runs the epilogue). With pieces p_0..p_{n-1} and this one at
// position me, the sum is ((p_0 + ... + p_{me-1}) + own) + p_{me+1} + ...
// evaluated left to right (own + L == L + own exactly).
template <class MT>
__device__ __forceinline__ bool finish_piece(const SplitPlan& p, typename MT::Acc (&acc)[kFI][kFJ],
                                             int v, int t, int* s_flag) {
  const int tid = threadIdx.x;
  int va, n;
  split_tile_owners(p, t, &va, &n);
  const int me = v - va;
  uint64_t* cnt = p.counters + 2 * (int64_t)t;
  if (tid == 0) *s_flag = (int)tagged_arrive(cnt, p.gen);
  __syncthreads();
  const bool last = (*s_flag == n - 1);
  __syncthreads();
  const rsrc_t pr = make_rsrc(p.partials, (uint32_t)((int64_t)p.nslots * 64 * kThreads * 16));
  if (!last) {
    const uint32_t base = (uint32_t)(piece_slot(p, v, t) * 64 * kThreads + tid) * 16;
#pragma unroll
    for (int c = 0; c < 64; ++c) buf_store16_coherent(pr, base + c * kThreads * 16, acc_chunk<MT>(acc, c));
    asm volatile("" ::: "memory");  // keep the stores ahead of the next piece's loads
    return false;
  }
  if (tid == 0) {
    const bool ok = wait_published(cnt + 1, p.gen, (uint32_t)(n - 1), p.spin_limit);
    *s_flag = ok ? 1 : 0;
    if (!ok) atomicAdd(&g_split_timeouts, 1u);
    // Every piece has arrived and published: nothing else touches this
    // tile's counters in this launch. Clearing them lets a later launch
    // with the same tag (a replay of a captured graph) count from zero.
    __hip_atomic_store(cnt, uint64_t(0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(cnt + 1, uint64_t(0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (*s_flag == 0) {  // gave up: write the tile as a visible sentinel
#pragma unroll
    for (int fi = 0; fi < kFI; ++fi)
#pragma unroll
      for (int fj = 0; fj < kFJ; ++fj)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[fi][fj][e] = MT::from_bits(MT::kPoisonBits);
    return true;
  }
  constexpr int kBatch = 16;
#pragma unroll
  for (int c0 = 0; c0 < 64; c0 += kBatch) {
    if (me > 0) {
      uint4 L[kBatch];
      const uint32_t b0 = (uint32_t)(piece_slot(p, va, t) * 64 * kThreads + tid) * 16;
#pragma unroll
      for (int c = 0; c < kBatch; ++c) L[c] = buf_load16_coherent(pr, b0 + (c0 + c) * kThreads * 16);
      for (int j = 1; j < me; ++j) {
        const uint32_t bj = (uint32_t)(piece_slot(p, va + j, t) * 64 * kThreads + tid) * 16;
#pragma unroll
        for (int c = 0; c < kBatch; ++c)
          L[c] = chunk_add<MT>(L[c], buf_load16_coherent(pr, bj + (c0 + c) * kThreads * 16));
      }
#pragma unroll
      for (int c = 0; c < kBatch; ++c) acc_chunk_add<MT>(acc, c0 + c, L[c]);
    }
    for (int j = me + 1; j < n; ++j) {
      const uint32_t bj = (uint32_t)(piece_slot(p, va + j, t) * 64 * kThreads + tid) * 16;
      uint4 R[kBatch];
#pragma unroll
      for (int c = 0; c < kBatch; ++c) R[c] = buf_load16_coherent(pr, bj + (c0 + c) * kThreads * 16);
#pragma unroll
      for (int c = 0; c < kBatch; ++c) acc_chunk_add<MT>(acc, c0 + c, R[c]);
    }
  }
  return true;
}

// Whether an epilogue stages per-tile data into LDS before the main loop.
template <class EP, class = void>
struct StagesBias : std::false_type {};
template <class EP>
struct StagesBias<EP, std::void_t<decltype(EP::kStagesBias)>> : std::integral_constant<bool, EP::kStagesBias> {};

// The work of virtual workgroup v of a product: one whole tile (no split),
// or its range of (tile, stage) iterations (stream-K).
template <class MT, int MAP, class PL, class QL, class EP>
__device__ __forceinline__ void gemm_body(const PL& pl, const QL& ql, const EP& ep, const SplitPlan& plan,
                                          int v, char* smem, int* s_flag_p) {
  typedef SmemLayout<PL, QL> L;
  static_assert(kThreads / 64 * EP::kWaveLds <= L::kBytes, "epilogue staging fits in the stage buffers");
  int& s_flag = *s_flag_p;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wi = wave % kWavesI, wj = wave / kWavesI;
  const int prow0 = wi * kWTI, qrow0 = wj * kWTJ;
  if (plan.counters == nullptr) {
    // whole tiles: v, v + G, v + 2G, ... (one each when G = T)
    const int T = (int)(plan.total / plan.nstages);
    for (int t = v; t < T; t += plan.grid) {
      const int i0 = (t % plan.tiles_i) * kBI, j0 = (t / plan.tiles_i) * kBJ;
      typename MT::Acc acc[kFI][kFJ];
#pragma unroll
      for (int fi = 0; fi < kFI; ++fi)
#pragma unroll
        for (int fj = 0; fj < kFJ; ++fj) zero_acc(acc[fi][fj]);
      const typename EP::Pre pre = ep.prefetch(j0 + qrow0, lane);
      if constexpr (StagesBias<EP>::value) {
        __syncthreads();
        ep.stage_bias(i0);
      }
      run_stages<MT, MAP>(pl, ql, smem, acc, i0, j0, 0, plan.nstages, prow0, qrow0, lane, nullptr, 0);
      ep.store(acc, pre, i0 + prow0, j0 + qrow0, lane, smem + wave * EP::kWaveLds);
    }
    return;
  }

  const int64_t hi = split_lo(plan, v + 1);
  uint64_t* pending = nullptr;  // published-partials counter to signal
  for (int64_t it = split_lo(plan, v); it < hi;) {
    int t, s0, s1;
    split_piece(plan, it, hi, &t, &s0, &s1);
    const int i0 = (t % plan.tiles_i) * kBI, j0 = (t / plan.tiles_i) * kBJ;

    typename MT::Acc acc[kFI][kFJ];
#pragma unroll
    for (int fi = 0; fi < kFI; ++fi)
#pragma unroll
      for (int fj = 0; fj < kFJ; ++fj) zero_acc(acc[fi][fj]);

    const typename EP::Pre pre = ep.prefetch(j0 + qrow0, lane);
    if constexpr (StagesBias<EP>::value) {
      __syncthreads();
      ep.stage_bias(i0);
    }
    run_stages<MT, MAP>(pl, ql, smem, acc, i0, j0, s0, s1, prow0, qrow0, lane, pending, plan.gen);
    pending = nullptr;
    if ((s0 == 0 && s1 == plan.nstages) || finish_piece<MT>(plan, acc, v, t, &s_flag))
      ep.store(acc, pre, i0 + prow0, j0 + qrow0, lane, smem + wave * EP::kWaveLds);
    else
      pending = plan.counters + 2 * (int64_t)t + 1;
    it += s1 - s0;
  }
  if (pending != nullptr) {
    // the last piece published: wait for its stores, then signal
    wait_vmem();
    __syncthreads();
    if (tid == 0) tagged_arrive(pending, plan.gen);
  }
}

template <class MT, int MAP, class PL, class QL, class EP>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(PL pl, QL ql, EP ep, SplitPlan plan) {
  typedef SmemLayout<PL, QL> L;
  __shared__ __attribute__((aligned(16))) char smem[L::kBytes];
  __shared__ int s_flag;
  gemm_body<MT, MAP>(pl, ql, ep, plan, cta_order(blockIdx.x, plan.grid), smem, &s_flag);
}

// Two independent products in one launch, each on its own share of every
// XCD: of the 8 * kt workgroups (one per CU, workgroup b on XCD b % 8),
// those with b / 8 < k1 run product 1, the others product 2, each
// stream-K over the first plan.grid (at most 8 * k1, resp. 8 * (kt - k1))
// of its workgroups, numbered XCD-contiguously; the rest of a share has no
// work. Used for the two STE backward products, which otherwise would each
// pay their split tail and launch on their own.
template <class MT, int MAP1, class PL1, class QL1, class EP1, int MAP2, class PL2, class QL2, class EP2>
__global__ __launch_bounds__(kThreads, 1) void gemm_pair_kernel(PL1 pl1, QL1 ql1, EP1 ep1, SplitPlan plan1,
                                                                PL2 pl2, QL2 ql2, EP2 ep2, SplitPlan plan2,
                                                                int k1) {
  typedef SmemLayout<PL1, QL1> L1;
  typedef SmemLayout<PL2, QL2> L2;
  __shared__ __attribute__((aligned(16))) char smem[L1::kBytes > L2::kBytes ? L1::kBytes : L2::kBytes];
  __shared__ int s_flag;
  const int x = blockIdx.x % 8, k = blockIdx.x / 8;
  if (k < k1) {
    const int b = 8 * k + x;
    if (b < plan1.grid) gemm_body<MT, MAP1>(pl1, ql1, ep1, plan1, cta_order(b, plan1.grid), smem, &s_flag);
  } else {
    const int b = 8 * (k - k1) + x;
    if (b < plan2.grid) gemm_body<MT, MAP2>(pl2, ql2, ep2, plan2, cta_order(b, plan2.grid), smem, &s_flag);
  }
}

// ---------------------------------------------------------------------------
// Host side: choice of the split, workspace, launch.
// ---------------------------------------------------------------------------

TestKnobs& test_knobs() {
  static TestKnobs knobs;
  return knobs;
}

hipError_t take_split_timeouts(unsigned int* count) {
  unsigned int* d = nullptr;
  if (hipError_t e = hipGetSymbolAddress(reinterpret_cast<void**>(&d), HIP_SYMBOL(g_split_timeouts))) return e;
  if (hipError_t e = hipDeviceSynchronize()) return e;
  if (hipError_t e = hipMemcpy(count, d, sizeof(unsigned int), hipMemcpyDeviceToHost)) return e;
  const unsigned int zero = 0;
  return hipMemcpy(d, &zero, sizeof(unsigned int), hipMemcpyHostToDevice);
}

int64_t debug_split_pieces(int64_t T, int S, int G, int32_t* v, int32_t* t, int32_t* s0, int32_t* s1,
                           int64_t* slot, int32_t* va, int32_t* n, int64_t cap) {
  SplitPlan p{};
  p.total = T * S;
  p.grid = G;
  p.nstages = S;
  p.nslots = partial_slots(T, G);
  int64_t k = 0;
  for (int w = 0; w < G; ++w) {
    const int64_t hi = split_lo(p, w + 1);
    for (int64_t it = split_lo(p, w); it < hi;) {
      int tt, a, b, o, c;
      split_piece(p, it, hi, &tt, &a, &b);
      split_tile_owners(p, tt, &o, &c);
      if (k < cap) {
        v[k] = w;
        t[k] = tt;
        s0[k] = a;
        s1[k] = b;
        slot[k] = piece_slot(p, w, tt);
        va[k] = o;
        n[k] = c;
      }
      ++k;
      it += b - a;
    }
  }
  return k;
}

void debug_cta_order(int G, int32_t* out) {
  for (int b = 0; b < G; ++b) out[b] = cta_order(b, G);
}

constexpr int kMaxGrid = 256;  // workgroups of a split launch (one per CU)
constexpr size_t kPartialBytes = (size_t)64 * kThreads * 16;  // one partial tile

struct GemmShape {
  int64_t tiles_i, tiles_j, nstages;
  int overhead;  // cost of a split piece's publish / fix-up, in stages
  int64_t tiles() const { return tiles_i * tiles_j; }
};

// Per-piece costs of a split launch, in the product's stages: the last
// piece of a split tile reads every other piece's 256 KiB partial tile on
// its own CU, and a chip with every CU busy runs at a lower clock than one
// with a few idle, so a split must save many stages to pay. Measured
// interleaved on one MI355X, whole tiles against splits over 128-256
// workgroups and the split the cost model picked:
//  - int8 forward at 512, 1024, 2048, 4096, 8192 tokens (K 6912, N 2560),
//    2048 and 4096 tokens (K 2560, N 6912) and 4096, 16384 tokens (K = N =
//    2560): whole tiles were fastest at every shape (4096 x 6912 -> 2560:
//    90.7 us against 100-114 us split; 512 tokens: 69.6 us on 20 CUs
//    against 84.6 us split over 80 workgroups);
//  - dX and dW launched alone at 1024-4096 tokens: 20 stages per piece
//    chooses the fastest or a near-fastest option at every shape (e.g. dX
//    at 4096 x 6912 -> 2560 whole, 144 us against 175 us split; at
//    4096 x 2560 -> 6912 split, 151 us against 163 us whole).
constexpr int kFwdPieceCost = 48;
constexpr int kBwdPieceCost = 20;

static GemmShape shape_of(GemmKind kind, int64_t M, int64_t N, int64_t K) {
  const int64_t Kp = k_pad(K);
  switch (kind) {
    case GemmKind::kFwd:
      return {(N + kBI - 1) / kBI, (M + kBJ - 1) / kBJ, (Kp + kStageBytes - 1) / kStageBytes, kFwdPieceCost};
    // a split piece costs the bf16 forward about 20 of its stages (measured
    // at 4096x2560->6912: whole tiles in two rounds 171 us, split over 256
    // workgroups 185 us)
    case GemmKind::kTtqFwd: return {(N + kBI - 1) / kBI, (M + kBJ - 1) / kBJ, (Kp + kRed16 - 1) / kRed16, 20};
    case GemmKind::kBwdDx:
      return {(K + kBI - 1) / kBI, (M + kBJ - 1) / kBJ, (N + kRed16 - 1) / kRed16, kBwdPieceCost};
    case GemmKind::kBwdDw: case GemmKind::kBwdPair: case GemmKind::kTtqBwd: break;
  }
  return {(K + kBI - 1) / kBI, (N + kBJ - 1) / kBJ, (M + kRed16 - 1) / kRed16, kBwdPieceCost};
}

// Workgroups of a split launch, or 0 for one whole tile per workgroup.
// A split pays when T tiles leave the last round of whole tiles on `cus`
// CUs partly idle; it spreads the T*S stages evenly over at most `cus`
// workgroups and about 4 pieces per tile. The split_ctas test knob
// (bitnet_set_test_knobs) forces a split over that many workgroups, or with
// a negative value whole tiles.
static int split_pays(const GemmShape& g, int cus) {
  const int64_t T = g.tiles(), S = g.nstages, W = T * S;
  if (W < 2 || cus < 1) return 0;
  const int64_t G = (int64_t)cus < 4 * T ? (int64_t)cus : 4 * T;
  const int64_t whole = (T + cus - 1) / cus * S;
  const int64_t split = (W + G - 1) / G + g.overhead;
  return split < whole ? (int)G : 0;
}
static int split_grid(const GemmShape& g, int cus) {
  const int f = test_knobs().split_ctas.load(std::memory_order_relaxed);
  if (f < 0) return 0;
  if (f > 0) {
    const int64_t W = g.tiles() * g.nstages;
    const int64_t G = f < kMaxGrid ? f : kMaxGrid;
    return (int)(G < W ? G : W);
  }
  return split_pays(g, cus);
}

// Split-launch workspace: the tile counters [T][2] (8 bytes each, rounded
// up to 256 bytes), then the partial tiles [partial_slots(T, G)].
static size_t split_control_bytes(const GemmShape& g) { return ((size_t)g.tiles() * 16 + 255) / 256 * 256; }
static size_t split_workspace(const GemmShape& g, int grid) {
  if (grid == 0) return 0;
  return split_control_bytes(g) + (size_t)partial_slots(g.tiles(), grid) * kPartialBytes;
}

// dW's x_hat buffer at the start of its workspace.
static size_t xhat_bytes(int64_t M, int64_t K) { return ((size_t)M * k_pad(K) * 2 + 255) / 256 * 256; }
static int64_t n_pad64(int64_t N) { return (N + 63) / 64 * 64; }
static size_t wt_bytes(int64_t N, int64_t K) { return ((size_t)k_pad(K) * (n_pad64(N) / 2) + 255) / 256 * 256; }

static int device_cus();

// The split grid a launch given ws_bytes of split workspace runs: the grid
// split_grid() chooses, or the largest smaller one whose workspace fits and
// whose split still beats whole tiles on `cus` CUs (a grid forced by the
// knob: the largest that fits); 0: whole tiles.
static int fit_split(const GemmShape& g, int cus, size_t ws_bytes) {
  const int want = split_grid(g, cus);
  if (want == 0 || split_workspace(g, want) <= ws_bytes) return want;
  const bool forced = test_knobs().split_ctas.load(std::memory_order_relaxed) > 0;
  const int64_t T = g.tiles(), S = g.nstages, W = T * S;
  const int64_t whole = (T + cus - 1) / cus * S;
  for (int G = want - 1; G >= 2; --G) {
    if (split_workspace(g, G) > ws_bytes) continue;
    if (forced) return G;
    return (W + G - 1) / G + g.overhead < whole ? G : 0;
  }
  return 0;
}

// TTQ backward: the wave-tile partials of the scale gradients come first.
static int64_t ttq_wave_tiles(int64_t N, int64_t K) {
  const GemmShape g = shape_of(GemmKind::kBwdDw, 1, N, K);
  return 4 * g.tiles();
}
static size_t ttq_partials_bytes(int64_t N, int64_t K) {
  return ((size_t)ttq_wave_tiles(N, K) * sizeof(float2) + 255) / 256 * 256;
}

static int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return kMaxGrid;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) n = kMaxGrid;
    cached[dev] = n < kMaxGrid ? n : kMaxGrid;
  }
  return cached[dev];
}

// Launch tags: a 48-bit counter started at a random value, so tags of
// different launches (and processes) differ.
static uint64_t next_gen() {
  static std::atomic<uint64_t> gen{0};
  static std::once_flag once;
  std::call_once(once, [] {
    std::random_device rd;
    gen.store(((uint64_t)rd() << 20) ^ (uint64_t)rd());
  });
  uint64_t g;
  do {
    g = gen.fetch_add(1) & ((uint64_t(1) << 48) - 1);
  } while (g == 0);
  return g;
}

uint64_t next_launch_tag() { return next_gen(); }

// Cost model of one product on G workgroups, in dX stage times (measured
// at 4096x2560->6912): a tile's pipeline fill and epilogue cost about 5.4
// stages. Per product, the cost of a stage and of each piece of a split
// range (fill, partial exchange, epilogue): dX 1.0 and 10 stages; dW 1.07
// and 21 (dW's pieces exchange more: measured at 4096x2560->6912 and
// 4096x6912->2560, a pair launch whose dW splits over 128 CUs takes
// 325-370 us where dW in whole tiles on 136 CUs takes 260-340 us, which 10
// stages per piece did not predict). Whole tiles taken in turn cost
// ceil(T/G) tiles; a split costs W/G stages plus its pieces (about
// W/(G*S) + 1 per workgroup).
constexpr double kTileCost = 5.4;
struct ProductCosts {
  double stage, piece;
};
constexpr ProductCosts kDxCosts{1.0, 10.0}, kDwCosts{1.07, 21.0};
struct PairCost {
  double t;
  bool split;
};
static PairCost product_cost(const GemmShape& g, int64_t G, const ProductCosts& c) {
  const double T = (double)g.tiles(), S = (double)g.nstages, W = T * S;
  const double whole = std::ceil(T / (double)G) * (S * c.stage + kTileCost);
  const int64_t Gs = G < 4 * g.tiles() ? G : 4 * g.tiles();
  const double split = W / (double)Gs * c.stage + (W / ((double)Gs * S) + 1.0) * c.piece;
  return split < whole ? PairCost{split, true} : PairCost{whole, false};
}

// The 8-workgroup columns (of kt) that run dX in a pair launch: the k1 that
// minimizes the slower product's modelled cost; 0: no pair launch (the
// split_ctas knob is set, or too few CUs). The pair_cols knob overrides k1.
static int pair_columns(const GemmShape& g1, const GemmShape& g2, int cus, int* kt, const ProductCosts& c1,
                        const ProductCosts& c2) {
  if (test_knobs().split_ctas.load(std::memory_order_relaxed) != 0) return 0;
  *kt = (cus < kMaxGrid ? cus : kMaxGrid) / 8;
  if (*kt < 2) return 0;
  const int f = test_knobs().pair_cols.load(std::memory_order_relaxed);
  if (f >= 1 && f < *kt) return f;
  int best = 1;
  double best_t = 1e300;
  for (int k1 = 1; k1 < *kt; ++k1) {
    const double t = std::max(product_cost(g1, 8 * k1, c1).t, product_cost(g2, 8 * (*kt - k1), c2).t);
    if (t < best_t) {
      best_t = t;
      best = k1;
    }
  }
  return best;
}

static SplitPlan split_plan(const GemmShape& g, int grid, void* ws) {
  SplitPlan plan{};
  plan.total = g.tiles() * g.nstages;
  plan.tiles_i = (int)g.tiles_i;
  plan.nstages = (int)g.nstages;
  plan.grid = grid;
  plan.spin_limit = test_knobs().spin_limit.load(std::memory_order_relaxed);
  plan.gen = next_gen();
  plan.nslots = partial_slots(g.tiles(), grid);
  plan.counters = static_cast<uint64_t*>(ws);
  plan.partials = reinterpret_cast<uint4*>(static_cast<char*>(ws) + split_control_bytes(g));
  return plan;
}

// Whole tiles taken in turn by `grid` workgroups (no split).
static SplitPlan whole_plan(const GemmShape& g, int grid) {
  SplitPlan plan{};
  plan.total = g.tiles() * g.nstages;
  plan.tiles_i = (int)g.tiles_i;
  plan.nstages = (int)g.nstages;
  plan.grid = grid;
  return plan;
}

template <class MT, int MAP, class PL, class QL, class EP>
static hipError_t run_gemm(const PL& pl, const QL& ql, const EP& ep, const GemmShape& g, void* ws,
                           size_t ws_bytes, hipStream_t stream) {
  const int grid = ws == nullptr ? 0 : fit_split(g, device_cus(), ws_bytes);
  const SplitPlan plan = grid > 0 ? split_plan(g, grid, ws) : whole_plan(g, (int)g.tiles());
  gemm_kernel<MT, MAP, PL, QL, EP><<<plan.grid, kThreads, 0, stream>>>(pl, ql, ep, plan);
  return hipGetLastError();
}

// Two products in one gemm_pair_kernel launch, each on its own share of the
// CUs (pair_columns), each splitting its tiles only when the cost model says
// that beats whole tiles taken in turn on its share (stage costs c1, c2).
// k1 == 0: no pair launch on this device. s1, s2: split workspace bytes.
struct PairPlan {
  int kt = 0, k1 = 0, G1 = 0, G2 = 0;
  bool sk1 = false, sk2 = false;
  size_t s1 = 0, s2 = 0;
};
static PairPlan plan_pair(const GemmShape& g1, const GemmShape& g2, int cus, const ProductCosts& c1,
                          const ProductCosts& c2) {
  PairPlan pp;
  pp.k1 = pair_columns(g1, g2, cus, &pp.kt, c1, c2);
  if (pp.k1 == 0) return pp;
  // every workgroup of a split needs a non-empty range, and more than about
  // 4 pieces per tile do not pay
  const auto cap = [](const GemmShape& g, int64_t G) {
    const int64_t W = g.tiles() * g.nstages, P = 4 * g.tiles();
    return (int)(G < W ? (G < P ? G : P) : (W < P ? W : P));
  };
  const int64_t share1 = 8 * pp.k1, share2 = 8 * (pp.kt - pp.k1);
  pp.sk1 = product_cost(g1, share1, c1).split;
  pp.sk2 = product_cost(g2, share2, c2).split;
  pp.G1 = pp.sk1 ? cap(g1, share1) : (int)(g1.tiles() < share1 ? g1.tiles() : share1);
  pp.G2 = pp.sk2 ? cap(g2, share2) : (int)(g2.tiles() < share2 ? g2.tiles() : share2);
  pp.s1 = pp.sk1 ? split_workspace(g1, pp.G1) : 0;
  pp.s2 = pp.sk2 ? split_workspace(g2, pp.G2) : 0;
  return pp;
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

// Few tokens run the decode-shaped kernels (the no_skinny test knob keeps
// the large-M GEMMs at any M).
static bool skinny(int64_t M) {
  return M <= kSkinnyMaxM && test_knobs().no_skinny.load(std::memory_order_relaxed) == 0;
}

hipError_t launch_fwd(const int8_t* x_q, const float* s_x, const uint8_t* w_packed,
                      const float* gamma, const uint16_t* bias, int64_t M, int64_t N, int64_t K, uint16_t* y,
                      int32_t* acc_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (skinny(M))
    return launch_fwd_skinny(x_q, s_x, w_packed, gamma, bias, M, N, K, y, acc_out, stream);
  const int64_t Kp = k_pad(K);
  PackedCodesLoader pl{w_packed, Kp / 4, N};
  CopyLoader<1, true> ql{reinterpret_cast<const char*>(x_q), Kp, M, Kp};
  if (bias != nullptr)
    return run_gemm<MfmaI8, 1>(pl, ql, FwdEpilogue<true>{y, acc_out, s_x, gamma, N, M, bias},
                               shape_of(GemmKind::kFwd, M, N, K), ws, ws_bytes, stream);
  return run_gemm<MfmaI8, 1>(pl, ql, FwdEpilogue<false>{y, acc_out, s_x, gamma, N, M, nullptr},
                             shape_of(GemmKind::kFwd, M, N, K), ws, ws_bytes, stream);
}

static hipError_t launch_wt(const uint8_t* w_packed, int64_t N, int64_t K, uint8_t* wt, hipStream_t stream) {
  const int64_t Kp = k_pad(K), Np = n_pad64(N);
  const int wt_bx = (int)(Kp / 64), wt_by = (int)((Np + 255) / 256);
  wt_fp4_kernel<<<wt_bx * wt_by, 256, 0, stream>>>(w_packed, N, Kp, Np, wt, wt_bx, wt_by);
  return hipGetLastError();
}

static hipError_t launch_xhat(const int8_t* x_q, const float* s_x, int64_t M, int64_t K, uint16_t* xhat,
                              hipStream_t stream) {
  const int64_t Kp = k_pad(K);
  const int64_t want = (M * (Kp / 16) + 255) / 256;
  xhat_kernel<<<(int)(want < 4096 ? want : 4096), 256, 0, stream>>>(x_q, s_x, M, Kp, xhat);
  return hipGetLastError();
}

hipError_t launch_bwd_dx(const uint16_t* dY, const uint8_t* w_packed, const float* gamma,
                         int64_t M, int64_t N, int64_t K, uint16_t* dX, void* ws, size_t ws_bytes,
                         hipStream_t stream) {
  const int64_t Kp = k_pad(K), Np = n_pad64(N);
  const size_t wb = wt_bytes(N, K);
  if (ws == nullptr || ws_bytes < wb) return hipErrorInvalidValue;  // the C ABI sized it
  uint8_t* wt = static_cast<uint8_t*>(ws);
  void* split_ws = static_cast<char*>(ws) + wb;
  const size_t split_bytes = ws_bytes - wb;
  if (hipError_t e = launch_wt(w_packed, N, K, wt, stream)) return e;
  if (skinny(M) && N % 8 == 0) return launch_dx_skinny(wt, dY, gamma, M, N, K, dX, stream);

  const RowCodesLoader<CodesFp4Frags> pl{wt, Np / 2, Kp};
  Bf16Epilogue<false> ep{dX, gamma, K, M};
  const GemmShape g = shape_of(GemmKind::kBwdDx, M, N, K);
  if (N % 8 == 0) {
    CopyLoader<2, true> ql{reinterpret_cast<const char*>(dY), 2 * N, M, 2 * N};
    return run_gemm<MfmaBf16, 1>(pl, ql, ep, g, split_ws, split_bytes, stream);
  }
  CopyLoader<2, false> ql{reinterpret_cast<const char*>(dY), 2 * N, M, 2 * N};
  return run_gemm<MfmaBf16, 1>(pl, ql, ep, g, split_ws, split_bytes, stream);
}

// The dW product on x_hat (already built) with epilogue ep.
template <class EP>
static hipError_t run_dw(const uint16_t* dY, const uint16_t* xhat, int64_t M, int64_t N, int64_t K, const EP& ep,
                         void* split_ws, size_t split_bytes, hipStream_t stream) {
  const int64_t Kp = k_pad(K);
  const GemmShape g = shape_of(GemmKind::kBwdDw, M, N, K);
  if (N % 8 == 0) {
    // both operands copied in their memory orientation, fragments read transposed
    const RowCopyBf16Loader<1> pc{xhat, Kp, M, Kp};
    const RowCopyBf16Loader<5> qc{dY, N, M, N};
    return run_gemm<MfmaBf16, 0>(pc, qc, ep, g, split_ws, split_bytes, stream);
  }
  const RowTransposeBf16Loader<true, 3> pl{xhat, Kp, M, Kp};
  if (N % 4 == 0) return run_gemm<MfmaBf16, 0>(pl, RowTransposeBf16Loader<true, 5>{dY, N, M, N}, ep, g, split_ws, split_bytes, stream);
  return run_gemm<MfmaBf16, 0>(pl, RowTransposeBf16Loader<false, 5>{dY, N, M, N}, ep, g, split_ws, split_bytes, stream);
}

// The few-token dW (dw_skinny_kernel, x_hat converted in the kernel from x_q
// and s): N % 8 == 0, a bf16 or f32 output (the 1-bit output runs the
// large-M GEMM's epilogue).
static bool dw_skinny_ok(int64_t M, int64_t N, int64_t K, DwOut dw_out) {
  const int64_t dw_tiles = (k_pad(K) + 255) / 256 * ((N + 63) / 64);
  return skinny(M) && N % 8 == 0 && dw_out != DwOut::kSign1 && dw_tiles < (int64_t(1) << 31);
}
static hipError_t launch_dw_skinny(const int8_t* x_q, const float* s_x, const uint16_t* dY, int64_t M, int64_t N,
                                   int64_t K, void* dW, DwOut dw_out, hipStream_t stream) {
  const int64_t Kp = k_pad(K);
  const int ktiles = (int)((Kp + 255) / 256);
  const unsigned grid = (unsigned)((Kp + 255) / 256 * ((N + 63) / 64));
  if (dw_out == DwOut::kF32)
    dw_skinny_kernel<true><<<grid, 256, 0, stream>>>(x_q, s_x, dY, (int)M, N, Kp, K, ktiles, dW);
  else
    dw_skinny_kernel<false><<<grid, 256, 0, stream>>>(x_q, s_x, dY, (int)M, N, Kp, K, ktiles, dW);
  return hipGetLastError();
}

// Few tokens with both outputs: one bwd_skinny_front_kernel launch (the fp4
// transposed codes and every dW tile), then the few-token dX.
static bool skinny_both_ok(int64_t M, int64_t N, int64_t K, DwOut dw_out) {
  return dw_skinny_ok(M, N, K, dw_out);  // dx_skinny needs N % 8 == 0 as well
}
static hipError_t launch_skinny_front(const uint8_t* w_packed, const int8_t* x_q, const float* s_x,
                                      const uint16_t* dY, int64_t M, int64_t N, int64_t K, uint8_t* wt, void* dW,
                                      DwOut dw_out, hipStream_t stream) {
  const int64_t Kp = k_pad(K), Np = n_pad64(N);
  const int wt_bx = (int)(Kp / 64), wt_by = (int)((Np + 255) / 256);
  const int ktiles = (int)((Kp + 255) / 256);
  const unsigned grid = (unsigned)(wt_bx * wt_by + (Kp + 255) / 256 * ((N + 63) / 64));
  if (dw_out == DwOut::kF32)
    bwd_skinny_front_kernel<true><<<grid, 256, 0, stream>>>(w_packed, Np, wt, wt_bx, wt_by, x_q, s_x, dY, (int)M, N,
                                                            Kp, K, ktiles, dW);
  else
    bwd_skinny_front_kernel<false><<<grid, 256, 0, stream>>>(w_packed, Np, wt, wt_bx, wt_by, x_q, s_x, dY, (int)M, N,
                                                             Kp, K, ktiles, dW);
  return hipGetLastError();
}
static void launch_prep(const uint8_t* w_packed, const int8_t* x_q, const float* s_x, int64_t M, int64_t N,
                        int64_t K, uint8_t* wt, uint16_t* xhat, hipStream_t stream) {
  const int64_t Kp = k_pad(K), Np = n_pad64(N);
  const int wt_bx = (int)(Kp / 64), wt_by = (int)((Np + 255) / 256);
  const int64_t want = (M * (Kp / 16) + 255) / 256;
  const int xhat_nb = (int)(want < 4096 ? want : 4096);
  bwd_prep_kernel<<<wt_bx * wt_by + xhat_nb, 256, 0, stream>>>(w_packed, N, Kp, Np, wt, wt_bx, wt_by, x_q, s_x, M,
                                                               xhat, xhat_nb);
}

hipError_t launch_bwd_dw(const uint16_t* dY, const int8_t* x_q, const float* s_x, int64_t M,
                         int64_t N, int64_t K, void* dW, DwOut dw_out, void* ws, size_t ws_bytes,
                         hipStream_t stream) {
  if (dw_skinny_ok(M, N, K, dw_out)) return launch_dw_skinny(x_q, s_x, dY, M, N, K, dW, dw_out, stream);
  const size_t xb = xhat_bytes(M, K);
  if (ws == nullptr || ws_bytes < xb) return hipErrorInvalidValue;  // the C ABI sized it
  uint16_t* xhat = static_cast<uint16_t*>(ws);
  void* split_ws = static_cast<char*>(ws) + xb;
  const size_t split_bytes = ws_bytes - xb;
  if (hipError_t e = launch_xhat(x_q, s_x, M, K, xhat, stream)) return e;
  switch (dw_out) {
    case DwOut::kF32: return run_dw(dY, xhat, M, N, K, Bf16Epilogue<true>{dW, nullptr, K, N}, split_ws, split_bytes, stream);
    case DwOut::kSign1:
      return run_dw(dY, xhat, M, N, K, Sign1Epilogue{static_cast<uint8_t*>(dW), k_pad(K), N}, split_ws, split_bytes, stream);
    default: return run_dw(dY, xhat, M, N, K, Bf16Epilogue<false>{dW, nullptr, K, N}, split_ws, split_bytes, stream);
  }
}

// The pair launch of plan_pair on ws (pp.s1 + pp.s2 bytes);
// hipErrorNotSupported (nothing launched): the device or the workspace does
// not allow it.
template <int MAP1, int MAP2, class PL1, class QL1, class EP1, class PL2, class QL2, class EP2>
static hipError_t run_pair(const PL1& p1, const QL1& q1, const EP1& e1, const GemmShape& g1,
                           const ProductCosts& c1, const PL2& p2, const QL2& q2, const EP2& e2, const GemmShape& g2,
                           const ProductCosts& c2, char* ws, size_t ws_bytes, hipStream_t stream) {
  const PairPlan pp = plan_pair(g1, g2, device_cus(), c1, c2);
  if (pp.k1 == 0 || ws_bytes < pp.s1 + pp.s2) return hipErrorNotSupported;
  const SplitPlan plan1 = pp.sk1 ? split_plan(g1, pp.G1, ws) : whole_plan(g1, pp.G1);
  const SplitPlan plan2 = pp.sk2 ? split_plan(g2, pp.G2, ws + pp.s1) : whole_plan(g2, pp.G2);
  gemm_pair_kernel<MfmaBf16, MAP1, PL1, QL1, EP1, MAP2, PL2, QL2, EP2>
      <<<8 * pp.kt, kThreads, 0, stream>>>(p1, q1, e1, plan1, p2, q2, e2, plan2, pp.k1);
  return hipGetLastError();
}

static bool skinny(int64_t M);

// The STE backward products run in one launch when N % 8 == 0, there are
// more than a few tokens and each product would split its tiles on the full
// device anyway.
// The paired launch runs when both products are large enough that their
// split tails and fills are worth sharing: each would split when launched
// alone under a 3-stage piece cost (the gate under which the pair's own
// cost model, plan_pair, was measured; at 4096 x 6912 -> 2560 the pair
// takes 287 us where dX whole and dW split alone take 144 + 190 us).
static bool pair_gate(int64_t M, int64_t N, int64_t K) {
  const int cus = device_cus();
  GemmShape dx = shape_of(GemmKind::kBwdDx, M, N, K), dw = shape_of(GemmKind::kBwdDw, M, N, K);
  dx.overhead = dw.overhead = 3;
  return split_pays(dx, cus) > 0 && split_pays(dw, cus) > 0;
}
static bool pair_eligible(int64_t M, int64_t N, int64_t K) {
  return N % 8 == 0 && !skinny(M) && pair_gate(M, N, K);
}
// TTQ's pair: both operands copied as stored (N, K multiples of 8).
static bool ttq_pair_eligible(int64_t M, int64_t N, int64_t K) {
  return N % 8 == 0 && K % 8 == 0 && pair_gate(M, N, K);
}
static size_t pair_split_bytes(int64_t M, int64_t N, int64_t K) {
  const PairPlan pp = plan_pair(shape_of(GemmKind::kBwdDx, M, N, K), shape_of(GemmKind::kBwdDw, M, N, K),
                                device_cus(), kDxCosts, kDwCosts);
  return pp.k1 == 0 ? 0 : pp.s1 + pp.s2;
}

// Workspace of each entry point, from the plan its launch runs on this
// device (the split grids, the pair's shares and modes). A backward call
// with one output reuses the paired call's workspace: its pre-pass buffer
// comes first and its split grid fits into the rest (fit_split).
size_t gemm_workspace_bytes(GemmKind kind, int64_t M, int64_t N, int64_t K) {
  const int cus = device_cus();
  const auto alone = [&](GemmKind k) {
    const GemmShape g = shape_of(k, M, N, K);
    return split_workspace(g, split_grid(g, cus));
  };
  switch (kind) {
    case GemmKind::kFwd:
      return skinny(M) ? 0 : alone(kind);  // the few-token forward needs none
    case GemmKind::kTtqFwd: return alone(kind);
    case GemmKind::kBwdDx: return wt_bytes(N, K) + (skinny(M) && N % 8 == 0 ? 0 : alone(kind));
    case GemmKind::kBwdDw: return xhat_bytes(M, K) + alone(kind);
    case GemmKind::kBwdPair: {
      // (any dW output: the sign output of few tokens takes the separate route)
      if (skinny_both_ok(M, N, K, DwOut::kBf16))  // the 1-bit dW output runs the two products separately
        return std::max(wt_bytes(N, K), std::max(gemm_workspace_bytes(GemmKind::kBwdDx, M, N, K),
                                                 gemm_workspace_bytes(GemmKind::kBwdDw, M, N, K)));
      if (pair_eligible(M, N, K) && pair_split_bytes(M, N, K) > 0)
        return std::max(wt_bytes(N, K) + xhat_bytes(M, K) + pair_split_bytes(M, N, K),
                        std::max(wt_bytes(N, K), xhat_bytes(M, K)));
      return std::max(gemm_workspace_bytes(GemmKind::kBwdDx, M, N, K),
                      gemm_workspace_bytes(GemmKind::kBwdDw, M, N, K));
    }
    case GemmKind::kTtqBwd: {
      if (ttq_pair_eligible(M, N, K) && pair_split_bytes(M, N, K) > 0)
        return ttq_partials_bytes(N, K) + pair_split_bytes(M, N, K);
      return ttq_partials_bytes(N, K) + std::max(alone(GemmKind::kBwdDx), alone(GemmKind::kBwdDw));
    }
  }
  return 0;
}

hipError_t launch_bwd_pair(const uint16_t* dY, const uint8_t* w_packed, const float* gamma, const int8_t* x_q,
                           const float* s_x, int64_t M, int64_t N, int64_t K, uint16_t* dX, void* dW,
                           DwOut dw_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (ws != nullptr && skinny_both_ok(M, N, K, dw_out) && ws_bytes >= wt_bytes(N, K)) {
    uint8_t* wt = static_cast<uint8_t*>(ws);
    if (hipError_t e = launch_skinny_front(w_packed, x_q, s_x, dY, M, N, K, wt, dW, dw_out, stream)) return e;
    return launch_dx_skinny(wt, dY, gamma, M, N, K, dX, stream);
  }
  if (!pair_eligible(M, N, K) || ws == nullptr) return hipErrorNotSupported;
  const GemmShape g1 = shape_of(GemmKind::kBwdDx, M, N, K), g2 = shape_of(GemmKind::kBwdDw, M, N, K);
  const size_t wb = wt_bytes(N, K), xb = xhat_bytes(M, K);
  const PairPlan pp = plan_pair(g1, g2, device_cus(), kDxCosts, kDwCosts);
  if (pp.k1 == 0 || ws_bytes < wb + xb + pp.s1 + pp.s2) return hipErrorNotSupported;
  char* base = static_cast<char*>(ws);
  uint8_t* wt = reinterpret_cast<uint8_t*>(base);
  uint16_t* xhat = reinterpret_cast<uint16_t*>(base + wb);
  const int64_t Kp = k_pad(K), Np = n_pad64(N);
  launch_prep(w_packed, x_q, s_x, M, N, K, wt, xhat, stream);
  if (hipError_t e = hipGetLastError()) return e;
  const RowCodesLoader<CodesFp4Frags> p1{wt, Np / 2, Kp};
  const CopyLoader<2, true> q1{reinterpret_cast<const char*>(dY), 2 * N, M, 2 * N};
  const Bf16Epilogue<false> e1{dX, gamma, K, M};
  const RowCopyBf16Loader<1> p2{xhat, Kp, M, Kp};
  const RowCopyBf16Loader<5> q2{dY, N, M, N};
  char* sws = base + wb + xb;
  const size_t sbytes = ws_bytes - wb - xb;
  hipError_t e;
  switch (dw_out) {
    case DwOut::kF32:
      e = run_pair<1, 0>(p1, q1, e1, g1, kDxCosts, p2, q2, Bf16Epilogue<true>{dW, nullptr, K, N}, g2, kDwCosts, sws,
                         sbytes, stream);
      break;
    case DwOut::kSign1:
      e = run_pair<1, 0>(p1, q1, e1, g1, kDxCosts, p2, q2, Sign1Epilogue{static_cast<uint8_t*>(dW), Kp, N}, g2,
                         kDwCosts, sws, sbytes, stream);
      break;
    default:
      e = run_pair<1, 0>(p1, q1, e1, g1, kDxCosts, p2, q2, Bf16Epilogue<false>{dW, nullptr, K, N}, g2, kDwCosts, sws,
                         sbytes, stream);
      break;
  }
  // (the C ABI's workspace covers the pair and pair_columns was checked
  // above, so this is not NotSupported; if it were, the separate launches
  // the caller falls back to rebuild both operands)
  return e;
}

// ---------------------------------------------------------------------------
// TTQ products ("TTQ_VERIFICATION.md": pure TTQ, unquantized bf16
// activations; the quantized weight wt [N][Kp] holds bf16(Wp), -bf16(Wn) or
// 0). All three are bf16 MFMA GEMMs with fp32 accumulation.
// ---------------------------------------------------------------------------

// y [M][N] = x [M][K] . wt^T: both operands copied as stored (reduction k
// contiguous).
hipError_t launch_ttq_fwd(const uint16_t* x, const uint16_t* wt, int64_t M, int64_t N, int64_t K, uint16_t* y,
                          void* ws, size_t ws_bytes, hipStream_t stream) {
  const int64_t Kp = k_pad(K);
  const CopyLoader<2, true, 1> pl{reinterpret_cast<const char*>(wt), 2 * Kp, N, 2 * Kp};
  const Bf16Epilogue<false> ep{y, nullptr, N, M};
  const GemmShape g = shape_of(GemmKind::kTtqFwd, M, N, K);
  const char* xb = reinterpret_cast<const char*>(x);
  if (K % 8 == 0) return run_gemm<MfmaBf16, 1>(pl, CopyLoader<2, true, 5>{xb, 2 * K, M, 2 * K}, ep, g, ws, ws_bytes, stream);
  return run_gemm<MfmaBf16, 1>(pl, CopyLoader<2, false, 5>{xb, 2 * K, M, 2 * K}, ep, g, ws, ws_bytes, stream);
}

// The forward from the stored codes: few tokens read the 2-bit codes once
// (launch_ttq_fwd_skinny); otherwise the codes become wt at the start of the
// workspace and the GEMM above runs on it. The no_skinny test knob keeps
// the second route at any M.
static bool ttq_codes_skinny(int64_t M, int64_t K) { return skinny(M) && K % 8 == 0; }
static size_t ttq_wt_bytes(int64_t N, int64_t K) { return ((size_t)N * k_pad(K) * 2 + 255) / 256 * 256; }

size_t ttq_codes_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  // none for the few-token route (a decode caller needs no 2*N*Kp buffer);
  // the no_skinny knob is read here too, so a size queried under it covers
  // the GEMM route
  if (ttq_codes_skinny(M, K)) return 0;
  return ttq_wt_bytes(N, K) + gemm_workspace_bytes(GemmKind::kTtqFwd, M, N, K);
}

hipError_t launch_ttq_fwd_codes(const uint16_t* x, const uint8_t* w_packed, const float* params, int64_t M,
                                int64_t N, int64_t K, uint16_t* y, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (ttq_codes_skinny(M, K)) return launch_ttq_fwd_skinny(x, w_packed, params, M, N, K, y, stream);
  const size_t wb = ttq_wt_bytes(N, K);
  if (ws == nullptr || ws_bytes < wb) return hipErrorInvalidValue;  // the C ABI sized it
  uint16_t* wt = static_cast<uint16_t*>(ws);
  if (hipError_t e = launch_ttq_expand(w_packed, N, K, params, wt, stream)) return e;
  return launch_ttq_fwd(x, wt, M, N, K, y, static_cast<char*>(ws) + wb, ws_bytes - wb, stream);
}

// dX [M][K] = dY [M][N] . wt: wt staged as stored (rows n) and read
// transposed (TrFrags), dY copied as stored.
static hipError_t launch_ttq_dx(const uint16_t* dY, const uint16_t* wt, int64_t M, int64_t N, int64_t K,
                                uint16_t* dX, void* ws, size_t ws_bytes, hipStream_t stream) {
  const int64_t Kp = k_pad(K);
  const RowCopyBf16Loader<5> pl{wt, Kp, N, K};
  const Bf16Epilogue<false> ep{dX, nullptr, K, M};
  const GemmShape g = shape_of(GemmKind::kBwdDx, M, N, K);
  const char* db = reinterpret_cast<const char*>(dY);
  if (N % 8 == 0) return run_gemm<MfmaBf16, 0>(pl, CopyLoader<2, true, 1>{db, 2 * N, M, 2 * N}, ep, g, ws, ws_bytes, stream);
  return run_gemm<MfmaBf16, 0>(pl, CopyLoader<2, false, 1>{db, 2 * N, M, 2 * N}, ep, g, ws, ws_bytes, stream);
}

// dW [N][K] = dY^T x with the masked sums (TtqDwEpilogue).
template <bool OUT_F32>
static hipError_t launch_ttq_dw(const uint16_t* dY, const uint16_t* x, const uint8_t* w_packed, int64_t M, int64_t N,
                                int64_t K, void* dW, float2* partials, void* ws, size_t ws_bytes, hipStream_t stream) {
  const GemmShape g = shape_of(GemmKind::kBwdDw, M, N, K);
  const TtqDwEpilogue<OUT_F32> ep{Bf16Epilogue<OUT_F32>{dW, nullptr, K, N}, w_packed, (uint32_t)(k_pad(K) / 4),
                                  partials, (int)(2 * g.tiles_i)};
  if (K % 8 == 0 && N % 8 == 0)
    return run_gemm<MfmaBf16, 0>(RowCopyBf16Loader<1>{x, K, M, K}, RowCopyBf16Loader<5>{dY, N, M, N}, ep, g, ws,
                                 ws_bytes, stream);
  if (K % 4 == 0 && N % 4 == 0)
    return run_gemm<MfmaBf16, 0>(RowTransposeBf16Loader<true, 3>{x, K, M, K},
                                 RowTransposeBf16Loader<true, 5>{dY, N, M, N}, ep, g, ws, ws_bytes, stream);
  return run_gemm<MfmaBf16, 0>(RowTransposeBf16Loader<false, 3>{x, K, M, K},
                               RowTransposeBf16Loader<false, 5>{dY, N, M, N}, ep, g, ws, ws_bytes, stream);
}

// dX and dW in one gemm_pair_kernel launch (as the BitNet backward):
// hipErrorNotSupported when the shape or the device does not allow it.
template <bool OUT_F32>
static hipError_t launch_ttq_pair(const uint16_t* dY, const uint16_t* x, const uint16_t* wt, const uint8_t* w_packed,
                                  int64_t M, int64_t N, int64_t K, uint16_t* dX, void* dW, float2* partials,
                                  char* ws, size_t ws_bytes, hipStream_t stream) {
  if (!ttq_pair_eligible(M, N, K)) return hipErrorNotSupported;
  const int64_t Kp = k_pad(K);
  const GemmShape g1 = shape_of(GemmKind::kBwdDx, M, N, K), g2 = shape_of(GemmKind::kBwdDw, M, N, K);
  const RowCopyBf16Loader<5> p1{wt, Kp, N, K};
  const CopyLoader<2, true, 1> q1{reinterpret_cast<const char*>(dY), 2 * N, M, 2 * N};
  const Bf16Epilogue<false> e1{dX, nullptr, K, M};
  const RowCopyBf16Loader<1> p2{x, K, M, K};
  const RowCopyBf16Loader<5> q2{dY, N, M, N};
  const TtqDwEpilogue<OUT_F32> e2{Bf16Epilogue<OUT_F32>{dW, nullptr, K, N}, w_packed, (uint32_t)(Kp / 4), partials,
                                  (int)(2 * g2.tiles_i)};
  // stage costs as for the BitNet pair: measured alone at 4096x2560->6912,
  // this dX (bf16 weight) takes 158-166 us and dW 176-189 us, about the
  // BitNet products' ratio; 15 of 32 columns for dX then give 260 us, 16
  // give 325 us (equal costs chose 16)
  return run_pair<0, 0>(p1, q1, e1, g1, kDxCosts, p2, q2, e2, g2, kDwCosts, ws, ws_bytes, stream);
}

hipError_t launch_ttq_bwd(const uint16_t* dY, const uint16_t* x, const uint16_t* wt, const uint8_t* w_packed,
                          int64_t M, int64_t N, int64_t K, uint16_t* dX, void* dW, bool dw_f32, float* grads,
                          void* ws, size_t ws_bytes, hipStream_t stream) {
  const size_t pb = ttq_partials_bytes(N, K);
  if (ws == nullptr || ws_bytes < pb) return hipErrorInvalidValue;  // the C ABI sized it
  float2* partials = static_cast<float2*>(ws);
  char* split_ws = static_cast<char*>(ws) + pb;
  const size_t split_bytes = ws_bytes - pb;
  float2* p = grads != nullptr ? partials : nullptr;
  if (dX != nullptr && dW != nullptr) {
    const hipError_t e =
        dw_f32 ? launch_ttq_pair<true>(dY, x, wt, w_packed, M, N, K, dX, dW, p, split_ws, split_bytes, stream)
               : launch_ttq_pair<false>(dY, x, wt, w_packed, M, N, K, dX, dW, p, split_ws, split_bytes, stream);
    if (e != hipErrorNotSupported) {
      if (e != hipSuccess || grads == nullptr) return e;
      ttq_grads_kernel<<<1, 256, 0, stream>>>(partials, (int)ttq_wave_tiles(N, K), grads);
      return hipGetLastError();
    }
  }
  if (dX != nullptr)
    if (hipError_t e = launch_ttq_dx(dY, wt, M, N, K, dX, split_ws, split_bytes, stream)) return e;
  if (dW != nullptr) {
    const hipError_t e = dw_f32 ? launch_ttq_dw<true>(dY, x, w_packed, M, N, K, dW, p, split_ws, split_bytes, stream)
                                : launch_ttq_dw<false>(dY, x, w_packed, M, N, K, dW, p, split_ws, split_bytes, stream);
    if (e != hipSuccess) return e;
    if (grads != nullptr) {
      ttq_grads_kernel<<<1, 256, 0, stream>>>(partials, (int)ttq_wave_tiles(N, K), grads);
      return hipGetLastError();
    }
  }
  return hipSuccess;
}

}  // namespace bitnet
