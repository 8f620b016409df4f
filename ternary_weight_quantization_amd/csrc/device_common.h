// Device helpers shared by the gfx950 kernels of libbitnet.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bitnet {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x16_t __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

// bf16 bit pattern -> float (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// bf16 values b[n .. n+3] as floats, 0 at or past N (n a multiple of 4,
// b 8-byte aligned).
__device__ __forceinline__ float4 bias4(const uint16_t* b, int64_t N, int64_t n) {
  if (n + 4 <= N) {
    const uint2 v = *reinterpret_cast<const uint2*>(b + n);
    return make_float4(bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y));
  }
  float r[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = n + e < N ? bf16_to_f32(b[n + e]) : 0.0f;
  return make_float4(r[0], r[1], r[2], r[3]);
}

// Two floats -> packed bf16 pair (lo in bits 0..15), round half to even.
// gfx950 has a native instruction for this (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  __bf16 a = (__bf16)lo;
  __bf16 b = (__bf16)hi;
  return uint32_t(__builtin_bit_cast(uint16_t, a)) | (uint32_t(__builtin_bit_cast(uint16_t, b)) << 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float v) {
  __bf16 a = (__bf16)v;
  return __builtin_bit_cast(uint16_t, a);
}

// Byte permute: selector bytes 0..3 pick bytes of `lo`, 4..7 bytes of `hi`.
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// Four 2-bit codes in the byte lanes of c (values 0, 1, 3) -> four int8.
__device__ __forceinline__ uint32_t codes4_to_i8(uint32_t c) {
  // table: code 0 -> 0x00, 1 -> 0x01, 3 -> 0xFF (code 2 never written)
  return perm(0u, 0xFF000100u, c);
}

// Sum over the 64 lanes of a wave in a fixed butterfly order; every lane
// receives a value, lane 0's is the one used (deterministic).
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

}  // namespace bitnet

namespace bitnet {

// Raw buffer access (CDNA buffer resource, stride 0): loads at byte offsets
// >= num_records return zeros, which gives branch-free zero fill for rows
// and stages past an operand's end. Offsets are 32-bit, so one operand
// addressed this way must stay below 2 GiB (checked by the C ABI).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOob = 0x80000000u;  // an offset past every resource

__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t num_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)num_bytes, 0x00020000);
}

__device__ __forceinline__ uint4 buf_load16(rsrc_t r, uint32_t off) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint2 buf_load8(rsrc_t r, uint32_t off) {
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 v = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
  return make_uint2(v.x, v.y);
}

__device__ __forceinline__ uint32_t buf_load4(rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}

// Streaming store (cache policy nt) at voffset + soffset (soffset uniform),
// for outputs written once and not read again by the launch, so that they
// take less L2 capacity from the operands still being read. A store whose
// voffset is >= num_records is dropped; callers keep voffset + soffset
// inside the resource for the stores they mean to happen.
constexpr int kNonTemporal = 2;

__device__ __forceinline__ void buf_store16_stream(rsrc_t r, uint32_t voff, uint32_t soff, uint4 v) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  __builtin_amdgcn_raw_buffer_store_b128(u32x4{v.x, v.y, v.z, v.w}, r, (int)voff, (int)soff, kNonTemporal);
}

// Device-coherent 16-byte access (cache policy sc1): stores write through
// and loads read past the XCD-private L2 caches, so data exchanged between
// workgroups on different XCDs needs no cache-wide writeback or invalidate.
constexpr int kDeviceCoherent = 16;

__device__ __forceinline__ void buf_store16_coherent(rsrc_t r, uint32_t off, uint4 v) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  __builtin_amdgcn_raw_buffer_store_b128(u32x4{v.x, v.y, v.z, v.w}, r, (int)off, 0, kDeviceCoherent);
}

__device__ __forceinline__ uint4 buf_load16_coherent(rsrc_t r, uint32_t off) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kDeviceCoherent));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Wait until every vector memory access of this wave has completed
// (s_waitcnt vmcnt(0)); for device-coherent stores, until they are visible
// to every workgroup on the device.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

}  // namespace bitnet
