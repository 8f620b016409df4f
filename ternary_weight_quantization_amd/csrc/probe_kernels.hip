// Rate probe: the MFMA pipes at full occupancy with nothing else to do, the
// practical ceiling the GEMMs' rates are also compared with (the published
// peaks assume a clock the chip does not hold under a full MFMA load).
//
// Every wave runs `iters` rounds of kChains independent MFMAs on register
// operands (no memory traffic, no LDS), so the pipe never waits on a
// dependency. One launch performs
//   blocks * 4 waves * iters * kChains * (2 * 32 * 32 * R)
// operations, R = 16 (bf16) or 32 (int8).

#include "device_common.h"
#include "internal.h"

namespace bitnet {

constexpr int kProbeChains = 8;
constexpr int kProbeBlocks = 2048;

template <bool I8>
__global__ __launch_bounds__(256) void mfma_probe_kernel(int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  if constexpr (I8) {
    i32x4_t a = {lane, lane + 1, lane + 2, lane + 3}, b = {3 * lane, 1, 2, lane};
    i32x16_t acc[kProbeChains];
#pragma unroll
    for (int c = 0; c < kProbeChains; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[c][e] = 0;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < kProbeChains; ++c) acc[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[c], 0, 0, 0);
    }
    int s = 0;
#pragma unroll
    for (int c = 0; c < kProbeChains; ++c) s += acc[c][lane & 15];
    if (s == 0x7fffffff) sink[blockIdx.x] = (float)s;  // keeps the work live; never true in practice
  } else {
    bf16x8_t a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = (__bf16)(float)(lane + e);
      b[e] = (__bf16)(float)(e - lane);
    }
    f32x16_t acc[kProbeChains];
#pragma unroll
    for (int c = 0; c < kProbeChains; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[c][e] = 0.0f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < kProbeChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < kProbeChains; ++c) s += acc[c][lane & 15];
    if (s == 1234.5f) sink[blockIdx.x] = s;  // keeps the work live; never true in practice
  }
}

hipError_t launch_mfma_probe(bool int8, int iters, float* sink, hipStream_t stream) {
  if (int8)
    mfma_probe_kernel<true><<<kProbeBlocks, 256, 0, stream>>>(iters, sink);
  else
    mfma_probe_kernel<false><<<kProbeBlocks, 256, 0, stream>>>(iters, sink);
  return hipGetLastError();
}

double mfma_probe_ops(bool int8, int iters) {
  return (double)kProbeBlocks * 4 * iters * kProbeChains * 2.0 * 32 * 32 * (int8 ? 32 : 16);
}

}  // namespace bitnet
