// Matrix-unit rate probe: back-to-back 16x16x32 bf16 MFMAs on operands held
// in registers, with no memory traffic inside the loop.  The products' MFMA
// fractions are quoted against the datasheet peak; this probe gives the rate
// the part sustains under its power limit with data that toggles like real
// operands, as a second reference.
//
// Each wave loads kProbeChains A and B fragments (16 bytes per lane each)
// from the caller's random bf16 buffer once, then runs `iters` rounds of
// kProbeChains independent matrix instructions (independent accumulators, so
// one instruction's latency is hidden behind the others; consecutive
// instructions take different operands).  The accumulators are summed into
// `sink` so that the loop is not removed.
#include "moe_common.h"
#include "moe_launch.h"
#include "moe_mi355x.h"

namespace moe {

constexpr int kProbeWaves = 8;                     // waves per workgroup
constexpr int kProbeChains = 8;                    // independent accumulators per wave
constexpr int kProbeFragElems = kWave * 8;         // bf16 elements of one 16x32 fragment

__global__ __launch_bounds__(kProbeWaves * kWave) void mfma_probe_kernel(const uint16_t* __restrict__ ops,
                                                                         int64_t nfrag, int64_t iters,
                                                                         float* __restrict__ sink) {
  const int lane = lane_id();
  const int64_t w = (int64_t)blockIdx.x * kProbeWaves + threadIdx.x / kWave;
  uint4 a[kProbeChains], b[kProbeChains];
  floatx4 acc[kProbeChains];
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c) {
    const int64_t fa = (w * 2 * kProbeChains + 2 * c) % nfrag;
    const int64_t fb = (w * 2 * kProbeChains + 2 * c + 1) % nfrag;
    a[c] = *reinterpret_cast<const uint4*>(ops + fa * kProbeFragElems + lane * 8);
    b[c] = *reinterpret_cast<const uint4*>(ops + fb * kProbeFragElems + lane * 8);
    acc[c] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
  for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < kProbeChains; ++c) acc[c] = mfma16x16x32(a[c], b[c], acc[c]);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  sink[w * kWave + lane] = s;
}

hipError_t launch_mfma_probe(const void* ops, int64_t num_ops, int64_t iters, float* sink, hipStream_t s) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(MOE_PROBE_WORKGROUPS), dim3(kProbeWaves * kWave), 0, s,
                     (const uint16_t*)ops, num_ops / kProbeFragElems, iters, sink);
  return hipGetLastError();
}

double mfma_probe_flops(int64_t iters) {
  return (double)MOE_PROBE_WORKGROUPS * kProbeWaves * kProbeChains * (double)iters * (2.0 * 16 * 16 * 32);
}

}  // namespace moe
