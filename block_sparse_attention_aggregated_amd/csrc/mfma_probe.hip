// The bf16 matrix-core rate the part sustains on operands like the attention's: a
// measurement helper for the attention's roofline, not a step of the method.
//
// Each lane holds eight pairs of operand fragments drawn from a counter hash
// (uniform in [-2, 2), so every bit of the bf16 values toggles as it would on
// activations) and runs eight independent accumulator chains of
// v_mfma_f32_32x32x16_bf16, the attention's instruction, with a new operand pair
// for every instruction.  Two workgroups of four wavefronts per CU: two wavefronts
// per SIMD, as in the attention.  Operands that stay fixed draw far less power than
// these and let the clock rise to its maximum, so the rate measured with them
// would not be reachable by any kernel that multiplies real data.

#include "sparstar_internal.h"

namespace sparstar {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kProbeThreads = 256;
constexpr int kProbeChains = 8;

__device__ inline float hash_uniform(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return (float)(x & 0xffffffu) * (4.0f / 16777216.0f) - 2.0f;
}

__global__ __launch_bounds__(kProbeThreads, 2) void mfma_probe_kernel(int32_t rounds, float* sink) {
  const uint32_t lane_id = blockIdx.x * (uint32_t)kProbeThreads + threadIdx.x;
  bf16x8 a[kProbeChains], b[kProbeChains];
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t h = lane_id * 64u + c * 8u + e;
      a[c][e] = (__bf16)hash_uniform(h);
      b[c][e] = (__bf16)hash_uniform(h ^ 0x9e3779b9u);
    }
  f32x16 acc[kProbeChains];
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
  // One round: 64 instructions, chain c paired with B fragment (c + u) mod 8 in sub-round u.
#pragma unroll 1
  for (int32_t it = 0; it < rounds; ++it) {
#pragma unroll
    for (int u = 0; u < kProbeChains; ++u)
#pragma unroll
      for (int c = 0; c < kProbeChains; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c], b[(c + u) % kProbeChains], acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  sink[lane_id] = s;
}

}  // namespace

int64_t mfma_probe_workgroups() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return -1;
  return 2 * (int64_t)cus;
}

hipError_t launch_mfma_probe(int32_t rounds, float* sink, int64_t workgroups, hipStream_t s) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3((unsigned)workgroups), dim3(kProbeThreads), 0, s, rounds, sink);
  return hipGetLastError();
}

double mfma_probe_flops(int32_t rounds, int64_t workgroups) {
  // per wavefront and round: 64 instructions of 32 x 32 x 16 multiply-adds
  return (double)workgroups * (kProbeThreads / 64) * rounds * 64.0 * (2.0 * 32 * 32 * 16);
}

}  // namespace sparstar
