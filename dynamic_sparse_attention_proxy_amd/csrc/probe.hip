// Measurement probe (not part of the CRISP ABI): sustained throughput of the
// MFMA instruction the attention kernels are built on, on caller-supplied
// operand data.  The chip's clock under load depends on the data the matrix
// cores see, so the benchmark feeds the same distribution the attention
// kernels see (N(0,1) bf16) and reports its kernels against this ceiling
// beside the vendor peak.
//
// Each wave keeps 8 A and 8 B operands in VGPRs and issues independent
// v_mfma_f32_32x32x16_bf16 chains into 4 accumulators; 256-thread
// workgroups with 64 KiB of LDS, two per CU, the occupancy of the attention
// kernel.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256, 2) void mfma_probe_kernel(const bf16x8* ops, float* sink, int iters) {
  __shared__ float pad[16384];  // 64 KiB: two workgroups per CU
  if (threadIdx.x == 0) pad[0] = 0.f;
  const int lane = threadIdx.x & 63;
  bf16x8 a[8], b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = ops[i * 64 + lane];
    b[i] = ops[(8 + i) * 64 + lane];
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 8; u += 4) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[u], b[u], c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[u + 1], b[(u + 3) & 7], c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[u + 2], b[(u + 5) & 7], c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[u + 3], b[(u + 6) & 7], c3, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < 8; u += 4) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[u], a[(u + 1) & 7], c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[u + 1], a[(u + 2) & 7], c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[u + 2], a[(u + 7) & 7], c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[u + 3], a[(u + 4) & 7], c3, 0, 0, 0);
    }
  }
  float s = pad[0];
#pragma unroll
  for (int v = 0; v < 16; ++v) s += c0[v] + c1[v] + c2[v] + c3[v];
  sink[blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// ops: 16 x 64 x 8 bf16 operand values (device), sink: nblocks x 256 floats
// (device).  Enqueues nblocks workgroups of `iters` trips on `stream`; each
// trip is 16 MFMAs of 32 x 32 x 16 per wave, 4 waves per workgroup.
// Returns 0, or 1 for bad arguments, 2 if the launch failed.
__attribute__((visibility("default"))) int crisp_probe_mfma_bf16(const void* ops, float* sink, int nblocks,
                                                                  int iters, void* stream) {
  if (ops == nullptr || sink == nullptr || nblocks <= 0 || iters <= 0) return 1;
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(nblocks), dim3(256), 0, (hipStream_t)stream, (const bf16x8*)ops, sink,
                     iters);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Floating-point operations one call performs.
__attribute__((visibility("default"))) double crisp_probe_mfma_bf16_flops(int nblocks, int iters) {
  return (double)nblocks * 4.0 * iters * 16.0 * (32.0 * 32.0 * 16.0 * 2.0);
}

}  // extern "C"
