// FlexPrefill's routing signal, the one C_struct replaces: a pooled attention
// estimate of the last query block over the key blocks, compared by
// Jensen-Shannon divergence with the proxy attention summed per key block.
//
// Source: "CRISP: Cliff-awaRe Input-adaptive Sparse Prefilling with
// Structural-Mass-Motivated Routing", ai.info summary, "Key Contributions"
// items 1 and 2 (C_struct drops the pooled matmul and the KL divergence of
// JSD routing and reproduces its decisions) and "Methodology in Plain
// English" (the pooled estimate is compared with the per-query attention to
// decide whether a head is concentrated).
//
// Three kernels:
//   jsd_qpool:  qbar[h] = mean of the head's last 128 query rows (fp32).
//   jsd_logits: one wave per (KV group, key block) mean-pools the block's
//               keys (128, or fewer in a partial last block) and scores it against qbar of every query head of
//               the group: logit2[h][kb] = scale * log2(e) * <qbar, kbar>.
//               This is the pass that reads all of K (HBM-bound).
//   jsd_final:  per head, softmax of the logits, the block-summed proxy
//               (lo + up + up2) / 128 from the block masses, their divergence and
//               the route.
//
// The divergence is evaluated as sum_kb (s/2) f(delta) with s the midpoint
// mass, delta = (a - p) / (a + p) and f(d) = (1+d) ln(1+d) + (1-d) ln(1-d),
// which equals the mean of the two KL terms against the midpoint but has no
// cancellation between them: f is even and non-negative, and near 0 its
// series d^2 + d^4/6 + d^6/15 + ... (coefficient 1 / (k (2k-1))) is used.

#include <hip/hip_runtime.h>
#include <math.h>

#include "common.h"
#include "internal.h"

namespace crisp {
namespace {

constexpr int kJWaves = 4;  // key blocks per workgroup of the logits pass

__global__ __launch_bounds__(256) void jsd_qpool_kernel(const __bf16* q, float* qbar, int n) {
  __shared__ float part[16][kHeadDim];
  const int h = blockIdx.x, tid = threadIdx.x;
  const __bf16* src = q + ((size_t)h * n + (n - kBlock)) * kHeadDim;
  const int dc = tid & 15, rg = tid >> 4;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
  for (int rr = 0; rr < 8; ++rr) {
    const u32x4 x = *(const u32x4*)(src + (size_t)(rg * 8 + rr) * kHeadDim + 8 * dc);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[2 * j] += bf16lo_to_f(x[j]);
      acc[2 * j + 1] += bf16hi_to_f(x[j]);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[rg][8 * dc + e] = acc[e];
  __syncthreads();
  if (tid < kHeadDim) {
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) s += part[r][tid];
    qbar[(size_t)h * kHeadDim + tid] = s * (1.f / kBlock);
  }
}

// Lane layout of one wave over a 128 x 128 bf16 key block: lane = 16 rg + dc
// holds dims 8dc .. 8dc+7 and rows rg, rg+4, ..., so each load instruction
// reads four whole 256-byte rows (1 KiB contiguous).
__global__ __launch_bounds__(256) void jsd_logits_kernel(const __bf16* k, const float* qbar, float* logit2, int n,
                                                         int nblk, int qpg, float scale_log2) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int kb = blockIdx.x * kJWaves + wave, g = blockIdx.y;
  if (kb >= nblk) return;
  const int dc = lane & 15, rg = lane >> 4;
  const int rows = min(kBlock, n - kb * kBlock);  // fewer in a partial last block
  const __bf16* src = k + ((size_t)g * n + (size_t)kb * kBlock + rg) * kHeadDim + 8 * dc;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    u32x4 x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const u32x4 zero = {0u, 0u, 0u, 0u};
      const int r = 4 * (16 * half + i) + rg;
      x[i] = r < rows ? *(const u32x4*)(src + (size_t)(4 * (16 * half + i)) * kHeadDim) : zero;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[2 * j] += bf16lo_to_f(x[i][j]);
        acc[2 * j + 1] += bf16hi_to_f(x[i][j]);
      }
  }
  // sum over the four row groups: every lane then holds 8 dims of the block's key sum
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    acc[e] += __shfl_xor(acc[e], 16);
    acc[e] += __shfl_xor(acc[e], 32);
  }
  const float sc = scale_log2 / (float)rows;
  for (int j = rg; j < qpg; j += 4) {
    const int h = g * qpg + j;
    const f32x4* qv = (const f32x4*)(qbar + (size_t)h * kHeadDim + 8 * dc);
    const f32x4 q0 = qv[0], q1 = qv[1];
    float d = acc[0] * q0[0] + acc[1] * q0[1] + acc[2] * q0[2] + acc[3] * q0[3] + acc[4] * q1[0] +
              acc[5] * q1[1] + acc[6] * q1[2] + acc[7] * q1[3];
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) d += __shfl_xor(d, o);
    if (dc == 0) logit2[(size_t)h * nblk + kb] = d * sc;
  }
}

// f(d) = (1+d) ln(1+d) + (1-d) ln(1-d) for |d| <= 1, with 0 ln 0 = 0.
__device__ __forceinline__ float jsd_f(float d) {
  const float a = fabsf(d);
  if (a < 0.25f) {
    const float d2 = d * d;
    return d2 * (1.f + d2 * (1.f / 6.f + d2 * (1.f / 15.f + d2 * (1.f / 28.f + d2 * (1.f / 45.f)))));
  }
  float r = (1.f + a) * log1pf(a);
  if (a < 1.f) r += (1.f - a) * log1pf(-a);
  return r;
}

constexpr int kFinalThreads = 1024;  // N <= 4096 key blocks: at most four per thread

__global__ __launch_bounds__(kFinalThreads) void jsd_final_kernel(const float* logit2, const float* mass,
                                                                  float* js_dist, int32_t* route,
                                                                  float* estimate, int hq, int nblk,
                                                                  float tau_jsd) {
  __shared__ float red[kFinalThreads / 64 + 1];
  const int h = blockIdx.x, tid = threadIdx.x;
  const float* l = logit2 + (size_t)h * nblk;
  const float* lo = mass + (size_t)h * nblk;
  const float* up = mass + ((size_t)hq + h) * nblk;
  const float* up2 = mass + ((size_t)2 * hq + h) * nblk;
  float m = -INFINITY;
  for (int b = tid; b < nblk; b += kFinalThreads) m = fmaxf(m, l[b]);
  m = block_max_f(m, red, tid, kFinalThreads);
  float z = 0.f;
  for (int b = tid; b < nblk; b += kFinalThreads) z += fast_exp2(l[b] - m);
  z = block_sum_f(z, red, tid, kFinalThreads);
  const float inv_z = 1.f / z;
  float acc = 0.f;
  for (int b = tid; b < nblk; b += kFinalThreads) {
    const float p = fast_exp2(l[b] - m) * inv_z;
    if (estimate != nullptr) estimate[(size_t)h * nblk + b] = p;
    const float a = (lo[b] + up[b] + up2[b]) * (1.f / kBlock);
    const float t = a + p;
    if (t > 0.f) acc += 0.25f * t * jsd_f((a - p) / t);  // (s / 2) f(delta), s = t / 2
  }
  const float jsd = block_sum_f(acc, red, tid, kFinalThreads);
  if (tid == 0) {
    const float dist = sqrtf(fmaxf(jsd, 0.f));
    js_dist[h] = dist;
    route[h] = dist >= tau_jsd ? 1 : 0;
  }
}

}  // namespace

size_t jsd_workspace_bytes(int hq, int n) {
  return (size_t)hq * kHeadDim * sizeof(float) + (size_t)hq * nblocks(n) * sizeof(float);
}

hipError_t launch_route_jsd(const __bf16* q, const __bf16* k, const float* mass, float* js_dist, int32_t* route,
                            float* estimate, void* workspace, int hq, int hkv, int n, float scale, float tau_jsd,
                            hipStream_t stream) {
  const int nblk = nblocks(n), qpg = hq / hkv;
  float* qbar = (float*)workspace;
  float* logit2 = qbar + (size_t)hq * kHeadDim;
  hipLaunchKernelGGL(jsd_qpool_kernel, dim3(hq), dim3(256), 0, stream, q, qbar, n);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(jsd_logits_kernel, dim3((nblk + kJWaves - 1) / kJWaves, hkv), dim3(64 * kJWaves), 0, stream, k,
                     qbar, logit2, n, nblk, qpg, scale * kLog2e);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(jsd_final_kernel, dim3(hq), dim3(kFinalThreads), 0, stream, logit2, mass, js_dist, route,
                     estimate, hq, nblk, tau_jsd);
  return hipGetLastError();
}

}  // namespace crisp
