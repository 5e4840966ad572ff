// Proxy attention map and structural-mass routing (gfx950).
//
// The proxy rows are the last 128 query positions of every head, attending
// causally to all n keys (CRISP, ai.info summary, "Key Contributions" item 2:
// C_struct reads a proxy attention map the method computes anyway).
//
// Pass 1 (stats): a workgroup takes one head and a chunk of 512 keys; wave w
//   owns proxy rows 32w..32w+31 with Q held as the A operand of S = Q.K^T.
//   K goes straight from global memory into the B operand (lane = key), so
//   each accumulator register holds one row and 32 consecutive keys across a
//   half-wave.  Each lane keeps a running (max, sum of exp2) per row; the 32
//   lanes of a row are merged with a butterfly at the end of the chunk.  The
//   next 32 keys are loaded while the current ones are used.
// Combine: one wavefront per (head, row) merges the chunk partials into the
//   row's log2-sum-exp.
// Pass 2 (map): recompute S and store exp2(t - lse2) - a half-wave writes
//   128 contiguous bytes of one row per store.
// Route: C_struct = mean over rows of the mass on the first sink_width and
//   the last recency_width columns; VS when C_struct >= tau.

#include "common.h"
#include "internal.h"

namespace crisp {

namespace {

struct ProxyArgs {
  const __bf16* q;
  const __bf16* k;
  float* amap;
  float* part;   // [Hq][128][chunks][2]
  float* lse2;   // [Hq][128]
  float* row_lse;
  int n;
  int qpg;
  int nchunks;
  float scale_log2;
};

// Proxy row held by accumulator register v of lane group lg in wave w.
__device__ __forceinline__ int acc_row(int w, int v, int lg) { return 32 * w + 8 * (v >> 2) + 4 * lg + (v & 3); }

__device__ __forceinline__ void merge_ml(float& m, float& l, float mo, float lo) {
  const float M = fmaxf(m, mo);
  if (M == -INFINITY) return;
  l = l * fast_exp2(m - M) + lo * fast_exp2(mo - M);
  m = M;
}

__device__ __forceinline__ void load_q_rows(const ProxyArgs& p, int h, int w, int l32, int lg, bf16x8 qf[8]) {
  const __bf16* qrow = p.q + ((size_t)h * p.n + (size_t)(p.n - kBlock + 32 * w + l32)) * kHeadDim + 8 * lg;
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) qf[kk] = as_bf16x8(*(const u32x4*)(qrow + 16 * kk));
}

__device__ __forceinline__ void load_k_tile(const __bf16* krow, bf16x8 kf[8]) {
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) kf[kk] = as_bf16x8(*(const u32x4*)(krow + 16 * kk));
}

__device__ __forceinline__ f32x16 qk_regs(const bf16x8 qf[8], const bf16x8 kf[8]) {
  f32x16 s;
#pragma unroll
  for (int v = 0; v < 16; ++v) s[v] = 0.f;
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) s = mfma32(qf[kk], kf[kk], s);
  return s;
}

// Partial statistics of proxy row r of head h over key chunk c live at
// part[((h * 128 + r) * nchunks + c) * 2 + {0: max, 1: sum}] (base 2).
__global__ __launch_bounds__(256) void proxy_stats_kernel(ProxyArgs p) {
  const int chunk = blockIdx.x, h = blockIdx.y, g = h / p.qpg;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l32 = lane & 31, lg = lane >> 5;
  bf16x8 qf[8];
  load_q_rows(p, h, w, l32, lg, qf);
  float m[16], l[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    m[v] = -INFINITY;
    l[v] = 0.f;
  }
  const int kbeg = chunk * kProxyChunk;
  const int kend = min(p.n, kbeg + kProxyChunk);
  const __bf16* kg = p.k + (size_t)g * p.n * kHeadDim + (size_t)l32 * kHeadDim + 8 * lg;
  const int pos0 = p.n - kBlock;
  // K sub-blocks of 32 keys, the next one in flight while this one is used
  bf16x8 ka[8], kb[8];
  load_k_tile(kg + (size_t)kbeg * kHeadDim, ka);
  auto consume = [&](const bf16x8 (&kf)[8], int key0) {
    const f32x16 s = qk_regs(qf, kf);
    const int key = key0 + l32;
    const bool masked_tile = key0 + 31 > pos0;  // only the last 128 keys can be masked
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      if (!masked_tile || key <= pos0 + acc_row(w, v, lg)) {
        const float t = s[v] * p.scale_log2;
        const float dlt = t - m[v];
        const float e = fast_exp2(-fabsf(dlt));
        const bool up = dlt > 0.f;
        l[v] = up ? l[v] * e + 1.f : l[v] + e;
        m[v] = up ? t : m[v];
      }
    }
  };
  for (int key0 = kbeg; key0 < kend; key0 += 64) {
    if (key0 + 32 < kend) load_k_tile(kg + (size_t)(key0 + 32) * kHeadDim, kb);
    consume(ka, key0);
    if (key0 + 32 >= kend) break;
    if (key0 + 64 < kend) load_k_tile(kg + (size_t)(key0 + 64) * kHeadDim, ka);
    consume(kb, key0 + 32);
  }
#pragma unroll
  for (int v = 0; v < 16; ++v) {
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) {
      const float mo = __shfl_xor(m[v], o);
      const float lo = __shfl_xor(l[v], o);
      merge_ml(m[v], l[v], mo, lo);
    }
  }
  // lane v of each half-wave writes row acc_row(w, v, lg)
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    if (l32 == v) {
      const int r = acc_row(w, v, lg);
      float* dst = p.part + (((size_t)h * kBlock + r) * p.nchunks + chunk) * 2;
      dst[0] = m[v];
      dst[1] = l[v];
    }
  }
}

// One wavefront per proxy row: lanes stride over the chunk partials, then a
// butterfly merge.
__global__ __launch_bounds__(256) void proxy_combine_kernel(ProxyArgs p) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);  // h * 128 + r
  float m = -INFINITY, l = 0.f;
  const float* src = p.part + (size_t)row * p.nchunks * 2;
  for (int c = lane; c < p.nchunks; c += 64) merge_ml(m, l, src[2 * c], src[2 * c + 1]);
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float mo = __shfl_xor(m, o);
    const float lo = __shfl_xor(l, o);
    merge_ml(m, l, mo, lo);
  }
  if (lane == 0) {
    const float lse2 = m + fast_log2(l);
    p.lse2[row] = lse2;
    if (p.row_lse != nullptr) p.row_lse[row] = lse2 * kLn2;
  }
}

__global__ __launch_bounds__(256) void proxy_map_kernel(ProxyArgs p) {
  const int chunk = blockIdx.x, h = blockIdx.y, g = h / p.qpg;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l32 = lane & 31, lg = lane >> 5;
  bf16x8 qf[8];
  load_q_rows(p, h, w, l32, lg, qf);
  float lse2[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) lse2[v] = p.lse2[h * kBlock + acc_row(w, v, lg)];
  const int kbeg = chunk * kProxyChunk;
  const int kend = min(p.n, kbeg + kProxyChunk);
  const __bf16* kg = p.k + (size_t)g * p.n * kHeadDim + (size_t)l32 * kHeadDim + 8 * lg;
  float* arow = p.amap + (size_t)h * kBlock * p.n;
  const int pos0 = p.n - kBlock;
  bf16x8 ka[8], kb[8];
  load_k_tile(kg + (size_t)kbeg * kHeadDim, ka);
  auto consume = [&](const bf16x8 (&kf)[8], int key0) {
    const f32x16 s = qk_regs(qf, kf);
    const int key = key0 + l32;
    const bool masked_tile = key0 + 31 > pos0;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = acc_row(w, v, lg);
      float a = fast_exp2(s[v] * p.scale_log2 - lse2[v]);
      if (masked_tile && key > pos0 + r) a = 0.f;
      arow[(size_t)r * p.n + key] = a;
    }
  };
  for (int key0 = kbeg; key0 < kend; key0 += 64) {
    if (key0 + 32 < kend) load_k_tile(kg + (size_t)(key0 + 32) * kHeadDim, kb);
    consume(ka, key0);
    if (key0 + 32 >= kend) break;
    if (key0 + 64 < kend) load_k_tile(kg + (size_t)(key0 + 64) * kHeadDim, ka);
    consume(kb, key0 + 32);
  }
}

__global__ __launch_bounds__(256) void route_kernel(const float* amap, float* c_struct, int32_t* route, int n,
                                                    int ws, int wr, float tau, int override_mode) {
  __shared__ float red[8];
  const int h = blockIdx.x, tid = threadIdx.x;
  const float* a = amap + (size_t)h * kBlock * n;
  const int width = ws + wr;
  float acc = 0.f;
  for (int e = tid; e < kBlock * width; e += 256) {
    const int r = e / width, c = e - r * width;
    const int j = (c < ws) ? c : (n - wr + (c - ws));
    acc += a[(size_t)r * n + j];
  }
  const float total = block_sum_f(acc, red, tid, 256);
  if (tid == 0) {
    const float c = total / (float)kBlock;
    c_struct[h] = c;
    int rt;
    if (override_mode == 1)
      rt = 1;
    else if (override_mode == 2)
      rt = 0;
    else
      rt = (c >= tau) ? 1 : 0;
    route[h] = rt;
  }
}

}  // namespace

hipError_t launch_proxy(const __bf16* q, const __bf16* k, float* amap, float* row_lse, void* scratch, int hq,
                        int hkv, int n, float scale, hipStream_t stream) {
  ProxyArgs a;
  a.q = q;
  a.k = k;
  a.amap = amap;
  a.nchunks = proxy_chunks(n);
  a.part = (float*)scratch;
  a.lse2 = a.part + (size_t)hq * a.nchunks * kBlock * 2;
  a.row_lse = row_lse;
  a.n = n;
  a.qpg = hq / hkv;
  a.scale_log2 = scale * kLog2e;
  hipLaunchKernelGGL(proxy_stats_kernel, dim3(a.nchunks, hq), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(proxy_combine_kernel, dim3(hq * kBlock / 4), dim3(256), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(proxy_map_kernel, dim3(a.nchunks, hq), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_route(const float* amap, float* c_struct, int32_t* route, int hq, int n, int sink_width,
                        int recency_width, float tau, int route_override, hipStream_t stream) {
  hipLaunchKernelGGL(route_kernel, dim3(hq), dim3(256), 0, stream, amap, c_struct, route, n, sink_width,
                     recency_width, tau, route_override);
  return hipGetLastError();
}

}  // namespace crisp
