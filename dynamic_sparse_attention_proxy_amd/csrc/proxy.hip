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
// Pass 2 (map): recompute S and form exp2(t - lse2).  It stores the map (a
//   half-wave writes 128 contiguous bytes of one row per store) and/or the
//   block masses: per (head, key block) the map's mass on and below the
//   tile diagonal (row >= column) and above it.  A workgroup's 512 keys are
//   4 whole key blocks and its 4 waves all 128 rows, so each block's masses
//   are complete inside one workgroup.
// Route: C_struct = mean over rows of the mass on the first sink_width and
//   the last recency_width columns (from the map, or from the block masses
//   of key blocks 0 and N-1 when both widths are 128); VS when
//   C_struct >= tau.

#include "common.h"
#include "internal.h"

namespace crisp {

namespace {

struct ProxyArgs {
  const __bf16* q;
  const __bf16* k;
  float* amap;
  float* mass;   // [2][Hq][N]: on/below, above the tile diagonal
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
  // A chunk is whole key blocks, so key0 + 32 < kend always; the second
  // prefetch is clamped into the chunk on the last trip (its data unused),
  // which keeps both loads unconditional.
  for (int key0 = kbeg; key0 < kend; key0 += 64) {
    load_k_tile(kg + (size_t)(key0 + 32) * kHeadDim, kb);
    consume(ka, key0);
    load_k_tile(kg + (size_t)min(key0 + 64, kend - 32) * kHeadDim, ka);
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

template <bool kMap, bool kMass>
__global__ __launch_bounds__(256) void proxy_map_kernel(ProxyArgs p) {
  __shared__ float part[4][4][2];  // [wave][key block of the chunk][lower, upper]
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
  float lo = 0.f, up = 0.f;  // this lane's mass of the current key block
  bf16x8 ka[8], kb[8];
  load_k_tile(kg + (size_t)kbeg * kHeadDim, ka);
  auto consume = [&](const bf16x8 (&kf)[8], int key0) {
    const f32x16 s = qk_regs(qf, kf);
    const int key = key0 + l32;
    const bool masked_tile = key0 + 31 > pos0;
    // Sub-block `sub` of the key block holds columns 32 sub .. 32 sub + 31;
    // wave w holds rows 32 w .. 32 w + 31: below the diagonal when sub < w,
    // above when sub > w, split per element when sub == w.
    const int sub = (key0 >> 5) & 3;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = acc_row(w, v, lg);
      float a = fast_exp2(s[v] * p.scale_log2 - lse2[v]);
      if (masked_tile && key > pos0 + r) a = 0.f;
      if (kMap) arow[(size_t)r * p.n + key] = a;
      if (kMass) {
        if (sub < w || (sub == w && r - 32 * w >= l32))
          lo += a;
        else
          up += a;
      }
    }
    if (kMass && sub == 3) {  // last sub-block of a key block: reduce and park the wave's sums
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        lo += __shfl_xor(lo, o);
        up += __shfl_xor(up, o);
      }
      if (lane == 0) {
        part[w][(key0 - kbeg) >> 7][0] = lo;
        part[w][(key0 - kbeg) >> 7][1] = up;
      }
      lo = 0.f;
      up = 0.f;
    }
  };
  // A chunk is whole key blocks, so key0 + 32 < kend always; the second
  // prefetch is clamped into the chunk on the last trip (its data unused),
  // which keeps both loads unconditional.
  for (int key0 = kbeg; key0 < kend; key0 += 64) {
    load_k_tile(kg + (size_t)(key0 + 32) * kHeadDim, kb);
    consume(ka, key0);
    load_k_tile(kg + (size_t)min(key0 + 64, kend - 32) * kHeadDim, ka);
    consume(kb, key0 + 32);
  }
  if (kMass) {
    __syncthreads();
    // the chunk's key blocks (n is a multiple of 128): sum the 4 waves in order
    const int nkb = (kend - kbeg) >> 7;
    if (tid < 2 * nkb) {
      const int j = tid >> 1, which = tid & 1;
      const float m = part[0][j][which] + part[1][j][which] + part[2][j][which] + part[3][j][which];
      const int N = p.n / kBlock, hq = gridDim.y;
      p.mass[((size_t)which * hq + h) * N + (kbeg >> 7) + j] = m;
    }
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

// C_struct from the block masses when sink and recency widths are both one
// block: the mass of key blocks 0 and N-1 over the 128 rows.
__global__ void route_mass_kernel(const float* mass, float* c_struct, int32_t* route, int hq, int nblk, float tau,
                                  int override_mode) {
  const int h = blockIdx.x * blockDim.x + threadIdx.x;
  if (h >= hq) return;
  const float* lo = mass + (size_t)h * nblk;
  const float* up = mass + ((size_t)hq + h) * nblk;
  const float c = (lo[0] + up[0] + lo[nblk - 1] + up[nblk - 1]) / (float)kBlock;
  c_struct[h] = c;
  route[h] = override_mode == 1 ? 1 : override_mode == 2 ? 0 : (c >= tau ? 1 : 0);
}

}  // namespace

hipError_t launch_proxy(const __bf16* q, const __bf16* k, float* amap, float* mass, float* row_lse, void* scratch,
                        int hq, int hkv, int n, float scale, hipStream_t stream) {
  ProxyArgs a;
  a.q = q;
  a.k = k;
  a.amap = amap;
  a.mass = mass;
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
  const dim3 grid(a.nchunks, hq);
  if (amap != nullptr && mass != nullptr)
    hipLaunchKernelGGL((proxy_map_kernel<true, true>), grid, dim3(256), 0, stream, a);
  else if (amap != nullptr)
    hipLaunchKernelGGL((proxy_map_kernel<true, false>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((proxy_map_kernel<false, true>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_route(const float* amap, const float* mass, float* c_struct, int32_t* route, int hq, int n,
                        int sink_width, int recency_width, float tau, int route_override, hipStream_t stream) {
  if (mass != nullptr)
    hipLaunchKernelGGL(route_mass_kernel, dim3((hq + 63) / 64), dim3(64), 0, stream, mass, c_struct, route, hq,
                       n / kBlock, tau, route_override);
  else
    hipLaunchKernelGGL(route_kernel, dim3(hq), dim3(256), 0, stream, amap, c_struct, route, n, sink_width,
                       recency_width, tau, route_override);
  return hipGetLastError();
}

}  // namespace crisp
