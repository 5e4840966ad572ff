// Device-side helpers shared by the CRISP kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace crisp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBlock = 128;    // query/key block (B)
constexpr int kHeadDim = 128;  // d
constexpr int kNumXcd = 8;     // MI355X: 8 accelerator dies, workgroups dealt round-robin
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 32x32x16 bf16 MFMA: C[32x32] += A[32x16] * B[16x32].
// Lane l holds row (A) / column (B) l % 32 and the 8 k-values of k-group l / 32;
// the accumulator lane l holds column l % 32, rows 8*(v/4) + 4*(l/32) + v%4.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// LDS chunk swizzles of [row][128 bf16] tiles (chunk position =
// chunk ^ swz(row)), chosen from measured bank-conflict counts on gfx950.  The K operand read has 16 lanes
// reading one chunk of rows {0..3, 8..11, 4..7, 12..15} (+ multiples of 16):
// any bijection of the row's low 4 bits keeps them apart; this one sends
// (r0, r1) to chunk bits (2, 3) and (r2, r3) to (0, 1).  The transposing
// V^T read has 32 lanes reading chunks c0 .. c0+3 of 4 consecutive rows: the
// row's bits 0-1 must move the chunk's bits 2-3, which (r & 3) << 2 does
// while leaving the other row bits free (so those offsets stay additive).
__device__ __forceinline__ int swz_k(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int swz_v(int r) { return (r & 3) << 2; }

// Buffer resource word 3: raw 32-bit data, no swizzle.
constexpr int kBufferFlags = 0x00020000;

// One LDS-DMA instruction: lane L copies the 16 bytes at byte offset
// voff + soff of buffer `rs` to LDS address lds_addr + 16 L.  Inline asm, so
// the compiler does not insert a vmcnt(0) before unrelated LDS reads; the
// caller waits (wait_dma*) and synchronises before reading.  One wait state
// separates the M0 write from the DMA that reads it.
__device__ __forceinline__ void lds_dma_16B(__amdgpu_buffer_rsrc_t rs, int voff, int soff, unsigned lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(rs), "s"(soff)
               : "memory", "m0");
}

// Wait until this wave's buffer loads (including LDS DMA) have landed.
__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// The same, except for the 4 most recently issued ones (loads complete in order).
__device__ __forceinline__ void wait_dma_but_4() { asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); }

// Lane index (0..63) from an asm statement with side effects, recomputed
// wherever it is written: a loop cannot hoist it or anything derived from it.
__device__ __forceinline__ int opaque_lane() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 u) { return __builtin_bit_cast(bf16x8, u); }

// Round-to-nearest-even fp32 -> bf16 of 8 values (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16x8 pack_bf16x8(float a0, float a1, float a2, float a3, float a4, float a5,
                                              float a6, float a7) {
  bf16x8 r;
  r[0] = (__bf16)a0; r[1] = (__bf16)a1; r[2] = (__bf16)a2; r[3] = (__bf16)a3;
  r[4] = (__bf16)a4; r[5] = (__bf16)a5; r[6] = (__bf16)a6; r[7] = (__bf16)a7;
  return r;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
constexpr bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};
// Sum of the 8 bf16 values of x added to acc (exact products with 1, fp32
// accumulation).  The attention kernels sum the bf16-rounded probabilities
// that enter the PV product, so each output row is an exact weighted mean of
// V rows whatever the rounding.
__device__ __forceinline__ float sum_rounded(bf16x8 x, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 0, 1), kOnes2, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 2, 3), kOnes2, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 4, 5), kOnes2, acc, false);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 6, 7), kOnes2, acc, false);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__device__ __forceinline__ int wave_sum_i(int x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Order-preserving key for non-negative floats with index tie-break:
// ascending key = descending value, then ascending index.
__device__ __forceinline__ uint64_t desc_key(float x, uint32_t idx) {
  uint32_t b = __float_as_uint(x);
  return ((uint64_t)(~b) << 32) | (uint64_t)idx;
}
__device__ __forceinline__ uint32_t key_index(uint64_t k) { return (uint32_t)(k & 0xffffffffu); }
__device__ __forceinline__ float key_value(uint64_t k) { return __uint_as_float(~(uint32_t)(k >> 32)); }

// In-LDS bitonic sort (ascending) of `P` (power of two) 64-bit keys by a
// whole workgroup of `nthreads` threads.  Caller syncs before and after.
__device__ inline void bitonic_sort_lds(uint64_t* keys, int P, int tid, int nthreads) {
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = tid; t < (P >> 1); t += nthreads) {
        int lo = 2 * t - (t & (stride - 1));
        int hi = lo + stride;
        bool up = ((lo & size) == 0);
        uint64_t a = keys[lo], b = keys[hi];
        if ((a > b) == up) {
          keys[lo] = b;
          keys[hi] = a;
        }
      }
      __syncthreads();
    }
  }
}

// Exclusive prefix sum of one int per thread over a workgroup (<= 1024
// threads); returns the exclusive prefix and writes the total.
__device__ inline int block_exclusive_scan(int x, int* lds_tmp, int tid, int nthreads, int* total) {
  const int lane = tid & 63, wid = tid >> 6, nw = (nthreads + 63) >> 6;
  int incl = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) lds_tmp[wid] = incl;
  __syncthreads();
  if (tid == 0) {
    int acc = 0;
    for (int w = 0; w < nw; ++w) {
      int t = lds_tmp[w];
      lds_tmp[w] = acc;
      acc += t;
    }
    lds_tmp[nw] = acc;
  }
  __syncthreads();
  int res = lds_tmp[wid] + incl - x;
  *total = lds_tmp[nw];
  __syncthreads();
  return res;
}

// Inclusive prefix sum of one float per thread in a fixed order
// (wave scan, then a serial pass over wave totals) - deterministic.
__device__ inline float block_inclusive_scan_f(float x, float* lds_tmp, int tid, int nthreads) {
  const int lane = tid & 63, wid = tid >> 6, nw = (nthreads + 63) >> 6;
  float incl = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    float y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) lds_tmp[wid] = incl;
  __syncthreads();
  if (tid == 0) {
    float acc = 0.f;
    for (int w = 0; w < nw; ++w) {
      float t = lds_tmp[w];
      lds_tmp[w] = acc;
      acc += t;
    }
  }
  __syncthreads();
  float res = lds_tmp[wid] + incl;
  __syncthreads();
  return res;
}

// Exclusive prefix sum of one float per thread in a fixed order.
__device__ inline float block_exclusive_scan_f(float x, float* lds_tmp, int tid, int nthreads) {
  const int lane = tid & 63, wid = tid >> 6, nw = (nthreads + 63) >> 6;
  float incl = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    float y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  float excl_w = __shfl_up(incl, 1);
  if (lane == 0) excl_w = 0.f;
  if (lane == 63) lds_tmp[wid] = incl;
  __syncthreads();
  if (tid == 0) {
    float acc = 0.f;
    for (int w = 0; w < nw; ++w) {
      float t = lds_tmp[w];
      lds_tmp[w] = acc;
      acc += t;
    }
  }
  __syncthreads();
  float res = lds_tmp[wid] + excl_w;
  __syncthreads();
  return res;
}

__device__ inline int block_min_i(int x, int* lds_tmp, int tid, int nthreads) {
  const int lane = tid & 63, wid = tid >> 6, nw = (nthreads + 63) >> 6;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = min(x, __shfl_xor(x, o));
  if (lane == 0) lds_tmp[wid] = x;
  __syncthreads();
  if (tid == 0) {
    int acc = lds_tmp[0];
    for (int w = 1; w < nw; ++w) acc = min(acc, lds_tmp[w]);
    lds_tmp[nw] = acc;
  }
  __syncthreads();
  int r = lds_tmp[nw];
  __syncthreads();
  return r;
}

__device__ inline int block_sum_i(int x, int* lds_tmp, int tid, int nthreads) {
  const int lane = tid & 63, wid = tid >> 6, nw = (nthreads + 63) >> 6;
  x = wave_sum_i(x);
  if (lane == 0) lds_tmp[wid] = x;
  __syncthreads();
  if (tid == 0) {
    int acc = 0;
    for (int w = 0; w < nw; ++w) acc += lds_tmp[w];
    lds_tmp[nw] = acc;
  }
  __syncthreads();
  int r = lds_tmp[nw];
  __syncthreads();
  return r;
}

__device__ __forceinline__ float bf16lo_to_f(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16hi_to_f(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Sum of one float per thread over a workgroup in a fixed order.
__device__ inline float block_sum_f(float x, float* lds_tmp, int tid, int nthreads) {
  const int lane = tid & 63, wid = tid >> 6, nw = (nthreads + 63) >> 6;
  float s = wave_sum(x);
  if (lane == 0) lds_tmp[wid] = s;
  __syncthreads();
  if (tid == 0) {
    float acc = 0.f;
    for (int w = 0; w < nw; ++w) acc += lds_tmp[w];
    lds_tmp[nw] = acc;
  }
  __syncthreads();
  float r = lds_tmp[nw];
  __syncthreads();
  return r;
}

// block_sum_f and block_max_f with one barrier: each wave's lane 0 writes
// its partial to lds_tmp[wave], and every thread then combines the partials
// in wave order, so every thread gets the value block_sum_f / block_max_f
// return.  lds_tmp must not be written again until every thread has read it
// (use a separate array for each reduction between two other barriers).
__device__ inline float block_sum_f1(float x, float* lds_tmp, int tid, int nthreads) {
  const int lane = tid & 63, wid = tid >> 6, nw = (nthreads + 63) >> 6;
  const float s = wave_sum(x);
  if (lane == 0) lds_tmp[wid] = s;
  __syncthreads();
  float acc = 0.f;
  for (int w = 0; w < nw; ++w) acc += lds_tmp[w];
  return acc;
}

__device__ inline float block_max_f1(float x, float* lds_tmp, int tid, int nthreads) {
  const int lane = tid & 63, wid = tid >> 6, nw = (nthreads + 63) >> 6;
  const float s = wave_max(x);
  if (lane == 0) lds_tmp[wid] = s;
  __syncthreads();
  float acc = -INFINITY;
  for (int w = 0; w < nw; ++w) acc = fmaxf(acc, lds_tmp[w]);
  return acc;
}

__device__ inline float block_max_f(float x, float* lds_tmp, int tid, int nthreads) {
  const int lane = tid & 63, wid = tid >> 6, nw = (nthreads + 63) >> 6;
  float s = wave_max(x);
  if (lane == 0) lds_tmp[wid] = s;
  __syncthreads();
  if (tid == 0) {
    float acc = -INFINITY;
    for (int w = 0; w < nw; ++w) acc = fmaxf(acc, lds_tmp[w]);
    lds_tmp[nw] = acc;
  }
  __syncthreads();
  float r = lds_tmp[nw];
  __syncthreads();
  return r;
}

// Workgroup -> (head, query block) map of the attention kernels.  Work is
// ordered KV group by KV group (at any time every die works on the same
// group, so the shared last-level cache holds one group's K/V), and within a
// group from the last query block (heaviest: causal rows grow with qb) to
// the first.
struct RowMap {
  int hq, hkv, qpg, nblk, xcd;
};

inline RowMap make_row_map(int hq, int hkv, int nblk) {
  RowMap m;
  m.hq = hq;
  m.hkv = hkv;
  m.qpg = hq / hkv;
  m.nblk = nblk;
  m.xcd = (nblk % 8 == 0) ? 1 : 0;
  return m;
}

// Workgroup id -> (head, query block).  Ids run KV group by KV group.  The
// dispatcher deals workgroups to the 8 XCDs round-robin (id % 8), each XCD
// with its own L2; when the block count is a multiple of 8, XCD x takes the
// query blocks x, x+8, x+16, ... counted from the last (heaviest) one and
// runs the qpg heads of each on consecutive slots, so heads that read the
// same K/V blocks at the same time share an L2.  Otherwise the heads of a
// query block take adjacent ids, heaviest block first.
__host__ __device__ inline void map_row(const RowMap& m, int id, int* h_out, int* qb_out) {
  const int per_group = m.qpg * m.nblk;
  const int g = id / per_group, rem = id - g * per_group;
  int hh, qi;
  if (m.xcd) {
    const int x = rem & 7, s = rem >> 3;
    hh = s % m.qpg;
    qi = 8 * (s / m.qpg) + x;
  } else {
    hh = rem % m.qpg;
    qi = rem / m.qpg;
  }
  *h_out = g * m.qpg + hh;
  *qb_out = m.nblk - 1 - qi;
}

// Query blocks in runs of 16 per XCD: map_row deals XCD x the blocks x,
// x+8, x+16, ... (counted from the last); this permutation of the query
// block gives it 16x .. 16x+15, then 16(x+8) .. 16(x+8)+15, ... instead,
// keeping each XCD's blocks in descending order (block count a multiple of
// 128).
__host__ __device__ inline int runs_of_16(int qb, int nblk) {
  const int qi = nblk - 1 - qb, x = qi & 7, t = qi >> 3;
  return nblk - 1 - (16 * (8 * (t >> 4) + x) + (t & 15));
}

}  // namespace crisp
