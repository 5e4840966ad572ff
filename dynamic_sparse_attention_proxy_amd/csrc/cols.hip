// Single key columns on top of the tile attention, for token-granular
// Vertical-Slash heads (ai-feeds summary, method module 2: the kept set is
// made of tokens above the noise floor; ai.info summary, "Why This Matters":
// exact softmax over what is kept).
//
// The tile kernel has already written, per query row, the softmax over the
// listed key blocks: the normalised output (fp32) and its log-sum-exp.  This
// kernel adds the kept columns that lie below the query block and outside
// its listed tiles, and merges the two softmaxes exactly:
//   out = (out_t 2^L_t + O_c) / (2^L_t + l_c 2^m_c),  L_t = lse_t log2(e),
// where O_c and l_c are the column part's unnormalised sums against its
// running max m_c (base 2).
//
// One workgroup per (head, 128-query block) with kept columns below it; its
// four waves own 32 query rows each, in the orientation of the tile kernel
// (S^T = K.Q^T, a lane owns a query row).  Columns stream 64 at a time:
// each lane reads one column index, a ballot turns "in range and not in a
// listed tile" into the step's 64-bit slot mask, and the K and V rows of the
// 64 columns are gathered into LDS by LDS DMA with per-lane row offsets, in
// the row-major swizzled layout the tile kernel uses, two stages deep.

#include "common.h"
#include "internal.h"

namespace crisp {

namespace {

constexpr int kCStep = 64;          // columns per step
constexpr int kMaxTiles = 4096;     // key blocks per head (n <= 524288)
typedef __bf16 gcc_bf16x4c __attribute__((__vector_size__(8)));
typedef __attribute__((address_space(3))) gcc_bf16x4c lds_bf16x4c;

struct ColArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const int32_t* count;      // tile lists
  const int32_t* idx;
  const int32_t* cols;       // [Hq][n] kept columns, ascending
  const int32_t* col_below;  // [Hq][N] kept columns below 128 qb
  float* out;                // [Hq][n][128]
  float* lse;                // [Hq][n]
  int n;
  int nblk;
  int qpg;
  float scale_log2;
  RowMap map;
};

// Key slot (0..31 within a 32-key half) of accumulator register v of lane
// group lg, for the permuted K-operand rows below.
__device__ __forceinline__ int slot_of(int v, int lg) { return (v < 8) ? (8 * lg + v) : (16 + 8 * lg + (v - 8)); }

__global__ __launch_bounds__(256, 2) void col_attn_kernel(ColArgs p) {
  // V stages 0-1, K stages 2-3
  __shared__ __attribute__((aligned(1024))) __bf16 lds[4][kCStep * kHeadDim];
  __shared__ uint32_t tbits[kMaxTiles / 32];

  int h, qb;
  map_row(p.map, blockIdx.x, &h, &qb);
  const int N = p.nblk;
  // kept columns below this query block (clamped: a malformed count only
  // changes which in-range rows are read)
  const int cnt = min(max(p.col_below[(size_t)h * N + qb], 0), p.n);
  if (cnt == 0 || qb == 0) return;
  const int g = h / p.qpg;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, lg = lane >> 5;
  const int wu = __builtin_amdgcn_readfirstlane(w);

  // listed tiles of (h, qb) as a bitmap
  for (int i = tid; i < kMaxTiles / 32; i += 256) tbits[i] = 0;
  __syncthreads();
  {
    const int tc = min(max(p.count[(size_t)h * N + qb], 0), qb + 1);
    const int32_t* list = p.idx + (size_t)h * ((size_t)N * (N + 1) / 2) + (size_t)qb * (qb + 1) / 2;
    for (int t = tid; t < tc; t += 256) {
      const int kb = min(max(list[t], 0), qb);
      atomicOr(&tbits[kb >> 5], 1u << (kb & 31));
    }
  }
  __syncthreads();

  const size_t nd = (size_t)p.n * kHeadDim;
  const int qpos = qb * kBlock + 32 * w + l32;
  bf16x8 qf[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk)
    qf[kk] = as_bf16x8(*(const u32x4*)(p.q + (size_t)h * nd + (size_t)qpos * kHeadDim + 16 * kk + 8 * lg));

  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.k + (size_t)g * nd), 0, (int)(nd * 2), kBufferFlags);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.v + (size_t)g * nd), 0, (int)(nd * 2), kBufferFlags);
  const int32_t* colh = p.cols + (size_t)h * p.n;
  const int limit = qb * kBlock - 1;  // gathered keys stay below the query block

  // Column of slot `lane` of step s and whether it counts.
  auto load_cols = [&](int s, int* col, uint64_t* mask) {
    const int slot = s * kCStep + lane;
    int c = 0;
    bool ok = false;
    if (slot < cnt) {
      c = min(max(colh[slot], 0), limit);
      ok = (tbits[c >> 12] >> ((c >> 7) & 31) & 1u) == 0;
    }
    *col = c;
    *mask = __ballot(ok);
  };
  // Gather of step s's K and V rows: wave w fills rows 16w .. 16w+15 of each
  // stage; lane L of instruction i row r = 16w + 4i + L/16, chunk position
  // L & 15, i.e. global chunk (L & 15) ^ swz(r) of column col[r].
  auto gather = [&](int stage, int col) {
    __bf16* vst = lds[stage];
    __bf16* kst = lds[2 + stage];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * w + 4 * i + (lane >> 4);
      const int cr = __shfl(col, r);
      const int base = cr * (kHeadDim * 2);
      const unsigned kaddr =
          (unsigned)(uintptr_t)(__attribute__((address_space(3))) void*)(kst + (16 * wu + 4 * i) * kHeadDim);
      const unsigned vaddr =
          (unsigned)(uintptr_t)(__attribute__((address_space(3))) void*)(vst + (16 * wu + 4 * i) * kHeadDim);
      lds_dma_16B(krs, base + (((lane & 15) ^ swz_k(r)) << 4), 0, kaddr);
      lds_dma_16B(vrs, base + (((lane & 15) ^ swz_v(r)) << 4), 0, vaddr);
    }
  };

  // K operand rows in the permuted order of the tile kernel: accumulator
  // registers 0..7 / 8..15 of lane group lg then hold slots 8lg.. / 16+8lg..,
  // the 8 contiguous keys each PV k-group takes as its B operand.
  const int ia = l32 >> 3, ig = (l32 >> 2) & 1, ib = l32 & 3;
  const int krow = 16 * (ia >> 1) + 8 * ig + 4 * (ia & 1) + ib;
  int k_off[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) k_off[kk] = krow * 256 + (((2 * kk + lg) ^ swz_k(krow)) << 4);
  // V^T operand through the transposing LDS read (as in the tile kernel).
  const int gq = lane >> 4, li = lane & 15;
  int v_base[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    const int r = 8 * (gq >> 1) + (li >> 2);
    const int d = 32 * db + 16 * (gq & 1) + 4 * (li & 3);
    v_base[db] = r * 256 + (((d >> 3) ^ swz_v(r)) << 4) + (d & 7) * 2;
  }

  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[db][v] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const int nsteps = (cnt + kCStep - 1) / kCStep;
  int col;
  uint64_t mask;
  load_cols(0, &col, &mask);
  gather(0, col);
  wait_dma();
  __syncthreads();
  for (int s = 0; s < nsteps; ++s) {
    const int st = s & 1;
    const uint64_t mcur = mask;
    if (s + 1 < nsteps) {
      load_cols(s + 1, &col, &mask);
      gather(st ^ 1, col);
    }
    // scores of the 64 gathered keys against the wave's 32 rows
    const char* kb8 = (const char*)lds[2 + st];
    f32x16 sc[2];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
      for (int v = 0; v < 16; ++v) sc[kb2][v] = 0.f;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
        sc[kb2] = mfma32(as_bf16x8(*(const u32x4*)(kb8 + k_off[kk] + kb2 * 8192)), qf[kk], sc[kb2]);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        if (!((mcur >> (32 * kb2 + slot_of(v, lg))) & 1ull)) sc[kb2][v] = -INFINITY;
        mx = fmaxf(mx, sc[kb2][v]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    if (mcur != 0ull) {  // uniform: the step has a counted column
      const float m_new = fmaxf(m_run, mx * p.scale_log2);
      const float alpha = fast_exp2(m_run - m_new);  // 0 while m_run is -inf
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[db][v] *= alpha;
      l_run *= alpha;
      m_run = m_new;
      bf16x8 pb[4];
      float ls = 0.f;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          float x[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            x[i] = fast_exp2(fmaf(sc[kb2][8 * f + i], p.scale_log2, -m_run));
            ls += x[i];
          }
          pb[2 * kb2 + f] = pack_bf16x8(x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]);
        }
      l_run += ls;
      __attribute__((address_space(3))) char* vb8 = (__attribute__((address_space(3))) char*)lds[st];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int db = u & 3, f = u >> 2;
        const int off = v_base[db] + (32 * (f >> 1) + 16 * (f & 1)) * 256;
        const bf16x4 lo = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4c*)(vb8 + off)));
        const bf16x4 hi =
            __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4c*)(vb8 + off + 4 * 256)));
        o[db] = mfma32(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), pb[f], o[db]);
      }
    }
    wait_dma();
    __syncthreads();
  }

  // merge with the tile softmax of the same row
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (!(l_tot > 0.f)) return;  // every gathered column of the row was already in a tile
  const size_t row = (size_t)h * p.n + qpos;
  const float lt = p.lse[row] * kLog2e;
  const float lc = m_run + fast_log2(l_tot);
  const float M = fmaxf(lt, lc);
  const float w1 = fast_exp2(lt - M), wc = fast_exp2(m_run - M);
  const float denom = w1 + l_tot * wc;
  const float inv = 1.f / denom;
  float* orow = p.out + row * kHeadDim;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      f32x4* ptr = (f32x4*)(orow + 32 * db + 8 * a + 4 * lg);
      const f32x4 t = *ptr;
      f32x4 r;
#pragma unroll
      for (int c = 0; c < 4; ++c) r[c] = (t[c] * w1 + o[db][4 * a + c] * wc) * inv;
      *ptr = r;
    }
  if (lg == 0) p.lse[row] = (M + fast_log2(denom)) * kLn2;
}

}  // namespace

hipError_t launch_col_attention(const __bf16* q, const __bf16* k, const __bf16* v, const int32_t* count,
                                const int32_t* idx, const int32_t* cols, const int32_t* col_below, float* out,
                                float* lse, int hq, int hkv, int n, float scale, hipStream_t stream) {
  ColArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.count = count;
  a.idx = idx;
  a.cols = cols;
  a.col_below = col_below;
  a.out = out;
  a.lse = lse;
  a.n = n;
  a.nblk = n / kBlock;
  a.qpg = hq / hkv;
  a.scale_log2 = scale * kLog2e;
  a.map = make_row_map(hq, hkv, a.nblk);
  hipLaunchKernelGGL(col_attn_kernel, dim3((unsigned)hq * (unsigned)a.nblk), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace crisp
