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
// One workgroup of eight waves per (head, pair of query blocks 2p, 2p+1):
// both blocks need the kept columns below 128 (2p), so every gathered
// column serves 256 query rows.  Waves 0-3 own the rows of block 2p, waves
// 4-7 those of block 2p+1, in the orientation of the tile kernel (S^T =
// K.Q^T, a lane owns a query row).  Columns stream 64 at a time through four
// LDS stages (three steps of lookahead): the K and V rows of a step are
// gathered by LDS DMA with per-lane row offsets, in the row-major swizzled
// layout the tile kernel uses.  Column indices are staged in LDS 2048 at a
// time (two halves, the next one loaded while the current one is used);
// each wave turns "before its block and not in its listed tiles" into the
// step's 64-bit slot mask with one ballot.

#include "common.h"
#include "internal.h"

namespace crisp {

namespace {

constexpr int kCStep = 64;                  // columns per step
constexpr int kCStages = 4;                 // K and V stages: three steps of lookahead
constexpr int kIdxChunk = 32 * kCStep;      // column indices per staged half
constexpr int kMaxTiles = 4096;             // key blocks per head (n <= 524288)
constexpr int kColThreads = 512;
constexpr float kColSumLimit = 65536.f;     // a lane's step sum above this raises the running max
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
  RowMap map;                // over pairs of query blocks
};

// Key slot (0..31 within a 32-key half) of accumulator register v of lane
// group lg, for the permuted K-operand rows below.
__device__ __forceinline__ int slot_of(int v, int lg) { return (v < 8) ? (8 * lg + v) : (16 + 8 * lg + (v - 8)); }

__global__ __launch_bounds__(kColThreads, 1) void col_attn_kernel(ColArgs p) {
  __shared__ __attribute__((aligned(1024))) __bf16 kst[kCStages][kCStep * kHeadDim];
  __shared__ __attribute__((aligned(1024))) __bf16 vst[kCStages][kCStep * kHeadDim];
  __shared__ __attribute__((aligned(16))) int32_t cidx[2][kIdxChunk];
  __shared__ uint32_t tbits[2][kMaxTiles / 32];

  int h, pi;
  map_row(p.map, blockIdx.x, &h, &pi);
  const int N = p.nblk;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, lg = lane >> 5;
  const int blk = w >> 2, wq = w & 3;
  const int qa = 2 * pi, qb2 = 2 * pi + 1;
  const bool has_b = qb2 < N;
  const int qmine = blk ? qb2 : qa;
  const bool active = blk == 0 || has_b;
  // kept columns below each block (clamped: malformed counts only change
  // which in-range rows are read)
  const int cnt_a = min(max(p.col_below[(size_t)h * N + qa], 0), p.n);
  const int cnt_b = has_b ? min(max(p.col_below[(size_t)h * N + qb2], 0), p.n) : 0;
  const int cnt = max(cnt_a, cnt_b);
  if (cnt == 0) return;
  const int cnt_mine = blk ? cnt_b : cnt_a;
  const int g = h / p.qpg;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int32_t* colh = p.cols + (size_t)h * p.n;
  const int limit = (has_b ? qb2 : qa) * kBlock - 1;  // gathered keys stay below the pair's last block

  // listed tiles of both blocks as bitmaps
  for (int i = tid; i < 2 * (kMaxTiles / 32); i += kColThreads) (&tbits[0][0])[i] = 0;
  __syncthreads();
  for (int b = 0; b < (has_b ? 2 : 1); ++b) {
    const int qq = b ? qb2 : qa;
    const int tc = min(max(p.count[(size_t)h * N + qq], 0), qq + 1);
    const int32_t* list = p.idx + (size_t)h * ((size_t)N * (N + 1) / 2) + (size_t)qq * (qq + 1) / 2;
    for (int t = tid; t < tc; t += kColThreads) {
      const int kb = min(max(list[t], 0), qq);
      atomicOr(&tbits[b][kb >> 5], 1u << (kb & 31));
    }
  }
  // column indices of steps 0 .. 31 (entries past cnt read as 0, clamped)
  auto load_idx = [&](int chunk, int32_t (&r)[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int slot = chunk * kIdxChunk + 4 * tid + e;
      r[e] = slot < cnt ? min(max(colh[slot], 0), limit) : 0;
    }
  };
  auto store_idx = [&](int chunk, const int32_t (&r)[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) cidx[chunk & 1][4 * tid + e] = r[e];
  };
  {
    int32_t r[4];
    load_idx(0, r);
    store_idx(0, r);
  }
  __syncthreads();

  const size_t nd = (size_t)p.n * kHeadDim;
  const int qpos = qmine * kBlock + 32 * wq + l32;
  bf16x8 qf[8];
  if (active) {
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      qf[kk] = as_bf16x8(*(const u32x4*)(p.q + (size_t)h * nd + (size_t)qpos * kHeadDim + 16 * kk + 8 * lg));
  }

  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.k + (size_t)g * nd), 0, (int)(nd * 2), kBufferFlags);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.v + (size_t)g * nd), 0, (int)(nd * 2), kBufferFlags);
  // Gather of step s: wave w fills rows 8w .. 8w+7 of the stage; lane L of
  // instruction i row r = 8w + 4i + L/16, chunk position L & 15, i.e. global
  // chunk (L & 15) ^ swz(r) of the row's column.
  auto gather = [&](int s) {
    const int st = s & (kCStages - 1);
    const int32_t* ci = cidx[(s >> 5) & 1] + (s & 31) * kCStep;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = 8 * w + 4 * i + (lane >> 4);
      const int base = ci[r] * (kHeadDim * 2);
      const unsigned ka =
          (unsigned)(uintptr_t)(__attribute__((address_space(3))) void*)(kst[st] + (8 * wu + 4 * i) * kHeadDim);
      const unsigned va =
          (unsigned)(uintptr_t)(__attribute__((address_space(3))) void*)(vst[st] + (8 * wu + 4 * i) * kHeadDim);
      lds_dma_16B(krs, base + (((lane & 15) ^ swz_k(r)) << 4), 0, ka);
      lds_dma_16B(vrs, base + (((lane & 15) ^ swz_v(r)) << 4), 0, va);
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
  bool started = false;  // wave-uniform: a counted step has set m_run

  const int nsteps = (cnt + kCStep - 1) / kCStep;
  const int nchunks = (cnt + kIdxChunk - 1) / kIdxChunk;
  // a step issues the gather three steps ahead
  auto issues = [&](int s) { return s + kCStages - 1 < nsteps; };
  for (int s = 0; s < kCStages - 1 && s < nsteps; ++s) gather(s);
  // step 0's rows must have landed: at most the gathers of steps 1 and 2 (4 each) outstanding
  if (nsteps >= 3)
    asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else if (nsteps == 2)
    asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  else
    wait_dma();
  __syncthreads();

  for (int s = 0; s < nsteps; ++s) {
    const int st = s & (kCStages - 1);
    if (issues(s)) gather(s + kCStages - 1);
    const bool refill = (s & 31) == 0 && (s >> 5) + 1 < nchunks;
    int32_t nxt[4];
    if (refill) load_idx((s >> 5) + 1, nxt);
    if (active) {
      // slot mask of this wave's query block
      const int slot = s * kCStep + lane;
      const int c = cidx[(s >> 5) & 1][(s & 31) * kCStep + lane];
      const bool ok = slot < cnt_mine && ((tbits[blk][c >> 12] >> ((c >> 7) & 31)) & 1u) == 0;
      const uint64_t mcur = __ballot(ok);
      if (mcur != 0ull) {  // uniform per wave
        const char* kb8 = (const char*)kst[st];
        f32x16 sc[2];
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
          for (int v = 0; v < 16; ++v) sc[kb2][v] = 0.f;
#pragma unroll
          for (int kk = 0; kk < 8; ++kk)
            sc[kb2] = mfma32(as_bf16x8(*(const u32x4*)(kb8 + k_off[kk] + kb2 * 8192)), qf[kk], sc[kb2]);
        }
        if (mcur != ~0ull) {  // a partial step: slots past the block or in a listed tile
#pragma unroll
          for (int kb2 = 0; kb2 < 2; ++kb2) {
            const uint32_t mh = (uint32_t)(mcur >> (32 * kb2));
            // register v < 8 holds slot 8lg + v, v >= 8 slot 16 + 8lg + (v - 8)
            const uint32_t bits = ((mh >> (8 * lg)) & 0xffu) | (((mh >> (16 + 8 * lg)) & 0xffu) << 8);
#pragma unroll
            for (int v = 0; v < 16; ++v)
              if (!((bits >> v) & 1u)) sc[kb2][v] = -INFINITY;
          }
        }
        // Lazy running max: set from the first counted step, raised only when
        // a step's probabilities sum past kSumLimit (any value keeps the
        // result exact; it only has to keep the exps in range).
        auto row_max = [&]() -> float {
          float mx = -INFINITY;
#pragma unroll
          for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
            for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sc[kb2][v]);
          return fmaxf(mx, __shfl_xor(mx, 32)) * p.scale_log2;
        };
        if (!started) {
          m_run = row_max();
          started = true;
        }
        bf16x8 pb[4];
        float ls = 0.f;
        auto exps = [&]() {
          ls = 0.f;
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
        };
        exps();
        if (__any(!(ls <= kColSumLimit))) {  // rare: raise the running max and redo the step
          const float m_new = fmaxf(m_run, row_max());
          const float alpha = fast_exp2(m_run - m_new);
#pragma unroll
          for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int v = 0; v < 16; ++v) o[db][v] *= alpha;
          l_run *= alpha;
          m_run = m_new;
          exps();
        }
        l_run += ls;
        __attribute__((address_space(3))) char* vb8 = (__attribute__((address_space(3))) char*)vst[st];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int db = u & 3, f = u >> 2;
          const int off = v_base[db] + (32 * (f >> 1) + 16 * (f & 1)) * 256;
          const bf16x4 lo =
              __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4c*)(vb8 + off)));
          const bf16x4 hi = __builtin_bit_cast(
              bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4c*)(vb8 + off + 4 * 256)));
          o[db] = mfma32(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), pb[f], o[db]);
        }
      }
    }
    if (refill) store_idx((s >> 5) + 1, nxt);
    // step s+1's rows must have landed; later gathers (4 per issuing step) may stay in flight
    const int ahead = (issues(s) ? 1 : 0) + (s >= 1 && issues(s - 1) ? 1 : 0);
    if (ahead == 2)
      asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else if (ahead == 1)
      asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else
      wait_dma();
    __syncthreads();
  }

  if (!active) return;
  // merge with the tile softmax of the same row
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (!(l_tot > 0.f)) return;  // no counted column for this row
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
  const int npairs = (a.nblk + 1) / 2;
  a.map = make_row_map(hq, hkv, npairs);
  hipLaunchKernelGGL(col_attn_kernel, dim3((unsigned)hq * (unsigned)npairs), dim3(kColThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace crisp
