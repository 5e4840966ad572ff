// Block selection of CRISP on gfx950.
//
// Vertical-Slash heads (ai.info summary, "Methodology in Plain English";
// ai-feeds summary, method module 2):
//   tile_sums  - one streaming pass over the proxy map: per (head, key block)
//                the mass on and below the tile diagonal (row >= column) and
//                above it (skipped when the proxy pass already produced
//                these block masses).  Proxy row r sits at position 128(N-1)+r, so key
//                128kb+c is at offset 128(N-1-kb)+(r-c): the lower triangle
//                falls in slash block N-1-kb, the upper one in N-2-kb.  The
//                vertical score of kb is the tile total.
//   vs_select  - per (head, direction): sort the block scores in LDS, floor =
//                alpha x lower median (or mean) of blocks 1..N-1, keep blocks
//                above it plus block 0, top up to k_min; or, for the
//                comparison chain, the shortest gamma-coverage prefix.
//   vs_expand  - per (head, query block): kept vertical blocks <= qb and the
//                two key blocks covered by each kept slash band, flagged per
//                key block and compacted in ascending order by one wave.
// Pooled-Estimation heads ("Key Contributions" item 2; gamma = 0.95 on PE):
//   pe_pool    - mean of each 128-row block of k (KV groups holding a PE head).
//   pe_logits  - per (head, 16 query blocks): mean of each query block of q,
//                then the pooled logits against every kb <= qb, each pooled
//                key read once for the 16 rows; a row's logits are written
//                into its own list row, which has exactly qb + 1 entries.
//   pe_select  - per (head, query block): the row's logits, softmax, radix
//                select of the shortest prefix reaching gamma, plus qb; the
//                list then overwrites the logits.

#include "common.h"
#include "internal.h"

namespace crisp {

namespace {

constexpr int kAlign = 256;

// Block masses from the proxy map: per (head, key block), the mass in each
// of the tile's slash bands and on the last 128 keys.  Entry (row r, column
// c) of key block kb lies r - c + t - 128 offsets into band N-1-kb (t: the
// positions of the last block): band N-1-kb when that is >= 0, N-2-kb when
// >= -128, else N-3-kb.  With 128 | n: on/below the diagonal, above it.
template <bool kRagged>
__global__ __launch_bounds__(256) void tile_sums_kernel(const float* amap, float* mass, int n, int nblk, int hq) {
  __shared__ float red[8];
  const int kb = blockIdx.x, h = blockIdx.y, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const float* base = amap + (size_t)h * kBlock * n + (size_t)kb * kBlock;
  const int c0 = 4 * (lane & 31), rs = lane >> 5;
  const int tl = n - kBlock * (nblk - 1);
  f32x4 x[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float* src = base + (size_t)(32 * w + 2 * i + rs) * n + c0;
    if (kRagged) {  // rows of n floats are not 16-byte aligned; no column past n
#pragma unroll
      for (int e = 0; e < 4; ++e) x[i][e] = kb * kBlock + c0 + e < n ? src[e] : 0.f;
    } else {
      x[i] = *(const f32x4*)src;
    }
  }
  float b0 = 0.f, b1 = 0.f, b2 = 0.f, rc = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = 32 * w + 2 * i + rs;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int dlt = r - (c0 + e) + tl - kBlock;
      if (dlt >= 0)
        b0 += x[i][e];
      else if (!kRagged || dlt >= -kBlock)
        b1 += x[i][e];
      else
        b2 += x[i][e];
      if (kRagged && kb == nblk - 2 && c0 + e >= tl) rc += x[i][e];
    }
  }
  b0 = block_sum_f(b0, red, tid, 256);
  b1 = block_sum_f(b1, red, tid, 256);
  if (kRagged) {
    b2 = block_sum_f(b2, red, tid, 256);
    rc = block_sum_f(rc, red, tid, 256);
  }
  if (tid == 0) {
    const size_t plane = (size_t)hq * nblk, at = (size_t)h * nblk + kb;
    mass[at] = b0;
    mass[plane + at] = b1;
    mass[2 * plane + at] = b2;
    mass[3 * plane + at] = kb == nblk - 1 ? b0 + b1 + b2 : rc;
  }
}

struct VsArgs {
  const float* mass;  // [4][Hq][N] block masses
  const int32_t* route;
  float* vscore;
  float* sscore;
  float* floor_v;
  float* floor_s;
  int32_t* vmask;
  int32_t* smask;
  int32_t* n_v;
  int32_t* n_s;
  int32_t* kept;  // [2][Hq] kept blocks per direction (read by the list expansion)
  int nblk;
  int pw2;  // power of two >= nblk
  float alpha;
  float gamma;
  int kmin;
  int nf_stat;
  int use_gamma;
};

constexpr int kVsThreads = 1024;

__global__ __launch_bounds__(kVsThreads) void vs_select_kernel(VsArgs p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int N = p.nblk, P = p.pw2;
  uint64_t* keys = (uint64_t*)smem;
  float* xl = (float*)(keys + P);
  uint8_t* mask = (uint8_t*)(xl + N);
  __shared__ float redf[20];
  __shared__ int redi[20];
  const int h = blockIdx.x, dir = blockIdx.y, tid = threadIdx.x;
  const int hq = gridDim.x;
  const float* lo = p.mass + (size_t)h * N;
  const float* up = lo + (size_t)hq * N;
  const float* up2 = up + (size_t)hq * N;
  float* xs = (dir == 0 ? p.vscore : p.sscore) + (size_t)h * N;
  for (int b = tid; b < N; b += kVsThreads) {
    float x;
    if (dir == 0)  // vertical: the block's mass in all its bands
      x = (lo[b] + up[b] + up2[b]) * (1.f / kBlock);
    else  // slash band b: from key blocks N-1-b, N-2-b, N-3-b
      x = (lo[N - 1 - b] + (b <= N - 2 ? up[N - 2 - b] : 0.f) + (b <= N - 3 ? up2[N - 3 - b] : 0.f)) *
          (1.f / kBlock);
    xl[b] = x;
    xs[b] = x;
    mask[b] = 0;
  }
  int32_t* mask_out = (dir == 0 ? p.vmask : p.smask) + (size_t)h * N;
  float* floor_out = dir == 0 ? p.floor_v : p.floor_s;
  int32_t* nsel_out = dir == 0 ? p.n_v : p.n_s;
  if (p.route[h] != 1) {
    for (int b = tid; b < N; b += kVsThreads) mask_out[b] = 0;
    if (tid == 0) {
      floor_out[h] = 0.f;
      nsel_out[h] = 0;
      p.kept[dir * hq + h] = 0;
    }
    return;
  }
  __syncthreads();
  const int want = min(p.kmin, N);
  if (!p.use_gamma) {
    // Noise floor over the candidates 1..N-1 (block 0 always kept).
    const int m = N - 1;
    for (int i = tid; i < P; i += kVsThreads) keys[i] = i < m ? desc_key(xl[i + 1], i + 1) : ~0ull;
    __syncthreads();
    bitonic_sort_lds(keys, P, tid, kVsThreads);
    float mu;
    if (p.nf_stat == 0) {
      const int kidx = (m - 1) / 2;          // lower median, ascending index
      mu = key_value(keys[m - 1 - kidx]);    // same value in descending order
    } else {
      float s = 0.f;
      for (int b = 1 + tid; b < N; b += kVsThreads) s += xl[b];
      mu = block_sum_f(s, redf, tid, kVsThreads) / (float)m;
    }
    const float T = p.alpha * mu;
    int above = 0;
    for (int i = tid; i < m; i += kVsThreads) above += key_value(keys[i]) > T ? 1 : 0;
    above = block_sum_i(above, redi, tid, kVsThreads);
    const int take = max(above, want - 1);
    for (int i = tid; i < take; i += kVsThreads) mask[key_index(keys[i])] = 1;
    if (tid == 0) {
      mask[0] = 1;
      floor_out[h] = T;
      nsel_out[h] = take + 1;
      p.kept[dir * hq + h] = take + 1;
    }
  } else {
    // gamma-cumulative coverage over all N blocks, then block 0 and k_min.
    for (int i = tid; i < P; i += kVsThreads) keys[i] = i < N ? desc_key(xl[i], i) : ~0ull;
    __syncthreads();
    bitonic_sort_lds(keys, P, tid, kVsThreads);
    const int per = (N + kVsThreads - 1) / kVsThreads;
    const int beg = min(N, tid * per), end = min(N, beg + per);
    float local = 0.f;
    for (int i = beg; i < end; ++i) local += key_value(keys[i]);
    float run = block_exclusive_scan_f(local, redf, tid, kVsThreads);
    int cut = 0x7fffffff;
    for (int i = beg; i < end; ++i) {
      run += key_value(keys[i]);
      if (run >= p.gamma) {
        cut = i;
        break;
      }
    }
    cut = block_min_i(cut, redi, tid, kVsThreads);
    if (cut == 0x7fffffff) cut = N - 1;
    for (int i = tid; i <= cut; i += kVsThreads) mask[key_index(keys[i])] = 1;
    __syncthreads();
    if (tid == 0) {
      int cnt = cut + 1;
      if (!mask[0]) {
        mask[0] = 1;
        ++cnt;
      }
      for (int pos = cut + 1; cnt < want && pos < N; ++pos) {
        const uint32_t b = key_index(keys[pos]);
        if (!mask[b]) {
          mask[b] = 1;
          ++cnt;
        }
      }
      floor_out[h] = key_value(keys[cut]);
      nsel_out[h] = cnt;
      p.kept[dir * hq + h] = cnt;
    }
  }
  __syncthreads();
  for (int b = tid; b < N; b += kVsThreads) mask_out[b] = mask[b];
}

// Mean of the 128 rows of a block, summed in a fixed order: 8 consecutive
// rows per thread (16 row groups), then the 16 group sums in order.  The
// query blocks pooled inside pe_logits_kernel follow the same order.  The
// mean is kept as bf16 hi + lo (the rounding of the fp32 mean and of its
// remainder).
__global__ __launch_bounds__(256) void pe_pool_kernel(const __bf16* k, const int32_t* route, float* kbar, int qpg,
                                                      int n) {
  __shared__ float part[16][kHeadDim];
  const int kb = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
  const int nblk = nblocks(n);
  const int rows = min(kBlock, n - kb * kBlock);  // fewer in a partial last block
  // pooled keys are only read by the Pooled-Estimation heads of the group
  bool any_pe = false;
  for (int t = 0; t < qpg; ++t) any_pe |= route[g * qpg + t] == 0;
  if (!any_pe) return;
  const __bf16* src = k + (size_t)g * n * kHeadDim;
  float* dst = kbar + (size_t)g * nblk * kHeadDim;
  const int dc = tid & 15, rg = tid >> 4;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  u32x4 x[8];
#pragma unroll
  for (int rr = 0; rr < 8; ++rr) {
    const u32x4 zero = {0u, 0u, 0u, 0u};
    x[rr] = rg * 8 + rr < rows ? *(const u32x4*)(src + (size_t)(kb * kBlock + rg * 8 + rr) * kHeadDim + 8 * dc) : zero;
  }
#pragma unroll
  for (int rr = 0; rr < 8; ++rr)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[2 * j] += bf16lo_to_f(x[rr][j]);
      acc[2 * j + 1] += bf16hi_to_f(x[rr][j]);
    }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[rg][8 * dc + e] = acc[e];
  __syncthreads();
  if (tid < kHeadDim) {
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) s += part[r][tid];
    // stored as a bf16 pair, hi + lo (16 significant bits), the operands of
    // the logit products: the block's 256-element row holds hi[128], lo[128]
    const float m = s / (float)rows;
    const __bf16 hi = (__bf16)m;
    __bf16* row = (__bf16*)dst + (size_t)kb * 2 * kHeadDim;
    row[tid] = hi;
    row[kHeadDim + tid] = (__bf16)(m - (float)hi);
  }
}

constexpr int kPeTile = 64;  // query blocks per pe_logits workgroup

struct PeLogitArgs {
  const __bf16* q;
  const float* kbar;
  const int32_t* route;
  int32_t* idx;
  int hq;
  int qpg;
  int n;
  int nblk;
  float scale_log2;
};

// One workgroup per (head, 64 consecutive query blocks) of a PE head,
// heaviest (last) tiles first.  The 64 pooled query rows go to LDS.  The
// pooled keys then stream through LDS 32 key blocks at a time (double
// buffered, each read from L2 once per workgroup), and wave w computes the
// logits of query rows 16w .. 16w+15 against them with bf16 matrix products
// on split operands: with x = hi(x) + lo(x) (each bf16), the dot product is
// taken as lo(q).hi(k) + hi(q).lo(k) + hi(q).hi(k), accumulated in fp32 by
// v_mfma_f32_16x16x32_bf16 over the 128 dimensions (the dropped lo.lo term
// and the split leave a relative error near 2^-16 of sum |q_d k_d|).  Lane l
// supplies dimensions 32c + 8 (l / 16) .. +7 of query row 16w + l % 16 (A)
// and of key block kb0 + l % 16 (B) for chunk c, and receives the logits of
// rows 16w + 4 (l / 16) .. +3 against key block kb0 + l % 16.  The logit of
// (qb, kb), in base 2, is stored as float bits at entry kb of qb's list row.
__global__ __launch_bounds__(256) void pe_logits_kernel(PeLogitArgs p) {
  constexpr int kPoolBatch = 4;  // query blocks pooled per round, their loads issued together
  constexpr int kKeyTile = 32;  // key blocks per LDS tile of pooled keys
  // the pooling partials and, once the queries are pooled, the key tiles
  // (double buffered) share one buffer: two workgroups fit a CU
  // Rows of the pooled queries and of the key tiles are padded by 16 bytes:
  // the products read 16 rows at one column offset, which with 512-byte rows
  // all fall in the same LDS banks.
  constexpr int kRow = kHeadDim + 4;
  __shared__ __attribute__((aligned(16))) float shared_u[2 * kKeyTile * kRow];
  __shared__ __attribute__((aligned(16))) float qs[kPeTile][kRow];
  static_assert(kPoolBatch * 16 <= 2 * kKeyTile, "pooling partials fit the key-tile buffer");
  auto& part = *(float (*)[kPoolBatch][16][kHeadDim])shared_u;
  auto& kt = *(float (*)[2][kKeyTile][kRow])shared_u;
  const int N = p.nblk, tiles = (N + kPeTile - 1) / kPeTile;
  const int h = blockIdx.x % p.hq, tile = tiles - 1 - (int)blockIdx.x / p.hq;
  if (p.route[h] != 0) return;
  const int qb0 = tile * kPeTile, nt = min(kPeTile, N - qb0), qbmax = qb0 + nt - 1;
  const int tid = threadIdx.x, dc = tid & 15, rg = tid >> 4;
  const __bf16* qh = p.q + (size_t)h * p.n * kHeadDim;
  // Pooled query rows in pe_pool_kernel's order; rows past the last block
  // are zeros, computed and not stored.
  for (int t0 = 0; t0 < kPeTile; t0 += kPoolBatch) {
    u32x4 x[kPoolBatch][8];
#pragma unroll
    for (int u = 0; u < kPoolBatch; ++u) {
      const int qb = qb0 + t0 + u;
      const int rows = t0 + u < nt ? min(kBlock, p.n - qb * kBlock) : 0;
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) {
        const u32x4 zero = {0u, 0u, 0u, 0u};
        x[u][rr] = rg * 8 + rr < rows
                       ? *(const u32x4*)(qh + (size_t)(qb * kBlock + rg * 8 + rr) * kHeadDim + 8 * dc)
                       : zero;
      }
    }
#pragma unroll
    for (int u = 0; u < kPoolBatch; ++u) {
      float acc[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
      for (int rr = 0; rr < 8; ++rr)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[2 * j] += bf16lo_to_f(x[u][rr][j]);
          acc[2 * j + 1] += bf16hi_to_f(x[u][rr][j]);
        }
#pragma unroll
      for (int e = 0; e < 8; ++e) part[u][rg][8 * dc + e] = acc[e];
    }
    __syncthreads();
    if (tid < kHeadDim) {
#pragma unroll
      for (int u = 0; u < kPoolBatch; ++u) {
        const int t = t0 + u;
        const int rows = t < nt ? min(kBlock, p.n - (qb0 + t) * kBlock) : 0;
        float s = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) s += part[u][r][tid];
        qs[t][tid] = rows > 0 ? s / (float)rows : 0.f;
      }
    }
    __syncthreads();
  }
  const float* kbase = p.kbar + (size_t)(h / p.qpg) * N * kHeadDim;
  int32_t* idx_h = p.idx + (size_t)h * ((size_t)N * (N + 1) / 2);
  const int lane = tid & 63, w = tid >> 6, li = lane & 15, kq = lane >> 4;
  bf16x8 ahi[4], alo[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float x = qs[16 * w + li][32 * c + 8 * kq + j];
      const __bf16 hi = (__bf16)x;
      ahi[c][j] = hi;
      alo[c][j] = (__bf16)(x - (float)hi);
    }
  // A key tile is 32 rows of 512 bytes: thread t loads 16-byte pieces
  // t + 256 e (e < 4); rows past the causal range read a valid row, results
  // unused.  Tiles are loaded two ahead into registers (two sets in turn) and
  // written to LDS one ahead, so a load has a whole tile's products to land.
  auto load_tile = [&](int kb0, f32x4 (&r)[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int piece = tid + 256 * e, row = piece >> 5;
      r[e] = *(const f32x4*)(kbase + (size_t)min(kb0 + row, qbmax) * kHeadDim + 4 * (piece & 31));
    }
  };
  auto store_tile = [&](int buf, const f32x4 (&r)[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int piece = tid + 256 * e;
      *(f32x4*)&kt[buf][piece >> 5][4 * (piece & 31)] = r[e];
    }
  };
  const int wq0 = qb0 + 16 * w;  // this wave's first query row
  auto products = [&](int kb0, int buf) {
#pragma unroll
    for (int sub = 0; sub < kKeyTile / 16; ++sub) {
      const int kbs = kb0 + 16 * sub;
      if (kbs <= qbmax && kbs <= wq0 + 15 && 16 * w < nt) {  // the wave has rows at or past these blocks
        const __bf16* krow = (const __bf16*)&kt[buf][16 * sub + li][0];  // hi[128], lo[128]
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const bf16x8 bhi = *(const bf16x8*)(krow + 32 * c + 8 * kq);
          const bf16x8 blo = *(const bf16x8*)(krow + kHeadDim + 32 * c + 8 * kq);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo[c], bhi, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi[c], blo, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi[c], bhi, acc, 0, 0, 0);
        }
        const int kb = kbs + li;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int t = 16 * w + 4 * kq + rr, qb = qb0 + t;
          if (t < nt && kb <= qb) ((float*)idx_h)[(size_t)qb * (qb + 1) / 2 + kb] = acc[rr] * p.scale_log2;
        }
      }
    }
  };
  const int ntile = qbmax / kKeyTile + 1;
  f32x4 r0[4], r1[4];
  load_tile(0, r0);
  if (ntile > 1) load_tile(kKeyTile, r1);
  store_tile(0, r0);
  __syncthreads();
  for (int i = 0; i < ntile; i += 2) {
    // tile i in buffer 0, tile i+1 in r1
    if (i + 2 < ntile) load_tile((i + 2) * kKeyTile, r0);
    products(i * kKeyTile, 0);
    if (i + 1 < ntile) store_tile(1, r1);
    __syncthreads();
    if (i + 1 >= ntile) break;
    // tile i+1 in buffer 1, tile i+2 in r0
    if (i + 3 < ntile) load_tile((i + 3) * kKeyTile, r1);
    products((i + 1) * kKeyTile, 1);
    if (i + 2 < ntile) store_tile(0, r0);
    __syncthreads();
  }
}

struct PeArgs {
  const int32_t* route;
  int32_t* count;
  int32_t* idx;
  int hq;
  int nblk;
  float gamma;
};

constexpr int kPeThreads = 256;
constexpr int kMaxBlocks = 4096;  // n <= 524288
constexpr float kFixOne = 2147483648.0f;  // 2^31: probabilities as 32-bit fixed point (a row sums to <= 2^31)

// Wave 0 of a workgroup: the smallest digit d with
// below + sum(hist[0..d]) >= target, and the mass below it; d = 256 if none.
__device__ inline void find_digit(const uint32_t* hist, uint32_t below, uint32_t target, int lane, int* d_out,
                                  uint32_t* below_out) {
  uint32_t s[4], tot = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    s[b] = hist[4 * lane + b];
    tot += s[b];
  }
  uint32_t incl = tot;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  uint32_t run = below + incl - tot;
  int cand = 256;
  uint32_t cand_below = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    if (cand == 256 && run + s[b] >= target) {
      cand = 4 * lane + b;
      cand_below = run;
    }
    run += s[b];
  }
  int best = cand;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) best = min(best, __shfl_xor(best, o));
  if (cand == best && cand < 256) {
    *d_out = cand;
    *below_out = cand_below;
  }
  if (lane == 0 && best == 256) *d_out = 256;
}

// The gamma cut's histogram bins hold (mass << 16) | count: masses are
// 2^-31 fixed point and a row's total is at most 2^31, counts at most 4096,
// so neither part overflows into the other.
constexpr int kCountBits = 16;

// Lane exchanges through ds_bpermute from a lane index l the caller takes
// from opaque_lane() once per use site: the compiler would otherwise hoist
// one address per offset out of the radix-pass loop and keep them all live
// across it.
__device__ __forceinline__ uint32_t lane_xor_u32(uint32_t x, int l, int o) {
  return (uint32_t)__builtin_amdgcn_ds_bpermute((l ^ o) << 2, (int)x);
}
__device__ __forceinline__ uint32_t lane_up_u32(uint32_t x, int l, int o) {  // lanes below o keep x
  return (uint32_t)__builtin_amdgcn_ds_bpermute((l >= o ? l - o : l) << 2, (int)x);
}

// find_digit over the mass parts of packed bins, also returning the number
// of keys in the chosen bin.
__device__ inline void find_digit_packed(const uint64_t* hist, uint32_t below, uint32_t target, int lane, int* d_out,
                                         uint32_t* below_out, uint32_t* count_out) {
  uint32_t s[4], c[4], tot = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const uint64_t v = hist[4 * lane + b];
    s[b] = (uint32_t)(v >> kCountBits);
    c[b] = (uint32_t)(v & ((1u << kCountBits) - 1));
    tot += s[b];
  }
  const int l = opaque_lane();
  uint32_t incl = tot;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = lane_up_u32(incl, l, o);
    if (lane >= o) incl += y;
  }
  uint32_t run = below + incl - tot;
  int cand = 256;
  uint32_t cand_below = 0, cand_count = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    if (cand == 256 && run + s[b] >= target) {
      cand = 4 * lane + b;
      cand_below = run;
      cand_count = c[b];
    }
    run += s[b];
  }
  int best = cand;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) best = min(best, (int)lane_xor_u32((uint32_t)best, l, o));
  if (cand == best && cand < 256) {
    *d_out = cand;
    *below_out = cand_below;
    *count_out = cand_count;
  }
  if (lane == 0 && best == 256) *d_out = 256;
}

// Adds `val` to bin `digit` for the valid lanes of a wave (all lanes must be
// active).  The lanes sharing the first valid lane's digit are summed in
// registers and added with one atomic: a row's probabilities are alike, so
// most lanes fall in one bin of the high digits.  Integer sums, so the bins
// do not depend on the grouping.
__device__ __forceinline__ void hist_add_packed(uint64_t* hist, bool valid, uint32_t digit, uint64_t val, int lane) {
  const uint64_t any = __ballot(valid);
  if (any == 0) return;  // no valid lane in the wave (a uniform branch)
  const uint32_t lead = __builtin_amdgcn_readlane(digit, (int)__builtin_ctzll(any));
  const bool same = valid && digit == lead;
  uint64_t sum = same ? val : 0ull;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o);
  if (lane == (int)__builtin_ctzll(__ballot(same))) atomicAdd((unsigned long long*)&hist[lead], sum);
  if (valid && !same) atomicAdd((unsigned long long*)&hist[digit], val);
}

// One workgroup per (head, query block) of a Pooled-Estimation head.
// The kept set is the shortest prefix, in (descending probability, ascending
// block) order, whose mass reaches gamma.  That order is the ascending order
// of desc_key(p, kb), so the cut is the smallest key K whose cumulative mass
// over keys <= K reaches gamma.  K is found digit by digit from the top
// (radix select): per 8-bit digit a 256-bin histogram of the mass of the
// keys that match the digits fixed so far, then the digit where the running
// mass crosses gamma.  Keys hold the probability's bits above the block index
// (< 4096, so key bits 16..31 are zero): 6 passes cover them.  Masses are
// 2^-31 fixed point (truncated; at most 4096 x 2^-31 below the real sum), so
// sums are exact integers and the result deterministic.
// Five workgroups per CU (at most 102 registers): the kernel waits on memory
// and barriers most of its time, and occupancy is what hides that.
__global__ __launch_bounds__(kPeThreads, 5) void pe_select_kernel(PeArgs p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ float red_max[4], red_sum[4];
  __shared__ int redi[8];
  __shared__ uint64_t hist2[2][256];
  __shared__ int sel_digit;
  __shared__ uint32_t sel_below, sel_count;
  __shared__ uint64_t sel_key;
  const int N = p.nblk;
  const int id = blockIdx.x;
  const int h = id % p.hq, qb = N - 1 - id / p.hq;
  if (p.route[h] != 0) return;
  const int L = qb + 1;
  float* pr = (float*)smem;
  uint8_t* flags = (uint8_t*)(pr + N);
  const int tid = threadIdx.x, lane = tid & 63;

  // the row's pooled logits (base 2), left in its list row by pe_logits_kernel
  int32_t* row = p.idx + (size_t)h * ((size_t)N * (N + 1) / 2) + (size_t)qb * (qb + 1) / 2;
  for (int kb = tid; kb < L; kb += kPeThreads) pr[kb] = __int_as_float(row[kb]);
  __syncthreads();
  float mx = -INFINITY;
  for (int kb = tid; kb < L; kb += kPeThreads) mx = fmaxf(mx, pr[kb]);
  mx = block_max_f1(mx, red_max, tid, kPeThreads);
  float loc = 0.f;
  for (int kb = tid; kb < L; kb += kPeThreads) {
    const float e = fast_exp2(pr[kb] - mx);
    pr[kb] = e;
    loc += e;
  }
  const float sum = block_sum_f1(loc, red_sum, tid, kPeThreads);
  // Thread t holds entries t + 256 u (u < U <= 16) of the row in registers
  // for the radix passes: the high word of its key (the complemented
  // probability bits) and its fixed-point mass.
  const int U = (L + kPeThreads - 1) / kPeThreads;
  uint32_t khi[kMaxBlocks / kPeThreads], mass[kMaxBlocks / kPeThreads];
#pragma unroll
  for (int u = 0; u < kMaxBlocks / kPeThreads; ++u) {
    const int i = tid + kPeThreads * u;
    khi[u] = 0xffffffffu;
    mass[u] = 0;
    if (u < U && i < L) {
      const float pv = pr[i] / sum;
      pr[i] = pv;
      khi[u] = ~__float_as_uint(pv);
      mass[u] = (uint32_t)(pv * kFixOne);
    }
  }
  hist2[0][tid] = 0;
  hist2[1][tid] = 0;
  __syncthreads();

  const uint32_t target = (uint32_t)(p.gamma * kFixOne);
  constexpr int kShift[6] = {56, 48, 40, 32, 8, 0};
  uint64_t decided = 0;
  uint32_t below = 0;
  bool keep_all = false;
#pragma unroll 1
  for (int pass = 0; pass < 6; ++pass) {
    const int sh = kShift[pass];
    const uint64_t hi_mask = pass == 0 ? 0ull : ~((uint64_t(1) << (sh + 8)) - 1);
    // two histograms in turn: this pass's starts cleared, and the other one
    // (last read before the previous pass's final barrier) is cleared for
    // the next pass
    uint64_t* hist = hist2[pass & 1];
    if (pass > 0) hist2[(pass + 1) & 1][tid] = 0;
    // a thread's matching entries, run by run of equal digits: a run goes
    // to the histogram when the digit changes, the last one with the wave
    uint32_t run_d = 0xffffffffu;
    uint64_t run_v = 0;
#pragma unroll
    for (int u = 0; u < kMaxBlocks / kPeThreads; ++u) {
      const int i = tid + kPeThreads * u;
      if (u < U && i < L) {
        const uint64_t key = ((uint64_t)khi[u] << 32) | (uint32_t)i;
        if ((key & hi_mask) == decided) {
          const uint32_t dg = (uint32_t)(key >> sh) & 255u;
          const uint64_t v = ((uint64_t)mass[u] << kCountBits) | 1ull;
          if (dg == run_d) {
            run_v += v;
          } else {
            if (run_d != 0xffffffffu) atomicAdd((unsigned long long*)&hist[run_d], run_v);
            run_d = dg;
            run_v = v;
          }
        }
      }
    }
    hist_add_packed(hist, run_d != 0xffffffffu, run_d, run_v, lane);
    __syncthreads();
    if (tid < 64) find_digit_packed(hist, below, target, lane, &sel_digit, &sel_below, &sel_count);
    __syncthreads();
    const int d = sel_digit;
    if (d == 256) {  // the whole row never reaches gamma (rounding): keep everything
      keep_all = true;
      break;
    }
    below = sel_below;
    decided |= (uint64_t)d << sh;
    if (sel_count == 1) {
      // one key carries the digits fixed so far: it is the cut, whatever
      // its remaining digits (the passes left would single it out)
      const uint64_t m = ~((uint64_t(1) << sh) - 1);
#pragma unroll
      for (int u = 0; u < kMaxBlocks / kPeThreads; ++u) {
        const int i = tid + kPeThreads * u;
        const uint64_t key = ((uint64_t)khi[u] << 32) | (uint32_t)i;
        if (u < U && i < L && (key & m) == decided) sel_key = key;
      }
      __syncthreads();
      decided = sel_key;
      break;
    }
  }

  // ascending compaction of the kept blocks plus the diagonal one
  const int per = (L + kPeThreads - 1) / kPeThreads;
  const int beg = min(L, tid * per), end = min(L, beg + per);
  int c = 0;
  for (int kb = beg; kb < end; ++kb) {
    const bool f = keep_all || kb == qb || desc_key(pr[kb], (uint32_t)kb) <= decided;
    flags[kb] = f;
    c += f;
  }
  int total;
  int pos = block_exclusive_scan(c, redi, tid, kPeThreads, &total);
  for (int kb = beg; kb < end; ++kb)
    if (flags[kb]) row[pos++] = kb;
  if (tid == 0) p.count[(size_t)h * N + qb] = total;
}

// The lists of a Vertical-Slash head are written by one of two kernels,
// chosen per head from its kept counts (both kernels decide alike): a
// thread-per-row merge when |V| + 2|S| <= N / 16 (its cost grows with the
// kept blocks), otherwise a wave per row that walks the row's key blocks
// and writes whole runs of the list at once (its cost grows with qb).
__device__ __forceinline__ bool expand_is_sparse(int nv, int ns, int N) { return 16 * (nv + 2 * ns) <= N; }

// Sparse heads: one workgroup per (head, 256 query blocks), one thread per
// query block.  The head's kept vertical blocks V and slash bands S are
// compacted once into ascending LDS lists; the list of qb is the merge of
// {v in V : v <= qb} with the tiles qb - s - 1, qb - s of the bands s in S
// taken from the widest band down (an ascending sequence in which
// neighbouring bands repeat one block), dropping repeats and blocks below 0.
// A thread's work grows with |V| + 2|S|, not with qb.
constexpr int kExpandRows = 256;

__global__ __launch_bounds__(256) void vs_expand_sparse_kernel(const int32_t* route, const int32_t* kept,
                                                               const int32_t* vmask, const int32_t* smask,
                                                               int32_t* count, int32_t* idx, int nblk) {
  __shared__ int32_t vl[kMaxBlocks], sl[kMaxBlocks];
  __shared__ int scan_tmp[8];
  const int N = nblk, h = blockIdx.y, tid = threadIdx.x;
  if (route[h] != 1 || !expand_is_sparse(kept[h], kept[gridDim.y + h], N)) return;
  // ascending compaction of both masks, 256 blocks per round
  int nv = 0, ns = 0;
  for (int b0 = 0; b0 < N; b0 += 256) {
    const int b = b0 + tid;
    const int fv = (b < N && vmask[(size_t)h * N + b] != 0) ? 1 : 0;
    const int fs = (b < N && smask[(size_t)h * N + b] != 0) ? 1 : 0;
    int tv, ts;
    const int pv = block_exclusive_scan(fv, scan_tmp, tid, 256, &tv);
    const int ps = block_exclusive_scan(fs, scan_tmp, tid, 256, &ts);
    if (fv) vl[nv + pv] = b;
    if (fs) sl[ns + ps] = b;
    nv += tv;
    ns += ts;
  }
  __syncthreads();
  const int qb = blockIdx.x * kExpandRows + tid;
  if (qb >= N) return;
  int32_t* out = idx + (size_t)h * ((size_t)N * (N + 1) / 2) + (size_t)qb * (qb + 1) / 2;
  constexpr int kNone = 0x7fffffff;
  int a = 0;           // next vertical block
  int bi = ns - 1;     // next band, widest first
  int ph = 0;          // 0: block qb - s - 1, 1: block qb - s
  auto next_b = [&]() -> int {  // next slash tile >= 0, or kNone
    while (bi >= 0) {
      const int e = qb - sl[bi] - 1 + ph;
      if (ph == 1) {
        ph = 0;
        --bi;
      } else {
        ph = 1;
      }
      if (e >= 0) return e;
    }
    return kNone;
  };
  int va = (a < nv && vl[a] <= qb) ? vl[a] : kNone;
  int vb = next_b();
  int last = -1, pos = 0;
  while (va != kNone || vb != kNone) {
    int e;
    if (va <= vb) {
      e = va;
      ++a;
      va = (a < nv && vl[a] <= qb) ? vl[a] : kNone;
    } else {
      e = vb;
      vb = next_b();
    }
    if (e != last) {
      out[pos++] = e;
      last = e;
    }
  }
  count[(size_t)h * N + qb] = pos;
}


// Dense heads: one wave per (head, query block), eight per workgroup.  Key block kb is in
// the list of qb when vertical block kb is kept, or a kept slash band covers
// it: band qb - kb (its tile qb - s) or band qb - kb - 1 (its tile
// qb - s - 1).  The wave walks kb = 0 .. qb 64 at a time, flags each block
// and writes the flagged ones at their rank (ballot and popcount), so the
// list is ascending and every store instruction writes consecutive entries.
constexpr int kExpandWaves = 8;

__global__ __launch_bounds__(64 * kExpandWaves) void vs_expand_dense_kernel(const int32_t* route,
                                                                            const int32_t* kept,
                                                                            const int32_t* vmask,
                                                                            const int32_t* smask, int32_t* count,
                                                                            int32_t* idx, int nblk) {
  __shared__ uint8_t vm[kMaxBlocks], sm[kMaxBlocks];
  const int N = nblk, h = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
  if (route[h] != 1 || expand_is_sparse(kept[h], kept[gridDim.y + h], N)) return;
  for (int b = tid; b < N; b += 64 * kExpandWaves) {
    vm[b] = vmask[(size_t)h * N + b] != 0;
    sm[b] = smask[(size_t)h * N + b] != 0;
  }
  __syncthreads();
  const int qb = blockIdx.x * kExpandWaves + (tid >> 6);
  if (qb >= N) return;
  int32_t* out = idx + (size_t)h * ((size_t)N * (N + 1) / 2) + (size_t)qb * (qb + 1) / 2;
  int pos = 0;
  for (int c0 = 0; c0 <= qb; c0 += 64) {
    const int kb = c0 + lane;
    bool f = false;
    if (kb <= qb) {
      const int s = qb - kb;
      f = vm[kb] || sm[s] || (s >= 1 && sm[s - 1]);
    }
    const uint64_t bal = __ballot(f);
    if (f) out[pos + __popcll(bal & ((1ull << lane) - 1))] = kb;
    pos += __popcll(bal);
  }
  if (lane == 0) count[(size_t)h * N + qb] = pos;
}

// ---------------------------------------------------------------------------
// Token-granular vertical selection (ai-feeds summary, method module 2: keep
// the tokens clearly above the noise floor).  One workgroup per VS head over
// its column masses c[j]: columns 0..127 are always kept (the sink tile);
// the floor is alpha x the lower median (or the mean) of columns 128..n-1;
// columns above it are kept, topped up to k_min tokens in all by the best
// remaining ones (descending mass, ties to the lower index).  The median and
// the top-up cut are exact radix selects over the masses' bit patterns
// (non-negative floats order like their bits).  Output: the kept columns past
// the sink tile in ascending order, their count, and per query block qb the
// number of them below 128 qb; v_mask becomes block 0 only (the sink tile).
// ---------------------------------------------------------------------------

constexpr int kTokThreads = 1024;
constexpr int kTokPer = 8;  // consecutive columns per thread in the in-order passes

struct TokArgs {
  const float* colmass;
  const int32_t* route;
  int32_t* cols;       // [Hq][n]
  int32_t* ncols;      // [Hq]
  int32_t* col_below;  // [Hq][N]
  int32_t* vmask;      // [Hq][N]
  float* floor_v;      // [Hq]
  int32_t* n_v;        // [Hq]
  int32_t* kept;       // [2][Hq] kept blocks per direction: vertical becomes block 0 only
  int n;
  int nblk;
  float alpha;
  int kmin_tokens;
  int nf_stat;
};

// Histogram of 8-bit digits with one LDS atomic per run of equal digits led
// by the wave's first active lane (column masses share their high bits).
__device__ __forceinline__ void hist_add(uint32_t* hist, bool valid, uint32_t digit, int lane) {
  const uint32_t mine = valid ? digit : 0xffffffffu;
  const uint32_t lead = __builtin_amdgcn_readfirstlane(mine);
  const bool same = mine == lead;
  const uint64_t bal = __ballot(same);
  if (same) {
    if (lead != 0xffffffffu && lane == (int)__builtin_ctzll(bal)) atomicAdd(&hist[lead], (uint32_t)__popcll(bal));
  } else if (valid) {
    atomicAdd(&hist[digit], 1u);
  }
}

// The bit pattern of rank k (0-based, ascending) among the candidate columns
// j in [kBlock, n) with (only_le ? bits <= le_bits : true).
__device__ uint32_t tok_radix_kth(const float* x, int n, bool only_le, uint32_t le_bits, uint32_t k, uint32_t* hist,
                                  int* sel_digit, uint32_t* sel_below, int tid) {
  const int lane = tid & 63;
  uint32_t prefix = 0, pmask = 0, below = 0;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += kTokThreads) hist[i] = 0;
    __syncthreads();
    for (int j0 = kBlock; j0 < n; j0 += kTokThreads * kTokPer) {
      uint32_t u[kTokPer];
#pragma unroll
      for (int e = 0; e < kTokPer; ++e) {  // all loads first: kTokPer in flight
        const int j = j0 + e * kTokThreads + tid;
        u[e] = j < n ? __float_as_uint(x[j]) : 0xffffffffu;
      }
#pragma unroll
      for (int e = 0; e < kTokPer; ++e) {
        const bool v = u[e] != 0xffffffffu && (u[e] & pmask) == prefix && (!only_le || u[e] <= le_bits);
        hist_add(hist, v, (u[e] >> shift) & 255u, lane);
      }
    }
    __syncthreads();
    if (tid < 64) find_digit(hist, below, k + 1, lane, sel_digit, sel_below);
    __syncthreads();
    const int d = *sel_digit;
    below = *sel_below;
    prefix |= (uint32_t)min(d, 255) << shift;
    pmask |= 255u << shift;
    __syncthreads();
  }
  return prefix;
}

__global__ __launch_bounds__(kTokThreads) void tok_select_kernel(TokArgs p) {
  __shared__ uint32_t hist[256];
  __shared__ int sel_digit;
  __shared__ uint32_t sel_below;
  __shared__ float redf[20];
  __shared__ int redi[20];
  const int h = blockIdx.x, tid = threadIdx.x, N = p.nblk, n = p.n;
  int32_t* below_out = p.col_below + (size_t)h * N;
  if (p.route[h] != 1) {
    for (int b = tid; b < N; b += kTokThreads) below_out[b] = 0;
    if (tid == 0) p.ncols[h] = 0;
    return;
  }
  const float* x = p.colmass + (size_t)h * n;
  const int m = n - kBlock;  // candidates
  float mu;
  if (p.nf_stat == 0) {
    mu = __uint_as_float(tok_radix_kth(x, n, false, 0u, (uint32_t)((m - 1) / 2), hist, &sel_digit, &sel_below, tid));
  } else {
    float sacc = 0.f;
    for (int j = kBlock + tid; j < n; j += kTokThreads) sacc += x[j];
    mu = block_sum_f(sacc, redf, tid, kTokThreads) / (float)m;
  }
  const float T = p.alpha * mu;
  int above = 0;
  for (int j = kBlock + tid; j < n; j += kTokThreads) above += x[j] > T ? 1 : 0;
  above = block_sum_i(above, redi, tid, kTokThreads);
  const int need = max(0, min(p.kmin_tokens, n) - kBlock - above);
  // top-up cut: the need-th largest among the columns at or below the floor
  uint32_t cut = 0xffffffffu;
  int ties = 0;
  if (need > 0) {
    const uint32_t tbits = __float_as_uint(T);
    const int le = m - above;
    cut = tok_radix_kth(x, n, true, tbits, (uint32_t)(le - need), hist, &sel_digit, &sel_below, tid);
    int gt = 0;
    for (int j = kBlock + tid; j < n; j += kTokThreads) {
      const float xv = x[j];
      gt += (!(xv > T) && __float_as_uint(xv) > cut) ? 1 : 0;
    }
    gt = block_sum_i(gt, redi, tid, kTokThreads);
    ties = need - gt;  // columns equal to the cut value taken, lowest index first
  }
  // in-order compaction, kTokPer consecutive columns per thread
  int kept_before = 0, ties_before = 0;
  for (int c0 = kBlock; c0 < n; c0 += kTokThreads * kTokPer) {
    const int jb = c0 + kTokPer * tid;
    uint32_t tie_bits = 0;
    int nt = 0;
#pragma unroll
    for (int e = 0; e < kTokPer; ++e) {
      const int j = jb + e;
      if (j < n) {
        const float xv = x[j];
        if (need > 0 && !(xv > T) && __float_as_uint(xv) == cut) {
          tie_bits |= 1u << e;
          ++nt;
        }
      }
    }
    int tie_tot;
    const int tie_excl = ties_before + block_exclusive_scan(nt, redi, tid, kTokThreads, &tie_tot);
    ties_before += tie_tot;
    uint32_t keep_bits = 0;
    int nk = 0, tr = tie_excl;
#pragma unroll
    for (int e = 0; e < kTokPer; ++e) {
      const int j = jb + e;
      if (j < n) {
        const float xv = x[j];
        bool keep = xv > T;
        if (!keep && need > 0) {
          const uint32_t u = __float_as_uint(xv);
          if (u > cut) keep = true;
          if (tie_bits & (1u << e)) keep = tr++ < ties;
        }
        if (keep) {
          keep_bits |= 1u << e;
          ++nk;
        }
      }
    }
    int kept_tot;
    int pos = kept_before + block_exclusive_scan(nk, redi, tid, kTokThreads, &kept_tot);
    int32_t* out = p.cols + (size_t)h * n;
#pragma unroll
    for (int e = 0; e < kTokPer; ++e) {
      const int j = jb + e;
      if (j < n && (j & (kBlock - 1)) == 0) below_out[j >> 7] = pos;  // kept columns below 128 qb
      if (keep_bits & (1u << e)) out[pos++] = j;
    }
    kept_before += kept_tot;
  }
  for (int b = tid; b < N; b += kTokThreads) p.vmask[(size_t)h * N + b] = b == 0 ? 1 : 0;
  if (tid == 0) {
    below_out[0] = 0;
    p.ncols[h] = kept_before;
    p.floor_v[h] = T;
    p.n_v[h] = kBlock + kept_before;
    p.kept[h] = 1;
  }
}

inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

inline int host_pow2_ceil(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

}  // namespace

size_t select_workspace_bytes(int hq, int hkv, int n) {
  const size_t N = (size_t)nblocks(n);
  size_t b = 0;
  b += align_up(4 * hq * N * sizeof(float));        // block masses from the map
  b += 2 * align_up(hq * N * sizeof(float));        // vscore, sscore
  b += 2 * align_up(hq * sizeof(float));            // floors
  b += 2 * align_up(hq * N * sizeof(int32_t));      // masks
  b += 2 * align_up(hq * sizeof(int32_t));          // kept counts
  b += align_up(2 * hq * sizeof(int32_t));          // kept blocks per direction, for the list expansion
  b += align_up(hkv * N * kHeadDim * sizeof(float));// kbar
  return b;
}

SelectBuffers carve_select_workspace(void* ws, int hq, int hkv, int n) {
  const size_t N = (size_t)nblocks(n);
  char* p = (char*)ws;
  SelectBuffers b;
  auto take = [&](size_t bytes) {
    char* r = p;
    p += align_up(bytes);
    return (void*)r;
  };
  b.mass = (float*)take(4 * hq * N * sizeof(float));
  b.vscore = (float*)take(hq * N * sizeof(float));
  b.sscore = (float*)take(hq * N * sizeof(float));
  b.floor_v = (float*)take(hq * sizeof(float));
  b.floor_s = (float*)take(hq * sizeof(float));
  b.vmask = (int32_t*)take(hq * N * sizeof(int32_t));
  b.smask = (int32_t*)take(hq * N * sizeof(int32_t));
  b.n_v = (int32_t*)take(hq * sizeof(int32_t));
  b.n_s = (int32_t*)take(hq * sizeof(int32_t));
  b.kept = (int32_t*)take(2 * hq * sizeof(int32_t));
  b.kbar = (float*)take(hkv * N * kHeadDim * sizeof(float));
  return b;
}

hipError_t launch_select(const __bf16* q, const __bf16* k, const float* amap, const float* mass, const int32_t* route,
                         const SelectBuffers& b, int32_t* count, int32_t* idx, int hq, int hkv, int n, float scale,
                         float alpha, float gamma_pe, int kmin, int nf_stat, bool use_gamma, float gamma,
                         const TokenCols* tok, hipStream_t stream) {
  const int N = nblocks(n);
  hipError_t e;
  if (mass == nullptr) {
    if (n % kBlock != 0)
      hipLaunchKernelGGL(tile_sums_kernel<true>, dim3(N, hq), dim3(256), 0, stream, amap, b.mass, n, N, hq);
    else
      hipLaunchKernelGGL(tile_sums_kernel<false>, dim3(N, hq), dim3(256), 0, stream, amap, b.mass, n, N, hq);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    mass = b.mass;
  }

  VsArgs va;
  va.mass = mass;
  va.route = route;
  va.vscore = b.vscore;
  va.sscore = b.sscore;
  va.floor_v = b.floor_v;
  va.floor_s = b.floor_s;
  va.vmask = b.vmask;
  va.smask = b.smask;
  va.n_v = b.n_v;
  va.n_s = b.n_s;
  va.kept = b.kept;
  va.nblk = N;
  va.pw2 = host_pow2_ceil(N);
  va.alpha = alpha;
  va.gamma = gamma;
  va.kmin = kmin;
  va.nf_stat = nf_stat;
  va.use_gamma = use_gamma ? 1 : 0;
  const size_t vs_lds = (size_t)va.pw2 * 8 + (size_t)N * 4 + (size_t)N;
  hipLaunchKernelGGL(vs_select_kernel, dim3(hq, 2), dim3(kVsThreads), vs_lds, stream, va);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (tok != nullptr) {  // token-granular vertical: replaces the vertical block selection
    TokArgs ta;
    ta.colmass = tok->colmass;
    ta.route = route;
    ta.cols = tok->cols;
    ta.ncols = tok->ncols;
    ta.col_below = tok->col_below;
    ta.vmask = b.vmask;
    ta.floor_v = b.floor_v;
    ta.n_v = b.n_v;
    ta.kept = b.kept;
    ta.n = n;
    ta.nblk = N;
    ta.alpha = alpha;
    ta.kmin_tokens = kmin * kBlock;
    ta.nf_stat = nf_stat;
    hipLaunchKernelGGL(tok_select_kernel, dim3(hq), dim3(kTokThreads), 0, stream, ta);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }

  hipLaunchKernelGGL(pe_pool_kernel, dim3(N, hkv), dim3(256), 0, stream, k, route, b.kbar, hq / hkv, n);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  PeLogitArgs la;
  la.q = q;
  la.kbar = b.kbar;
  la.route = route;
  la.idx = idx;
  la.hq = hq;
  la.qpg = hq / hkv;
  la.n = n;
  la.nblk = N;
  la.scale_log2 = scale * kLog2e;
  hipLaunchKernelGGL(pe_logits_kernel, dim3(hq * ((N + kPeTile - 1) / kPeTile)), dim3(256), 0, stream, la);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  PeArgs pa;
  pa.route = route;
  pa.count = count;
  pa.idx = idx;
  pa.hq = hq;
  pa.nblk = N;
  pa.gamma = use_gamma ? gamma : gamma_pe;
  const size_t pe_lds = (size_t)N * 4 + (size_t)N;
  hipLaunchKernelGGL(pe_select_kernel, dim3(hq * N), dim3(kPeThreads), pe_lds, stream, pa);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  hipLaunchKernelGGL(vs_expand_sparse_kernel, dim3((N + kExpandRows - 1) / kExpandRows, hq), dim3(256), 0, stream,
                     route, b.kept, b.vmask, b.smask, count, idx, N);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(vs_expand_dense_kernel, dim3((N + kExpandWaves - 1) / kExpandWaves, hq), dim3(64 * kExpandWaves),
                     0, stream, route, b.kept, b.vmask, b.smask, count, idx, N);
  return hipGetLastError();
}

}  // namespace crisp
