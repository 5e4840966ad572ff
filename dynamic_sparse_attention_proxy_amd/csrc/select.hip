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
//                two key blocks covered by each kept slash band, compacted in
//                ascending order.
// Pooled-Estimation heads ("Key Contributions" item 2; gamma = 0.95 on PE):
//   pe_pool    - mean of each 128-row block of q (PE heads) and k (KV groups
//                holding a PE head).
//   pe_select  - per (head, query block): pooled logits against kb <= qb,
//                softmax, radix select of the shortest prefix reaching
//                gamma, plus qb.

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
    }
  }
  __syncthreads();
  for (int b = tid; b < N; b += kVsThreads) mask_out[b] = mask[b];
}

__global__ __launch_bounds__(256) void pe_pool_kernel(const __bf16* q, const __bf16* k, const int32_t* route,
                                                      float* qbar, float* kbar, int hq, int qpg, int n) {
  __shared__ float part[16][kHeadDim];
  const int kb = blockIdx.x, which = blockIdx.y, tid = threadIdx.x;
  const int nblk = nblocks(n);
  const int rows = min(kBlock, n - kb * kBlock);  // fewer in a partial last block
  const __bf16* src;
  float* dst;
  if (which < hq) {
    if (route[which] != 0) return;
    src = q + (size_t)which * n * kHeadDim;
    dst = qbar + (size_t)which * nblk * kHeadDim;
  } else {
    const int g = which - hq;
    // pooled keys are only read by the Pooled-Estimation heads of the group
    bool any_pe = false;
    for (int t = 0; t < qpg; ++t) any_pe |= route[g * qpg + t] == 0;
    if (!any_pe) return;
    src = k + (size_t)g * n * kHeadDim;
    dst = kbar + (size_t)g * nblk * kHeadDim;
  }
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
    dst[(size_t)kb * kHeadDim + tid] = s / (float)rows;
  }
}

struct PeArgs {
  const float* qbar;
  const float* kbar;
  const int32_t* route;
  int32_t* count;
  int32_t* idx;
  int hq;
  int qpg;
  int nblk;
  float scale_log2;
  float gamma;
};

constexpr int kPeThreads = 256;
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
__global__ __launch_bounds__(kPeThreads) void pe_select_kernel(PeArgs p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ float redf[8];
  __shared__ int redi[8];
  __shared__ uint32_t hist[256];
  __shared__ int sel_digit;
  __shared__ uint32_t sel_below;
  const int N = p.nblk;
  const int id = blockIdx.x;
  const int h = id % p.hq, qb = N - 1 - id / p.hq;
  if (p.route[h] != 0) return;
  const int L = qb + 1;
  float* pr = (float*)smem;
  uint8_t* flags = (uint8_t*)(pr + N);
  const int tid = threadIdx.x, l16 = tid & 15, grp = tid >> 4, lane = tid & 63;
  const int g = h / p.qpg;

  // pooled logits (base 2): 16 lanes per key block, 8 dims each; four
  // groups of 16 key blocks per iteration, their loads issued together
  const float* qv = p.qbar + ((size_t)h * N + qb) * kHeadDim + 8 * l16;
  const f32x4 qa = *(const f32x4*)qv, qc = *(const f32x4*)(qv + 4);
  const float* kbase = p.kbar + (size_t)g * N * kHeadDim + 8 * l16;
  constexpr int kPeUnroll = 4;
  for (int kb0 = 0; kb0 < L; kb0 += 16 * kPeUnroll) {
    f32x4 ka[kPeUnroll], kc[kPeUnroll];
#pragma unroll
    for (int u = 0; u < kPeUnroll; ++u) {
      const int kb = min(kb0 + 16 * u + grp, L - 1);  // rows past the causal range: a valid row, result unused
      ka[u] = *(const f32x4*)(kbase + (size_t)kb * kHeadDim);
      kc[u] = *(const f32x4*)(kbase + (size_t)kb * kHeadDim + 4);
    }
#pragma unroll
    for (int u = 0; u < kPeUnroll; ++u) {
      const int kb = kb0 + 16 * u + grp;
      float dot = qa[0] * ka[u][0] + qa[1] * ka[u][1] + qa[2] * ka[u][2] + qa[3] * ka[u][3] + qc[0] * kc[u][0] +
                  qc[1] * kc[u][1] + qc[2] * kc[u][2] + qc[3] * kc[u][3];
      dot += __shfl_xor(dot, 1);
      dot += __shfl_xor(dot, 2);
      dot += __shfl_xor(dot, 4);
      dot += __shfl_xor(dot, 8);
      if (kb < L && l16 == 0) pr[kb] = dot * p.scale_log2;
    }
  }
  __syncthreads();
  float mx = -INFINITY;
  for (int kb = tid; kb < L; kb += kPeThreads) mx = fmaxf(mx, pr[kb]);
  mx = block_max_f(mx, redf, tid, kPeThreads);
  float loc = 0.f;
  for (int kb = tid; kb < L; kb += kPeThreads) {
    const float e = fast_exp2(pr[kb] - mx);
    pr[kb] = e;
    loc += e;
  }
  const float sum = block_sum_f(loc, redf, tid, kPeThreads);
  for (int i = tid; i < L; i += kPeThreads) pr[i] = pr[i] / sum;
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
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < L; i += kPeThreads) {
      const uint64_t key = desc_key(pr[i], (uint32_t)i);
      if ((key & hi_mask) == decided)
        atomicAdd(&hist[(key >> sh) & 255], (uint32_t)(pr[i] * kFixOne));
    }
    __syncthreads();
    if (tid < 64) find_digit(hist, below, target, lane, &sel_digit, &sel_below);
    __syncthreads();
    const int d = sel_digit;
    if (d == 256) {  // the whole row never reaches gamma (rounding): keep everything
      keep_all = true;
      break;
    }
    below = sel_below;
    decided |= (uint64_t)d << sh;
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
  int32_t* out = p.idx + (size_t)h * ((size_t)N * (N + 1) / 2) + (size_t)qb * (qb + 1) / 2;
  for (int kb = beg; kb < end; ++kb)
    if (flags[kb]) out[pos++] = kb;
  if (tid == 0) p.count[(size_t)h * N + qb] = total;
}

// One workgroup per (head, 256 query blocks), one thread per query block.
// The head's kept vertical blocks V and slash bands S are compacted once
// into ascending LDS lists; the list of qb is the merge of {v in V : v <= qb}
// with the tiles qb - s - 1, qb - s of the bands s in S taken from the widest
// band down (an ascending sequence in which neighbouring bands repeat one
// block), dropping repeats and blocks below 0.
constexpr int kExpandRows = 256;
constexpr int kMaxBlocks = 4096;  // n <= 524288

__global__ __launch_bounds__(256) void vs_expand_kernel(const int32_t* route, const int32_t* vmask,
                                                        const int32_t* smask, int32_t* count, int32_t* idx, int nblk) {
  __shared__ int32_t vl[kMaxBlocks], sl[kMaxBlocks];
  __shared__ int scan_tmp[8];
  const int N = nblk, h = blockIdx.y, tid = threadIdx.x;
  if (route[h] != 1) return;
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
  b += align_up(hq * N * kHeadDim * sizeof(float)); // qbar
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
  b.qbar = (float*)take(hq * N * kHeadDim * sizeof(float));
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
    ta.n = n;
    ta.nblk = N;
    ta.alpha = alpha;
    ta.kmin_tokens = kmin * kBlock;
    ta.nf_stat = nf_stat;
    hipLaunchKernelGGL(tok_select_kernel, dim3(hq), dim3(kTokThreads), 0, stream, ta);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }

  hipLaunchKernelGGL(pe_pool_kernel, dim3(N, hq + hkv), dim3(256), 0, stream, q, k, route, b.qbar, b.kbar, hq,
                     hq / hkv, n);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  PeArgs pa;
  pa.qbar = b.qbar;
  pa.kbar = b.kbar;
  pa.route = route;
  pa.count = count;
  pa.idx = idx;
  pa.hq = hq;
  pa.qpg = hq / hkv;
  pa.nblk = N;
  pa.scale_log2 = scale * kLog2e;
  pa.gamma = use_gamma ? gamma : gamma_pe;
  const size_t pe_lds = (size_t)N * 4 + (size_t)N;
  hipLaunchKernelGGL(pe_select_kernel, dim3(hq * N), dim3(kPeThreads), pe_lds, stream, pa);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  hipLaunchKernelGGL(vs_expand_kernel, dim3((N + kExpandRows - 1) / kExpandRows, hq), dim3(256), 0, stream, route,
                     b.vmask, b.smask, count, idx, N);
  return hipGetLastError();
}

}  // namespace crisp
