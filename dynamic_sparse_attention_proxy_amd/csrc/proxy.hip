// Proxy attention map and structural-mass routing (gfx950).
//
// The proxy rows are the last 128 query positions of every head, attending
// causally to all n keys (CRISP, ai.info summary, "Key Contributions" item 2:
// C_struct reads a proxy attention map the method computes anyway).
//
// Both passes run one workgroup per (head, chunk of kProxyChunk keys): its 4
// wavefronts own proxy rows 32w..32w+31 and compute S^T = K.Q^T with Q in
// VGPRs, so each lane owns one row (keys split between lanes l and l ^ 32).
// K streams through three LDS stages, 64 keys per step, by LDS DMA shared by
// the 4 waves (one barrier per step).
// Pass 1 (stats): per lane a running (max, sum of exp2) of its row over its
//   keys of the chunk; the running max only has to keep the exps in range,
//   so it is taken from the first step and raised only when a step's sum
//   exceeds kSumLimit.  Lanes l and l ^ 32 merge at the end.  When the block
//   masses are the only output, this pass also keeps each row's mass per key
//   block, split at the tile diagonal, against its running max, and writes
//   it at the end of every key block.
// Combine: one wavefront per (head, row) merges the chunk partials into the
//   row's log2-sum-exp; with the per-row block parts, one more small kernel
//   weighs them by 2^(max - lse2) and sums the 128 rows into the block masses.
// Pass 2 (map, or block masses beside the map or the column masses):
//   recompute S and form exp2(t - lse2).  It stores the map and/or the block
//   masses (per (head, key block) the map's mass on and below the tile
//   diagonal, row >= column, and above it) and/or the column masses.  A
//   chunk is whole key blocks and its 4 waves cover all 128 rows, so each
//   block's masses are complete inside one workgroup.
// Route: C_struct = mean over rows of the mass on the first sink_width and
//   the last recency_width columns (from the map, or from the block masses
//   when both widths are 128); VS when C_struct >= tau.
//
// Block masses: proxy row r (position n-128+r) against key j lies at offset
// n-128+r-j, in slash band (offset) / 128.  With t = n - 128 (N-1) positions
// in the last key block, entry (r, column c) of key block kb lies in band
// N-1-kb + floor((r - c + t - 128) / 128): band N-1-kb ("lo"), N-2-kb ("up")
// or, only when t < 128, N-3-kb ("up2").  Against the 32 rows of wave w, the
// 32 columns of sub-tile st give r - c + t - 128 = D + (l32 - cc) with
// D = 32 (w - st) + t - 128, so a sub-tile lies in one band or straddles one
// band edge (0 or -128), which a per-element compare splits.  With t = 128
// this is the tile diagonal: below for st < w, above for st > w, split for
// st = w.  The fourth plane is the mass on the last 128 keys: all of block
// N-1, and the columns c >= t of block N-2.

#include "common.h"
#include "internal.h"

namespace crisp {

namespace {

constexpr int kPStep = 64;          // keys per pipeline step
constexpr int kPStages = 3;         // K tiles in LDS: the current one and two in flight
constexpr float kSumLimit = 65536.f; // a step's sum above this raises the running max

struct ProxyArgs {
  const __bf16* q;
  const __bf16* k;
  float* amap;
  float* mass;   // [4][Hq][N]: slash bands N-1-kb, N-2-kb, N-3-kb of each key block; its recency mass
  float* colmass;  // [Hq][n]: column mass, the map's column sums over the rows / 128
  float* part;   // [Hq][128][chunks][2]
  f32x4* bpart;  // [Hq][N][128]: per row and key block, (lo, up, up2, max) in base 2 against that max
  float* rpart;  // [Hq][128]: per row, the recency part of key block N-2 against its bpart max
  float* lse2;   // [Hq][128]
  float* row_lse;
  int n;
  int nblk;
  int tlast;     // positions in the last key block, 1..128
  int qpg;
  int nchunks;
  float scale_log2;
  RowMap map;    // workgroup id -> (head, key chunk), over the chunks as blocks
};

// Band class of sub-tile st against the rows of wave w (see the top):
// 0, 1, 2 = wholly in band lo, up, up2; 3 = split at edge 0 (lo / up);
// 4 = split at edge -128 (up / up2).  D = 32 (w - st) + tlast - 128.
__device__ __forceinline__ int band_class(int D) {
  if (D - 31 >= 0) return 0;
  if (D + 31 < -128) return 2;
  if (D + 31 < 0 && D - 31 >= -128) return 1;
  return D + 31 >= 0 ? 3 : 4;
}

// Adds this lane's 16 values of a sub-tile of class `cls` into the three
// band sums; x = l32 + D - edge decides a split sub-tile per element (the
// upper band when x >= the element's column).
template <typename KeyOf>
__device__ __forceinline__ void add_bands(const float (&e)[16], float tot, int cls, int x, KeyOf key_of,
                                          float& b0, float& b1, float& b2) {
  // Every band takes a predicated add: a branch that picks which of
  // b0 / b1 / b2 to update becomes a pointer select, and the three sums are
  // then kept in scratch memory, whose waits also cover the K prefetch.
  if (cls < 3) {
    b0 += cls == 0 ? tot : 0.f;
    b1 += cls == 1 ? tot : 0.f;
    b2 += cls == 2 ? tot : 0.f;
    return;
  }
  float hi = 0.f, lo = 0.f;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    if (x >= key_of(v))
      hi += e[v];
    else
      lo += e[v];
  }
  const bool c3 = cls == 3;
  b0 += c3 ? hi : 0.f;
  b1 += c3 ? lo : hi;
  b2 += c3 ? 0.f : lo;
}

__device__ __forceinline__ void merge_ml(float& m, float& l, float mo, float lo) {
  const float M = fmaxf(m, mo);
  if (M == -INFINITY) return;
  l = l * fast_exp2(m - M) + lo * fast_exp2(mo - M);
  m = M;
}

// Key offset (0..31 within a 32-key half) of accumulator register v in
// lane group lg: rows 8 (v / 4) + 4 lg + v % 4 of the K operand.
__device__ __forceinline__ int acc_key(int v, int lg) { return 8 * (v >> 2) + 4 * lg + (v & 3); }

// Sum over the 32 rows of a wave of each of a lane's 16 key values (one
// 32-key half of a step): reduce-scatter by halving over lane bits 4..1 of
// l32 (8 + 4 + 2 + 1 exchanges), then one exchange with lane ^ 1.  Lane l32
// returns the total of register v = l32 >> 1 (both lanes of a pair hold it).
__device__ __forceinline__ float rows_sum_scatter(const float (&a)[16], int l32) {
  float r8[8], r4[4], r2[2];
  const bool b4 = l32 & 16, b3 = l32 & 8, b2 = l32 & 4, b1 = l32 & 2;
#pragma unroll
  for (int e = 0; e < 8; ++e) r8[e] = (b4 ? a[e + 8] : a[e]) + __shfl_xor(b4 ? a[e] : a[e + 8], 16);
#pragma unroll
  for (int e = 0; e < 4; ++e) r4[e] = (b3 ? r8[e + 4] : r8[e]) + __shfl_xor(b3 ? r8[e] : r8[e + 4], 8);
#pragma unroll
  for (int e = 0; e < 2; ++e) r2[e] = (b2 ? r4[e + 2] : r4[e]) + __shfl_xor(b2 ? r4[e] : r4[e + 2], 4);
  const float r1 = (b1 ? r2[1] : r2[0]) + __shfl_xor(b1 ? r2[0] : r2[1], 2);
  return r1 + __shfl_xor(r1, 1);
}

// kPass 0: row statistics.  kPass 1: map (kMap) and/or block masses (kMass),
// and the column masses (kCols).
template <int kPass, bool kMap, bool kMass, bool kCols, bool kRagged>
__global__ __launch_bounds__(256) void proxy_pass_kernel(ProxyArgs p) {
  __shared__ __attribute__((aligned(1024))) __bf16 ks[kPStages][kPStep * kHeadDim];
  __shared__ float part[4][kProxyChunk / kBlock][4];  // masses per wave and key block of the chunk
  // column masses of a step per wave, by step parity: summed over the waves
  // by the first 64 threads in the next step (after its barrier)
  __shared__ float colpart[kCols ? 2 : 1][4][kPStep];
  // map path: each wave's 32 x 32 tile of the map (one key half of a step),
  // row stride 36 floats so that the per-lane 16-byte writes of 16 rows hit
  // distinct banks
  constexpr int kTStride = 36;
  __shared__ __attribute__((aligned(16))) float tbuf[kMap ? 4 * 32 * kTStride : 1];
  // The heads of a KV group read the same K chunk: the row map deals them
  // to one XCD on consecutive slots, so K comes from that XCD's L2 once per
  // group instead of from HBM once per head.
  int chunk, h;
  map_row(p.map, blockIdx.x, &h, &chunk);
  const int g = h / p.qpg;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l32 = lane & 31, lg = lane >> 5;
  const int kbeg = chunk * kProxyChunk, kend = min(p.n, kbeg + kProxyChunk);
  // whole key blocks (even, >= 2): a partial last block runs both steps
  const int nsteps = 2 * ((kend - kbeg + kBlock - 1) / kBlock);
  const int pos0 = p.n - kBlock;
  const int row = 32 * w + l32;

  // Q row as the B operand: d = 16 kk + 8 lg + [0, 8)
  bf16x8 qf[8];
  const __bf16* qrow = p.q + ((size_t)h * p.n + pos0 + row) * kHeadDim + 8 * lg;
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) qf[kk] = as_bf16x8(*(const u32x4*)(qrow + 16 * kk));

  // LDS DMA of a 64-key tile: wave w fills rows 16w .. 16w+15, lane L of
  // instruction i row 16w + 4i + L/16 at chunk position L & 15.
  const size_t nd = (size_t)p.n * kHeadDim;
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.k + (size_t)g * nd), 0, (int)(nd * 2), kBufferFlags);
  int dma_k[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 16 * w + 4 * i + (lane >> 4);
    dma_k[i] = r * 256 + (((lane & 15) ^ swz_k(r)) << 4);
  }
  const int wu = __builtin_amdgcn_readfirstlane(w);
  auto dma_tile = [&](int stage, int step) {
    const int key0 = kbeg + step * kPStep;
    const bool past = kRagged && key0 + kPStep > p.n;  // rows past n read row n-1 (masked: past every proxy row)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * w + 4 * i + (lane >> 4);
      const int voff = past ? min(key0 + r, p.n - 1) * (kHeadDim * 2) + (dma_k[i] & 255) : dma_k[i];
      lds_dma_16B(krs, voff, past ? 0 : key0 * (kHeadDim * 2),
                  (unsigned)(uintptr_t)(__attribute__((address_space(3))) void*)(ks[stage] + (16 * wu + 4 * i) *
                                                                                              kHeadDim));
    }
  };
  // K operand of this lane: row l32 of each 32-key half, logical chunk 2 kk + lg.
  int k_off[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) k_off[kk] = l32 * 256 + (((2 * kk + lg) ^ swz_k(l32)) << 4);
  auto qk = [&](int stage, f32x16 (&s)[2]) {
    const char* kb8 = (const char*)ks[stage];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      f32x16 acc = {};
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) acc = mfma32(as_bf16x8(*(const u32x4*)(kb8 + k_off[kk] + kb2 * 8192)), qf[kk], acc);
      s[kb2] = acc;
    }
  };

  float m = -INFINITY, l = 0.f;  // pass 1: this lane's running max (scaled) and sum
  float neg_lse = 0.f;           // pass 2
  if (kPass == 1) neg_lse = -p.lse2[h * kBlock + row];
  float lo = 0.f, up = 0.f;      // this lane's masses of the current key block (pass 2: final; pass 1: against m)
  float up2 = 0.f, rc = 0.f;     // kRagged: band N-3-kb, and the recency part of key block N-2
  auto key_of = [&](int v) { return acc_key(v, lg); };

  // Q and the row log-sum-exp land here, in a wait the compiler sees: left
  // pending into the loop, the compiler would wait for them before the QK
  // MFMAs of every step, and those waits also cover the K DMA in flight.
  __builtin_amdgcn_s_waitcnt(0);
  dma_tile(0, 0);
  dma_tile(1, 1);
  wait_dma();
  __syncthreads();
  for (int j = 0; j < nsteps; ++j) {
    const bool ahead = j + 2 < nsteps;
    if (ahead) dma_tile((j + 2) % kPStages, j + 2);
    f32x16 s[2];
    qk(j % kPStages, s);
    const int key0 = kbeg + j * kPStep;
    if (key0 + kPStep - 1 > pos0) {  // keys past the first proxy row: causal mask
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (key0 + 32 * kb2 + acc_key(v, lg) > pos0 + row) s[kb2][v] = -INFINITY;
    }
    if (kPass == 0) {
      // the running max starts at the first step's max: -inf only for a lane
      // that sees none of the chunk's first keys, and then none later either
      if (j == 0) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[kb2][v]);
        m = mx * p.scale_log2;
      }
      const float neg_m = (m == -INFINITY) ? 0.f : -m;
      // this step's row sum and, with kMass, its part below / above the tile
      // diagonal (sub-tile t of the key block against row group w: all below
      // when t < w, all above when t > w, split by row >= column when equal)
      const int half = (key0 >> 6) & 1;
      const int kbk = key0 >> 7;  // key block of this step
      float ls = 0.f, bl = 0.f, bu = 0.f, bu2 = 0.f, brc = 0.f;
      auto step_sums = [&](float nm) {
        ls = bl = bu = bu2 = brc = 0.f;
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
          const int t = 2 * half + kb2;
          float e[16];
#pragma unroll
          for (int v = 0; v < 16; ++v) e[v] = fast_exp2(fmaf(s[kb2][v], p.scale_log2, nm));
          if (kRagged) {
            float t8[8];
#pragma unroll
            for (int v = 0; v < 8; ++v) t8[v] = e[v] + e[v + 8];
#pragma unroll
            for (int v = 0; v < 4; ++v) t8[v] += t8[v + 4];
            const float sum = (t8[0] + t8[2]) + (t8[1] + t8[3]);
            ls += sum;
            if (kMass) {
              const int D = 32 * (w - t) + p.tlast - kBlock;
              const int cls = band_class(D);
              add_bands(e, sum, cls, l32 + D - (cls == 4 ? -kBlock : 0), key_of, bl, bu, bu2);
              if (kbk == p.nblk - 2) {  // keys >= n - 128: columns >= R of this sub-tile
                const int R = pos0 - key0 - 32 * kb2;
                if (R <= 0) {
                  brc += sum;
                } else if (R < 32) {
#pragma unroll
                  for (int v = 0; v < 16; ++v)
                    if (acc_key(v, lg) >= R) brc += e[v];
                }
              }
            }
          } else if (kMass && t == w) {
            float dl = 0.f, du = 0.f;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              if (l32 >= acc_key(v, lg))
                dl += e[v];
              else
                du += e[v];
            }
            ls += dl + du;
            bl += dl;
            bu += du;
          } else {
            float t8[8];
#pragma unroll
            for (int v = 0; v < 8; ++v) t8[v] = e[v] + e[v + 8];
#pragma unroll
            for (int v = 0; v < 4; ++v) t8[v] += t8[v + 4];
            const float sum = (t8[0] + t8[2]) + (t8[1] + t8[3]);
            ls += sum;
            if (kMass) {
              // predicated (see add_bands): the sub-tile is wholly below or above
              bl += t < w ? sum : 0.f;
              bu += t < w ? 0.f : sum;
            }
          }
        }
      };
      step_sums(neg_m);
      if (__any(!(ls <= kSumLimit))) {  // rare: raise this lane's max to its step max, redo the sums
        float mx = -INFINITY;
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[kb2][v]);
        const float m_new = fmaxf(m, mx * p.scale_log2);
        if (m_new != -INFINITY) {
          const float r = fast_exp2(m - m_new);
          l *= r;
          lo *= r;
          up *= r;
          if (kRagged) {
            up2 *= r;
            rc *= r;
          }
          m = m_new;
          step_sums(-m);
        }
      }
      l += ls;
      if (kMass) {
        lo += bl;
        up += bu;
        if (kRagged) {
          up2 += bu2;
          rc += brc;
        }
        if (half == 1) {  // end of a key block: this row's parts, against a common max
          const float mo = __shfl_xor(m, 32), loo = __shfl_xor(lo, 32), upo = __shfl_xor(up, 32);
          const float up2o = kRagged ? __shfl_xor(up2, 32) : 0.f, rco = kRagged ? __shfl_xor(rc, 32) : 0.f;
          const float M = fmaxf(m, mo);
          // M = -inf: the row sees no key of this chunk yet (a partial last
          // chunk that starts past the row), and every part is 0
          const bool none = M == -INFINITY;
          const float a = none ? 0.f : fast_exp2(m - M), b = none ? 0.f : fast_exp2(mo - M);
          if (lg == 0) {
            f32x4 rec;
            rec[0] = lo * a + loo * b;
            rec[1] = up * a + upo * b;
            rec[2] = kRagged ? up2 * a + up2o * b : 0.f;
            rec[3] = M;
            p.bpart[((size_t)h * p.nblk + kbk) * kBlock + row] = rec;
            if (kRagged && kbk == p.nblk - 2) p.rpart[h * kBlock + row] = rc * a + rco * b;
          }
          lo = 0.f;
          up = 0.f;
          up2 = 0.f;
          rc = 0.f;
        }
      }
    } else {
      // sub-tile t (32 keys) of the key block against row group w: all
      // below the diagonal when t < w, all above when t > w, split when equal
      // (with 128 | n; band_class in general)
      const int half = (key0 >> 6) & 1;
      const int kbk = key0 >> 7;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        const int t = 2 * half + kb2;
        float a[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) a[v] = fast_exp2(fmaf(s[kb2][v], p.scale_log2, neg_lse));
        if (kMass && kRagged) {
          float t8[8];
#pragma unroll
          for (int v = 0; v < 8; ++v) t8[v] = a[v] + a[v + 8];
#pragma unroll
          for (int v = 0; v < 4; ++v) t8[v] += t8[v + 4];
          const float sum = (t8[0] + t8[2]) + (t8[1] + t8[3]);
          const int D = 32 * (w - t) + p.tlast - kBlock;
          const int cls = band_class(D);
          add_bands(a, sum, cls, l32 + D - (cls == 4 ? -kBlock : 0), key_of, lo, up, up2);
          if (kbk == p.nblk - 2) {
            const int R = pos0 - key0 - 32 * kb2;
            if (R <= 0) {
              rc += sum;
            } else if (R < 32) {
#pragma unroll
              for (int v = 0; v < 16; ++v)
                if (acc_key(v, lg) >= R) rc += a[v];
            }
          }
        } else if (kMass) {
          if (t == w) {  // the diagonal sub-tile: split by row >= column
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              if (l32 >= acc_key(v, lg))
                lo += a[v];
              else
                up += a[v];
            }
          } else {  // wave-uniform: the whole sub-tile on one side
            float t8[8];
#pragma unroll
            for (int v = 0; v < 8; ++v) t8[v] = a[v] + a[v + 8];
#pragma unroll
            for (int v = 0; v < 4; ++v) t8[v] += t8[v + 4];
            const float sum = (t8[0] + t8[2]) + (t8[1] + t8[3]);
            lo += t < w ? sum : 0.f;  // predicated (see add_bands)
            up += t < w ? 0.f : sum;
          }
        }
        if (kCols) {
          const float cs = rows_sum_scatter(a, l32);
          if ((l32 & 1) == 0) colpart[j & 1][w][32 * kb2 + acc_key(l32 >> 1, lg)] = cs;
        }
        if (kMap) {
          // Through the wave's LDS tile (row l32, keys 8 q4 + 4 lg + [0, 4)),
          // then row-major out: instruction i writes rows 8i .. 8i+7 of the
          // wave, 128 contiguous bytes each, with non-temporal stores (the
          // map is written once).  The wave reads back only its own writes,
          // and LDS operations of a wave complete in order.
          float* t = tbuf + (32 * w + l32) * kTStride + 4 * lg;
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            f32x4 o;
            o[0] = a[4 * q4];
            o[1] = a[4 * q4 + 1];
            o[2] = a[4 * q4 + 2];
            o[3] = a[4 * q4 + 3];
            *(f32x4*)(t + 8 * q4) = o;
          }
          const int rr = lane >> 3, cc = 4 * (lane & 7);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 8 * i + rr;
            const f32x4 o = *(const f32x4*)(tbuf + (32 * w + r) * kTStride + cc);
            float* dst = p.amap + ((size_t)h * kBlock + 32 * w + r) * p.n + key0 + 32 * kb2 + cc;
            if (kRagged) {  // rows of n floats are not 16-byte aligned; no column past n
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (key0 + 32 * kb2 + cc + e < p.n) __builtin_nontemporal_store(o[e], dst + e);
            } else {
              __builtin_nontemporal_store(o, (f32x4*)dst);
            }
          }
        }
      }
      if (kCols && j > 0 && tid < kPStep && key0 - kPStep + tid < p.n) {  // the previous step's column masses
        const float* cp = &colpart[(j - 1) & 1][0][tid];
        p.colmass[(size_t)h * p.n + key0 - kPStep + tid] =
            (cp[0] + cp[kPStep] + cp[2 * kPStep] + cp[3 * kPStep]) * (1.f / kBlock);
      }
      if (kMass && half == 1) {  // end of a key block: reduce and park the wave's sums
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          lo += __shfl_xor(lo, o);
          up += __shfl_xor(up, o);
          if (kRagged) {
            up2 += __shfl_xor(up2, o);
            rc += __shfl_xor(rc, o);
          }
        }
        if (lane == 0) {
          part[w][(key0 - kbeg) >> 7][0] = lo;
          part[w][(key0 - kbeg) >> 7][1] = up;
          part[w][(key0 - kbeg) >> 7][2] = kRagged ? up2 : 0.f;
          part[w][(key0 - kbeg) >> 7][3] = kRagged ? rc : 0.f;
        }
        lo = 0.f;
        up = 0.f;
        up2 = 0.f;
        rc = 0.f;
      }
    }
    if (ahead)
      wait_dma_but_4();
    else
      wait_dma();
    __syncthreads();
  }

  if (kPass == 0) {
    // lanes l and l ^ 32 hold the same row: merge, then one lane writes it
    const float mo = __shfl_xor(m, 32), lo2 = __shfl_xor(l, 32);
    merge_ml(m, l, mo, lo2);
    if (lg == 0) {
      float* dst = p.part + (((size_t)h * kBlock + row) * p.nchunks + chunk) * 2;
      dst[0] = m;
      dst[1] = l;
    }
  } else {
    const int klast = kbeg + (nsteps - 1) * kPStep;  // first key of the last step
    if (kCols && tid < kPStep && klast + tid < p.n) {  // the last step's column masses
      const float* cp = &colpart[(nsteps - 1) & 1][0][tid];
      p.colmass[(size_t)h * p.n + klast + tid] =
          (cp[0] + cp[kPStep] + cp[2 * kPStep] + cp[3 * kPStep]) * (1.f / kBlock);
    }
  }
  if (kPass == 1 && kMass) {
    // the loop's last barrier orders every wave's parked sums before this
    const int nkb = nsteps >> 1;
    if (tid < 4 * nkb) {
      const int jb = tid >> 2, which = tid & 3, kb = (kbeg >> 7) + jb;
      const int N = p.nblk, hq = p.map.hq;
      float v;
      if (which < 3) {
        v = part[0][jb][which] + part[1][jb][which] + part[2][jb][which] + part[3][jb][which];
      } else if (kb == N - 1) {  // the recency window holds every visible key of the last block
        v = 0.f;
#pragma unroll
        for (int c = 0; c < 3; ++c) v += part[0][jb][c] + part[1][jb][c] + part[2][jb][c] + part[3][jb][c];
      } else {
        v = part[0][jb][3] + part[1][jb][3] + part[2][jb][3] + part[3][jb][3];
      }
      p.mass[((size_t)which * hq + h) * N + kb] = v;
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

// Block masses from the stats pass's per-row parts: for each band plane,
// mass[c][h][kb] = sum over the 128 rows of part_c * 2^(max - lse2); the
// recency plane is the whole of block N-1 and the rows' recency parts of
// block N-2.  One workgroup per (head, 8 key blocks), 32 lanes per key block.
__global__ __launch_bounds__(256) void mass_combine_kernel(ProxyArgs p) {
  const int h = blockIdx.y, hq = gridDim.y, tid = threadIdx.x;
  const int N = p.nblk;
  const int kb = blockIdx.x * 8 + (tid >> 5), li = tid & 31;
  float lo = 0.f, up = 0.f, up2 = 0.f, rc = 0.f;
  if (kb < N) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = li + 32 * i;
      const f32x4 rec = p.bpart[((size_t)h * N + kb) * kBlock + r];
      const float wgt = fast_exp2(rec[3] - p.lse2[h * kBlock + r]);
      lo += rec[0] * wgt;
      up += rec[1] * wgt;
      up2 += rec[2] * wgt;
      if (p.tlast < kBlock && kb == N - 2) rc += p.rpart[h * kBlock + r] * wgt;
    }
  }
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) {
    lo += __shfl_xor(lo, o);
    up += __shfl_xor(up, o);
    up2 += __shfl_xor(up2, o);
    rc += __shfl_xor(rc, o);
  }
  if (kb < N && li == 0) {
    p.mass[(size_t)h * N + kb] = lo;
    p.mass[((size_t)hq + h) * N + kb] = up;
    p.mass[((size_t)2 * hq + h) * N + kb] = up2;
    p.mass[((size_t)3 * hq + h) * N + kb] = kb == N - 1 ? lo + up + up2 : rc;
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

// C_struct from the column masses (the map's column sums over the rows /
// 128), for any sink and recency widths: the same sum as route_kernel's,
// over one row of column masses instead of the map's 128 rows.
__global__ __launch_bounds__(256) void route_cols_kernel(const float* colmass, float* c_struct, int32_t* route, int n,
                                                         int ws, int wr, float tau, int override_mode) {
  __shared__ float red[8];
  const int h = blockIdx.x, tid = threadIdx.x;
  const float* c_h = colmass + (size_t)h * n;
  float acc = 0.f;
  for (int e = tid; e < ws + wr; e += 256) acc += c_h[e < ws ? e : n - wr + (e - ws)];
  const float c = block_sum_f(acc, red, tid, 256);
  if (tid == 0) {
    c_struct[h] = c;
    route[h] = override_mode == 1 ? 1 : override_mode == 2 ? 0 : (c >= tau ? 1 : 0);
  }
}

// C_struct from the block masses when sink and recency widths are both one
// block: the mass of key block 0 (the first 128 keys) and the recency plane
// (the last 128 keys: block N-1 and the tail of block N-2) over the 128 rows.
__global__ void route_mass_kernel(const float* mass, float* c_struct, int32_t* route, int hq, int nblk, float tau,
                                  int override_mode) {
  const int h = blockIdx.x * blockDim.x + threadIdx.x;
  if (h >= hq) return;
  const size_t plane = (size_t)hq * nblk;
  const float* m0 = mass + (size_t)h * nblk;
  const float* rec = m0 + 3 * plane;
  const float c = (m0[0] + m0[plane] + m0[2 * plane] + rec[nblk - 2] + rec[nblk - 1]) / (float)kBlock;
  c_struct[h] = c;
  route[h] = override_mode == 1 ? 1 : override_mode == 2 ? 0 : (c >= tau ? 1 : 0);
}

}  // namespace

hipError_t launch_proxy(const __bf16* q, const __bf16* k, float* amap, float* mass, float* colmass, float* row_lse,
                        void* scratch, int hq, int hkv, int n, float scale, hipStream_t stream) {
  ProxyArgs a;
  a.q = q;
  a.k = k;
  a.amap = amap;
  a.mass = mass;
  a.colmass = colmass;
  a.nchunks = proxy_chunks(n);
  a.nblk = nblocks(n);
  a.tlast = n - kBlock * (a.nblk - 1);
  a.part = (float*)scratch;
  a.lse2 = a.part + (size_t)hq * a.nchunks * kBlock * 2;
  a.bpart = (f32x4*)(a.lse2 + (size_t)hq * kBlock);
  a.rpart = (float*)(a.bpart + (size_t)hq * a.nblk * kBlock);
  a.row_lse = row_lse;
  a.n = n;
  a.qpg = hq / hkv;
  a.scale_log2 = scale * kLog2e;
  const bool ragged = a.tlast != kBlock;
  a.map = make_row_map(hq, hkv, a.nchunks);
  const dim3 grid(a.nchunks * hq);
  // Block masses alone come out of the stats pass (per-row parts against the
  // running max) and one small combine: no second pass over K.
  const bool one_pass = mass != nullptr && amap == nullptr && colmass == nullptr;
  if (one_pass && ragged)
    hipLaunchKernelGGL((proxy_pass_kernel<0, false, true, false, true>), grid, dim3(256), 0, stream, a);
  else if (one_pass)
    hipLaunchKernelGGL((proxy_pass_kernel<0, false, true, false, false>), grid, dim3(256), 0, stream, a);
  else if (ragged)
    hipLaunchKernelGGL((proxy_pass_kernel<0, false, false, false, true>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((proxy_pass_kernel<0, false, false, false, false>), grid, dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(proxy_combine_kernel, dim3(hq * kBlock / 4), dim3(256), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (one_pass) {
    hipLaunchKernelGGL(mass_combine_kernel, dim3((a.nblk + 7) / 8, hq), dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  if (colmass != nullptr) {  // with the block masses, without the map
    if (ragged)
      hipLaunchKernelGGL((proxy_pass_kernel<1, false, true, true, true>), grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((proxy_pass_kernel<1, false, true, true, false>), grid, dim3(256), 0, stream, a);
  } else if (mass != nullptr) {  // the map and the block masses
    if (ragged)
      hipLaunchKernelGGL((proxy_pass_kernel<1, true, true, false, true>), grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((proxy_pass_kernel<1, true, true, false, false>), grid, dim3(256), 0, stream, a);
  } else {
    if (ragged)
      hipLaunchKernelGGL((proxy_pass_kernel<1, true, false, false, true>), grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((proxy_pass_kernel<1, true, false, false, false>), grid, dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_route_cols(const float* colmass, float* c_struct, int32_t* route, int hq, int n, int sink_width,
                             int recency_width, float tau, int route_override, hipStream_t stream) {
  hipLaunchKernelGGL(route_cols_kernel, dim3(hq), dim3(256), 0, stream, colmass, c_struct, route, n, sink_width,
                     recency_width, tau, route_override);
  return hipGetLastError();
}

hipError_t launch_route(const float* amap, const float* mass, float* c_struct, int32_t* route, int hq, int n,
                        int sink_width, int recency_width, float tau, int route_override, hipStream_t stream) {
  if (mass != nullptr)
    hipLaunchKernelGGL(route_mass_kernel, dim3((hq + 63) / 64), dim3(64), 0, stream, mass, c_struct, route, hq,
                       nblocks(n), tau, route_override);
  else
    hipLaunchKernelGGL(route_kernel, dim3(hq), dim3(256), 0, stream, amap, c_struct, route, n, sink_width,
                       recency_width, tau, route_override);
  return hipGetLastError();
}

}  // namespace crisp
