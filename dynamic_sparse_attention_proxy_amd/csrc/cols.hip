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
// step's 64-bit slot mask with one ballot.  In a partial last block (128
// does not divide n) the query rows past n-1 are computed from row n-1 and
// not written; every gathered column lies below the pair's blocks.

#include <type_traits>

#include "common.h"
#include "internal.h"

namespace crisp {

namespace {

constexpr int kCStep = 64;                  // columns per step
constexpr int kCStages = 4;                 // K and V stages: three steps of lookahead
constexpr int kIdxChunk = 32 * kCStep;      // column indices per staged half
constexpr int kMaxTiles = 4096;             // key blocks per head (n <= 524288)
constexpr int kColThreads = 512;
constexpr int kColBits = (1 << 20) - 1;    // column index bits (entries hold them shifted by 8)
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
  int* queue;                // 8 claim counters, zero at launch
  int items;                 // Hq * pairs
};

struct ColLds {
  __bf16 kst[kCStages][kCStep * kHeadDim];
  __bf16 vst[kCStages][kCStep * kHeadDim];
  int32_t cidx[2][kIdxChunk];
  uint32_t tbits[2][kMaxTiles / 32];
  int next_item;
};

// One (head, pair of query blocks) item.  Every wave returns having passed
// the same barriers; the caller synchronises before reusing LDS.
__device__ __forceinline__ void col_item(const ColArgs& p, ColLds& L, int h, int pi) {
  auto& kst = L.kst;
  auto& vst = L.vst;
  auto& cidx = L.cidx;
  auto& tbits = L.tbits;
  const int N = p.nblk;
  // The lane index comes from an asm statement the compiler may not hoist
  // out of the item loop (see opaque_lane).
  const int lane = opaque_lane(), w = (int)threadIdx.x >> 6, tid = 64 * w + lane;
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
  const int g = h / p.qpg;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int32_t* colh = p.cols + (size_t)h * p.n;
  const int limit = (has_b ? qb2 : qa) * kBlock - 1;  // gathered keys stay below the pair's last block

  // listed tiles of both blocks as bitmaps
  for (int i = tid; i < 2 * (kMaxTiles / 32); i += kColThreads) (&tbits[0][0])[i] = 0;
  __syncthreads();
  for (int b = 0; b < (has_b ? 2 : 1); ++b) {
    const int qq = b ? qb2 : qa;
    // the tile kernel's reading of a list: the last entry is the diagonal
    // block, every other entry clamped to [0, qq-1]
    const int tc = min(max(p.count[(size_t)h * N + qq], 1), qq + 1);
    const int32_t* list = p.idx + (size_t)h * ((size_t)N * (N + 1) / 2) + (size_t)qq * (qq + 1) / 2;
    for (int t = tid; t < tc; t += kColThreads) {
      const int kb = t == tc - 1 ? qq : min(max(list[t], 0), qq - 1);
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
  // A staged entry holds the column times 256 (the byte offset of its K or V
  // row; a column is below 2^19) and, in bits 30 and 31, whether the slot
  // does not count for block 2p or 2p+1: past the kept columns below that
  // block, or inside one of its listed tiles.
  auto store_idx = [&](int chunk, const int32_t (&r)[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int slot = chunk * kIdxChunk + 4 * tid + e;
      const int c = r[e];
      const uint32_t wb = (uint32_t)((c >> 7) & 31), word = (uint32_t)(c >> 12);
      const bool off_a = slot >= cnt_a || ((tbits[0][word] >> wb) & 1u);
      const bool off_b = slot >= cnt_b || ((tbits[1][word] >> wb) & 1u);
      cidx[chunk & 1][4 * tid + e] =
          (int32_t)(((uint32_t)c << 8) | ((uint32_t)off_a << 30) | ((uint32_t)off_b << 31));
    }
  };
  {
    int32_t r[4];
    load_idx(0, r);
    __syncthreads();  // the bitmaps are complete before store_idx reads them
    store_idx(0, r);
  }
  __syncthreads();

  const size_t nd = (size_t)p.n * kHeadDim;
  const int qpos = qmine * kBlock + 32 * wq + l32;
  bf16x8 qf[8];
  if (active) {
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      qf[kk] = as_bf16x8(
          *(const u32x4*)(p.q + (size_t)h * nd + (size_t)min(qpos, p.n - 1) * kHeadDim + 16 * kk + 8 * lg));
  }
  // Q lands here, once, in a wait the compiler sees.  Its first use sits
  // under `active`, so without this the loads count as pending in the loop
  // and the compiler waits for them (vmcnt(7) .. vmcnt(0)) before the QK
  // MFMAs of every step; those waits also cover the column gathers in
  // flight, which it cannot see (measured without effect on the 512k token
  // chain: the gathers have landed by then).
  __builtin_amdgcn_s_waitcnt(0);

  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.k + (size_t)g * nd), 0, (int)(nd * 2), kBufferFlags);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.v + (size_t)g * nd), 0, (int)(nd * 2), kBufferFlags);
  // Gather of step s: wave w fills rows 8w .. 8w+7 of the stage; lane L of
  // instruction i row r = 8w + 4i + L/16, chunk position L & 15, i.e. global
  // chunk (L & 15) ^ swz(r) of the row's column.
  // this lane's byte address of its first gathered row's entry in a staged chunk
  const char* ci_lane = (const char*)&cidx[0][0] + 4 * (8 * w + (lane >> 4));
  auto gather = [&](int s, int st) {
    const int soff = ((s >> 5) & 1) * (kIdxChunk * 4) + (s & 31) * (kCStep * 4);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = 8 * w + 4 * i + (lane >> 4);
      const int base = *(const int32_t*)(ci_lane + soff + 16 * i) & (kColBits << 8);
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

  // Slot mask of step s for this wave's query block.
  const char* cm_lane = (const char*)&cidx[0][0] + 4 * lane;
  auto mask_of = [&](int s) -> uint64_t {
    const uint32_t e = *(const uint32_t*)(cm_lane + ((s >> 5) & 1) * (kIdxChunk * 4) + (s & 31) * (kCStep * 4));
    return __ballot(((e >> (30 + blk)) & 1u) == 0);
  };
  // Operand reads from the stage of a step: `s` need only equal the step
  // modulo 4 (the loop below passes the stage itself, a constant).
  auto kread = [&](int s, int t) -> bf16x8 {  // K operand of MFMA t (key half t & 1, d slice t / 2)
    const char* kb8 = (const char*)kst[s & (kCStages - 1)];
    return as_bf16x8(*(const u32x4*)(kb8 + k_off[t >> 1] + (t & 1) * 8192));
  };
  auto vread = [&](int s, int u) -> bf16x8 {  // V^T operand of PV MFMA u (d slice u & 3, P operand u / 4)
    __attribute__((address_space(3))) char* vb8 =
        (__attribute__((address_space(3))) char*)vst[s & (kCStages - 1)];
    const int db = u & 3, f = u >> 2;
    const int off = v_base[db] + (32 * (f >> 1) + 16 * (f & 1)) * 256;
    const bf16x4 lo = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4c*)(vb8 + off)));
    const bf16x4 hi =
        __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4c*)(vb8 + off + 4 * 256)));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  // register v < 8 of lane group lg holds slot 8lg + v, v >= 8 slot 16 + 8lg + (v - 8)
  auto lane_bits = [&](uint64_t m, int kb2) -> uint32_t {
    const uint32_t mh = (uint32_t)(m >> (32 * kb2));
    return ((mh >> (8 * lg)) & 0xffu) | (((mh >> (16 + 8 * lg)) & 0xffu) << 8);
  };
  auto row_max = [&](const f32x16 (&sc)[2]) -> float {
    float mx = -INFINITY;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sc[kb2][v]);
    return fmaxf(mx, __shfl_xor(mx, 32)) * p.scale_log2;
  };

  for (int s = 0; s < kCStages - 1 && s < nsteps; ++s) gather(s, s);
  // steps 0 and 1 must have landed: at most the gather of step 2 (4 per wave) outstanding
  if (nsteps >= 3)
    asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  else
    wait_dma();
  __syncthreads();

  // Iteration s: block 1 computes S_{s+1} = K_{s+1} Q^T (MFMA) beside the
  // exps of the second key half of S_s (VALU); S_{s+1} is masked if need be;
  // block 2 computes O += V_s P_s (MFMA) beside the exps of S_{s+1}'s first
  // key half, carried to the next iteration in pn / ls_lo (pc / ls_lo there:
  // the two operand pairs swap roles from step to step, so no copy is
  // made).  S_s arrives masked in
  // `sc`.  Lazy running max: set from the first counted step and raised
  // (rare) when a step's probabilities sum past kColSumLimit, the step's
  // exps then redone from `sc`; any value keeps the result exact.
  f32x16 sa[2], sb[2];
  uint64_t m_cur = 0;
  bf16x8 p_lo_a[2], p_lo_b[2];
  float ls_lo = 0.f;
  bool lo_ready = false;  // pc / ls_lo hold the first key half of S_s against m_run
  if (active) {
    m_cur = mask_of(0);
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      f32x16 acc = {};
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) acc = mfma32(kread(0, 2 * kk + kb2), qf[kk], acc);
      sa[kb2] = acc;
    }
    if (m_cur != ~0ull) {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        const uint32_t bits = lane_bits(m_cur, kb2);
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (!((bits >> v) & 1u)) sa[kb2][v] = -INFINITY;
      }
    }
  }
  // exps of one key half, packed as two PV B operands
  auto half_exps = [&](const f32x16& x, bf16x8& pa, bf16x8& pbb) -> float {
    float e[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) e[i] = fast_exp2(fmaf(x[i], p.scale_log2, -m_run));
    pa = pack_bf16x8(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]);
    pbb = pack_bf16x8(e[8], e[9], e[10], e[11], e[12], e[13], e[14], e[15]);
    return sum_rounded(pbb, sum_rounded(pa, 0.f));  // the rounded values that enter PV
  };

  auto iter = [&](int s, auto st_in, f32x16 (&sc)[2], f32x16 (&sn)[2], bf16x8 (&pc)[2], bf16x8 (&pn)[2]) {
    const int st = st_in;  // stage of step s (s mod 4), a constant in the unrolled loop
    // The next chunk of column indices, staged before this step's gather is
    // issued (its wait then only drains the previous step's gather).
    if ((s & 31) == 0 && (s >> 5) + 1 < nchunks) {
      int32_t nxt[4];
      load_idx((s >> 5) + 1, nxt);
      store_idx((s >> 5) + 1, nxt);
    }
    if (issues(s)) gather(s + kCStages - 1, (st + kCStages - 1) & (kCStages - 1));
    if (active) {
      const bool has_next = s + 1 < nsteps;
      const uint64_t m_next = has_next ? mask_of(s + 1) : 0ull;
      const bool cur_on = m_cur != 0ull;
      if (cur_on && !started) {
        m_run = row_max(sc);
        started = true;
        lo_ready = false;
      }
      if (cur_on && !lo_ready) ls_lo = half_exps(sc[0], pc[0], pc[1]);
      bf16x8 pb[4];
      float ls = 0.f;
      if (has_next && cur_on) {
        // block 1: MFMA t of S_{s+1} beside score t of the second key half of S_s
        bf16x8 kr[4];
        kr[0] = kread(st + 1, 0);
        kr[1] = kread(st + 1, 1);
        kr[2] = kread(st + 1, 2);
        const f32x16 zero = {};
        float e[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          sn[t & 1] = mfma32(kr[t & 3], qf[t >> 1], t < 2 ? zero : sn[t & 1]);
          if (t + 3 < 16) kr[(t + 3) & 3] = kread(st + 1, t + 3);
          e[t] = fast_exp2(fmaf(sc[1][t], p.scale_log2, -m_run));
          if ((t & 7) == 7)
            pb[2 + (t >> 3)] = pack_bf16x8(e[t - 7], e[t - 6], e[t - 5], e[t - 4], e[t - 3], e[t - 2], e[t - 1], e[t]);
          __builtin_amdgcn_sched_barrier(0);
        }
        ls = sum_rounded(pb[3], sum_rounded(pb[2], 0.f));
      } else {
        if (has_next) {
#pragma unroll
          for (int kb2 = 0; kb2 < 2; ++kb2) {
            f32x16 acc = {};
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) acc = mfma32(kread(st + 1, 2 * kk + kb2), qf[kk], acc);
            sn[kb2] = acc;
          }
        }
        if (cur_on) ls = half_exps(sc[1], pb[2], pb[3]);
      }
      if (cur_on) {
        ls += ls_lo;
        if (__any(!(ls <= kColSumLimit))) {  // rare: raise the running max, redo the step's exps
          const float m_new = fmaxf(m_run, row_max(sc));
          const float alpha = fast_exp2(m_run - m_new);
#pragma unroll
          for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int v = 0; v < 16; ++v) o[db][v] *= alpha;
          l_run *= alpha;
          m_run = m_new;
          ls = half_exps(sc[0], pc[0], pc[1]) + half_exps(sc[1], pb[2], pb[3]);
        }
        l_run += ls;
      }
      // S_{s+1}'s slots that do not count for this block, masked in a pass
      // of its own: most steps need none, and a check per unit inside the
      // block below cost more than the pass.
      const bool mask_next = has_next && m_next != ~0ull;
      const bool next_lo = has_next && m_next != 0ull && started;
      if (mask_next) {
        const uint32_t nb0 = lane_bits(m_next, 0), nb1 = lane_bits(m_next, 1);
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          const uint32_t bits = (i >> 4) ? nb1 : nb0;
          if (!((bits >> (i & 15)) & 1u)) sn[i >> 4][i & 15] = -INFINITY;
        }
      }
      // block 2: PV MFMA u beside the exp of score u of S_{s+1} (first key half)
      float lsn = 0.f;
      if (cur_on && next_lo) {
        bf16x8 vr[4];
        vr[0] = vread(st, 0);
        vr[1] = vread(st, 1);
        vr[2] = vread(st, 2);
        float e[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          o[u & 3] = mfma32(vr[u & 3], (u >> 2) < 2 ? pc[u >> 2] : pb[u >> 2], o[u & 3]);
          if (u + 3 < 16) vr[(u + 3) & 3] = vread(st, u + 3);
          e[u] = fast_exp2(fmaf(sn[0][u], p.scale_log2, -m_run));
          if ((u & 7) == 7)
            pn[u >> 3] = pack_bf16x8(e[u - 7], e[u - 6], e[u - 5], e[u - 4], e[u - 3], e[u - 2], e[u - 1], e[u]);
          __builtin_amdgcn_sched_barrier(0);
        }
        lsn = sum_rounded(pn[1], sum_rounded(pn[0], 0.f));
      } else {
        if (cur_on) {
#pragma unroll
          for (int u = 0; u < 16; ++u) o[u & 3] = mfma32(vread(st, u), (u >> 2) < 2 ? pc[u >> 2] : pb[u >> 2], o[u & 3]);
        }
        if (next_lo) lsn = half_exps(sn[0], pn[0], pn[1]);
      }
      ls_lo = lsn;
      lo_ready = next_lo;
      m_cur = m_next;
    }
    // K_{s+2} and V_{s+1} must have landed: only this iteration's gather may stay in flight
    if (issues(s))
      asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else
      wait_dma();
    __syncthreads();
  };
  // Four steps per trip, one per stage, so that every stage's LDS offsets
  // are instruction immediates; s is a multiple of 4 after the loop.
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  using S3 = std::integral_constant<int, 3>;
  int s = 0;
  for (; s + 3 < nsteps; s += 4) {
    iter(s, S0{}, sa, sb, p_lo_a, p_lo_b);
    iter(s + 1, S1{}, sb, sa, p_lo_b, p_lo_a);
    iter(s + 2, S2{}, sa, sb, p_lo_a, p_lo_b);
    iter(s + 3, S3{}, sb, sa, p_lo_b, p_lo_a);
  }
  if (s < nsteps) iter(s, S0{}, sa, sb, p_lo_a, p_lo_b);
  if (s + 1 < nsteps) iter(s + 1, S1{}, sb, sa, p_lo_b, p_lo_a);
  if (s + 2 < nsteps) iter(s + 2, S2{}, sa, sb, p_lo_a, p_lo_b);

  if (!active) return;
  // merge with the tile softmax of the same row
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (!(l_tot > 0.f)) return;  // no counted column for this row
  if (qpos >= p.n) return;     // a row of a partial last block past n
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
      for (int c = 0; c < 4; ++c) r[c] = fmaf(t[c], w1, o[db][4 * a + c] * wc) * inv;
      *ptr = r;
    }
  if (lg == 0) p.lse[row] = (M + fast_log2(denom)) * kLn2;
}

// Persistent workgroups, one per CU, take items from eight queues as the
// tile kernel does (queue x holds item ids x, x+8, ..., heaviest first per
// KV group; a workgroup starts with its XCD's queue, then takes from the
// others).  Item costs spread from a few microseconds to milliseconds (the
// kept columns below a pair grow with its position), which hardware
// dispatch, placing workgroups in order, turns into idle CUs.  The next
// item is claimed once the current one is done, so items start in the order
// their CUs free up.
__global__ __launch_bounds__(kColThreads, 1) void col_attn_kernel(ColArgs p) {
  __shared__ __attribute__((aligned(1024))) ColLds L;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const bool claimer = wave == 0;
  // workgroup b runs on XCD b mod 8 (round-robin dispatch)
  int queue = (int)(blockIdx.x & 7), tried = 0;
  auto claim = [&]() -> int {
    while (tried < 8) {
      int old = 0;
      if (opaque_lane() == 0) old = atomicAdd(p.queue + queue, 1);
      const int id = 8 * __builtin_amdgcn_readfirstlane(old) + queue;
      if (id < p.items) return id;
      queue = (queue + 1) & 7;
      ++tried;
    }
    return -1;
  };
  for (;;) {
    if (claimer) {
      const int next = claim();
      if (opaque_lane() == 0) L.next_item = next;
    }
    __syncthreads();
    const int item = L.next_item;
    if (item < 0) break;
    int h, pi;
    map_row(p.map, item, &h, &pi);
    col_item(p, L, h, pi);
    __syncthreads();
  }
}

__global__ void clear_col_queue_kernel(int* queue) {
  if (threadIdx.x < 8) queue[threadIdx.x] = 0;
}

}  // namespace

hipError_t launch_col_attention(const __bf16* q, const __bf16* k, const __bf16* v, const int32_t* count,
                                const int32_t* idx, const int32_t* cols, const int32_t* col_below, float* out,
                                float* lse, int hq, int hkv, int n, float scale, int* queue, hipStream_t stream) {
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
  a.nblk = nblocks(n);
  a.qpg = hq / hkv;
  a.scale_log2 = scale * kLog2e;
  const int npairs = (a.nblk + 1) / 2;
  a.map = make_row_map(hq, hkv, npairs);
  a.queue = queue;
  a.items = hq * npairs;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(clear_col_queue_kernel, dim3(1), dim3(64), 0, stream, queue);
  hipLaunchKernelGGL(col_attn_kernel, dim3((unsigned)min(a.items, max(cus, 1))), dim3(kColThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace crisp
