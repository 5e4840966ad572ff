// Block-sparse and dense causal flash attention for gfx950.
//
// Exact softmax attention over the key blocks selected for each query block
// (CRISP, ai.info summary, "Why This Matters": exact softmax over the kept
// blocks; dense attention is the baseline of "Main Findings").
//
// One workgroup computes one (head, 128-query block).  Its four waves own 32
// query rows each.  Keys stream through LDS 64 at a time, double buffered:
// K row-major ([key][d]) and V transposed ([d][key]).  Per step a wave
//   S^T[64 keys x 32 queries] = K . Q^T      (16 MFMA 32x32x16, Q in VGPRs)
//   online softmax in base 2                  (each lane owns one query row)
//   O^T[128 d x 32 queries] += V^T . P^T     (16 MFMA 32x32x16)
// Computing the transposed products puts a query's scores in one lane and
// in exactly the layout the second product takes as its B operand, so no
// cross-lane traffic is needed besides one max exchange with lane ^ 32.
// Rows of the K operand are loaded in a permuted order chosen so that the
// accumulator registers 0..7 / 8..15 of lane group g hold keys 8g..8g+7 and
// 16+8g..16+8g+7, the 8 contiguous keys each PV k-group needs.
//
// When 128 does not divide n the last block holds fewer than 128 positions
// (kRagged): its K and V rows past n are read as copies of row n-1 (finite,
// and never weighted: every key past n lies past every real query), query
// rows past n are computed from row n-1 and not stored.

#include <type_traits>

#include "common.h"
#include "internal.h"

namespace crisp {

namespace {

constexpr int kStep = 64;              // keys per pipeline step
typedef __bf16 gcc_bf16x4 __attribute__((__vector_size__(8)));
typedef __attribute__((address_space(3))) gcc_bf16x4 lds_bf16x4;
constexpr int kKStages = 3;             // K tiles in flight: the next one is used, one more prefetched
constexpr float kSumLimit = 65536.f;     // a lane's step sum above this raises the running max

struct AttnArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const int32_t* count;
  const int32_t* idx;
  void* out;
  float* lse;
  int n;
  int nblk;
  int qpg;
  float scale_log2;
  int out_fp32;
  RowMap map;
  int* queue;  // 8 claim counters, zero at launch
  int items;   // Hq * nblk, or Hq * pairs of blocks for the two-block kernel
  // This kernel's pair of decision words, written by the decide pass (null:
  // no choice to make): the one-block kernels run unless two_block_pays
  // holds for them, the two-block kernel only if it does.
  const unsigned long long* sched;
};

// Key index (0..31) held by accumulator register v of lane group lg.
__device__ __forceinline__ int acc_key(int v, int lg) { return (v < 8) ? (8 * lg + v) : (16 + 8 * lg + (v - 8)); }

typedef __bf16 AttnLds[2 + kKStages][kStep * kHeadDim];
// The two-block kernel: the same five stages, then the merged list (tile 5)
// and the two blocks' list bitmaps (tile 6); after the main loop all eight
// tiles stage the 256 output rows.
typedef __bf16 PairLds[8][kStep * kHeadDim];
constexpr int kListTile = 5, kBitsTile = 6;
// Ownership bits of a merged-list entry (bit 16: block 2p lists the key
// block, bit 17: block 2p + 1 does); the key block is in bits 0-15.
constexpr int kOwnShift = 16;

__device__ __forceinline__ void wait_dma_but_2() { asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); }

// One item: (head, query block qb) with four waves, or with eight waves
// (kPair) the query blocks qb and qb + 1 of one head, which walk the union of
// their two lists together: every K/V tile is loaded once for both blocks,
// and a block's waves give weight zero to the steps of key blocks its own
// list does not hold.  Leaves LDS in use until its last read of the output
// staging; the caller synchronises before reusing it.
template <bool kDense, bool kRagged, bool kPair, typename LdsT, typename LoopEnd>
__device__ __forceinline__ void attend(const AttnArgs& p, LdsT& lds, int h, int qb, int w, LoopEnd&& loop_end) {
  auto kstage = [&](int i) -> __bf16* { return lds[2 + i]; };
  auto vstage = [&](int i) -> __bf16* { return lds[i]; };

  const int g = h / p.qpg;
  // w: the wave index (scalar).  The lane index comes from an asm statement
  // the compiler may not move: otherwise it computes every offset derived
  // from the thread index once, before the item loop, and keeps them all
  // live (and spilled) across it.
  const int lane = opaque_lane();
  const int tid = 64 * w + lane;
  const int l32 = lane & 31, lg = lane >> 5;
  // kPair: waves 0-3 serve block qb, waves 4-7 block qb + 1 (if it exists;
  // otherwise they compute rows past n from row n - 1 and store nothing).
  const int half = kPair ? (w >> 2) : 0;
  const int wq = kPair ? (w & 3) : w;
  const int qm = qb + half;
  const bool has_b = kPair && qb + 1 < p.nblk;

  const size_t nd = (size_t)p.n * kHeadDim;
  const __bf16* qh = p.q + (size_t)h * nd;
  const __bf16* kg = p.k + (size_t)g * nd;
  const __bf16* vg = p.v + (size_t)g * nd;

  // cnt: key blocks walked; last_e: the entry of the last one (which is
  // diagonal to the last query block).
  int cnt, last_e = qb;
  const int32_t* list = nullptr;
  const int32_t* ulist = nullptr;
  if (kPair && kDense) {
    // blocks 0 .. qb + 1: block qb + 1 lies after every row of block qb
    cnt = has_b ? qb + 2 : qb + 1;
    last_e = has_b ? (qb + 1) | (2 << kOwnShift) : qb | (1 << kOwnShift);
  } else if (kPair) {
    // Merge the two lists into one ascending list of distinct blocks with
    // ownership bits.  Each list is read as the one-block kernel reads it:
    // count clamped to [1, qq + 1], the last entry taken as qq, the others
    // clamped to [0, qq - 1].  So the merged list ends with qb, qb + 1, and
    // a repeated entry is walked once.
    uint32_t* bits = (uint32_t*)lds[kBitsTile];  // [2][128] words, then the merged count
    int32_t* ul = (int32_t*)lds[kListTile];
    if (tid < 256) bits[tid] = 0;
    __syncthreads();
    for (int b2 = 0; b2 < (has_b ? 2 : 1); ++b2) {
      const int qq = qb + b2;
      const int tc = min(max(p.count[(size_t)h * p.nblk + qq], 1), qq + 1);
      const int32_t* lq = p.idx + (size_t)h * ((size_t)p.nblk * (p.nblk + 1) / 2) + (size_t)qq * (qq + 1) / 2;
      for (int t = tid; t < tc; t += 512) {
        const int kb = t == tc - 1 ? qq : min(max(lq[t], 0), qq - 1);
        atomicOr(&bits[128 * b2 + (kb >> 5)], 1u << (kb & 31));
      }
    }
    __syncthreads();
    if (w == 0) {
      // lane l writes the set bits of words 2l and 2l + 1 at its offset in
      // the merged list (a prefix sum of the words' bit counts)
      const uint32_t a0 = bits[2 * lane], a1 = bits[2 * lane + 1];
      const uint32_t b0 = bits[128 + 2 * lane], b1 = bits[128 + 2 * lane + 1];
      const int c = __popc(a0 | b0) + __popc(a1 | b1);
      int incl = c;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
      }
      int pos = incl - c;
      auto emit = [&](uint32_t a, uint32_t b, int word) {
        uint32_t u = a | b;
        while (u) {
          const int bit = __builtin_ctz(u);
          u &= u - 1;
          ul[pos++] = (32 * word + bit) | (((a >> bit) & 1u) << kOwnShift) | (((b >> bit) & 1u) << (kOwnShift + 1));
        }
      };
      emit(a0, b0, 2 * lane);
      emit(a1, b1, 2 * lane + 1);
      if (lane == 63) bits[256] = incl;
    }
    __syncthreads();
    cnt = __builtin_amdgcn_readfirstlane(((const int*)bits)[256]);
    ulist = ul;
    last_e = __builtin_amdgcn_readfirstlane(ul[cnt - 1]);
  } else if (kDense) {
    cnt = qb + 1;
  } else {
    // A malformed count or entry is clamped so that reads stay inside the
    // head's rows 0 .. 128(qb+1)-1; well-formed lists are unaffected.
    cnt = min(max(p.count[(size_t)h * p.nblk + qb], 1), qb + 1);
    list = p.idx + (size_t)h * ((size_t)p.nblk * (p.nblk + 1) / 2) + (size_t)qb * (qb + 1) / 2;
  }
  const int nsteps = 2 * cnt;

  // Q rows as the B operand of K.Q^T: query row 32 wq + l32 of block qm,
  // d = 16kk + 8lg + [0, 8).
  const int qpos = qm * kBlock + 32 * wq + l32;
  const int qrow = (kRagged || kPair) ? min(qpos, p.n - 1) : qpos;
  bf16x8 qf[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk)
    qf[kk] = as_bf16x8(*(const u32x4*)(qh + (size_t)qrow * kHeadDim + 16 * kk + 8 * lg));

  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[db][v] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  // Global -> LDS by DMA (buffer_load ... lds): each wave instruction fills
  // 1 KiB of LDS, lane L at byte 16 L.  K and V tiles are stored row-major
  // (a 64-key step is 64 rows of 256 B) with the 16-byte chunk c of row r at
  // chunk position c ^ swz(r), one swizzle per tile (see swz_k, swz_v).
  // Wave w fills rows R w .. R w + R - 1 with R / 4 instructions (R = 16
  // with four waves, 8 with eight); lane L of instruction i writes row
  // r = R w + 4i + L/16 at position L & 15, so it loads global chunk
  // (L & 15) ^ swz(r) of that row.
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)kg, 0, (int)(nd * 2), kBufferFlags);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)vg, 0, (int)(nd * 2), kBufferFlags);
  // swz_v depends only on the row's bits 0-1 (lane / 16 here), so the V
  // offsets of a wave's instructions differ by exactly 1024 bytes; swz_k
  // also takes bits 2-3 and needs one offset per instruction.
  constexpr int kDmaPerTile = kPair ? 2 : 4;
  constexpr int kRowsPerWave = 4 * kDmaPerTile;
  constexpr int kDmaStride = 16 / kDmaPerTile;  // MFMAs between a wave's DMA instructions in the main loop
  int dma_k[kDmaPerTile];
#pragma unroll
  for (int i = 0; i < kDmaPerTile; ++i) {
    const int r = kRowsPerWave * w + 4 * i + (lane >> 4);
    dma_k[i] = r * 256 + (((lane & 15) ^ swz_k(r)) << 4);
  }
  const int dma_v = (kRowsPerWave * w + (lane >> 4)) * 256 + (((lane & 15) ^ swz_v(lane >> 4)) << 4);

  // List entries: 64 at a time in one VGPR (lane i holds entry c0 + i),
  // picked out with readlane; a chunk is reloaded only when a block past it
  // is needed.  The entry's whole byte offset goes in the lane offset, which
  // the buffer's range check covers, so entries past `cnt` read as 0.  The
  // last entry is taken as the diagonal block qb and every other entry is
  // clamped to [0, qb-1]: reads stay inside the head's rows, and only the
  // two masked steps of the diagonal block ever see a key past a query,
  // whatever the list holds.
  // kPair: the merged list sits in LDS; an entry carries the key block and
  // the two ownership bits, and the same readlane scheme picks it out.
  const __amdgpu_buffer_rsrc_t lrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)list, 0, (kDense || kPair) ? 0 : cnt * 4, kBufferFlags);
  int chunk_base = 0;
  int chunk = kDense ? 0 : kPair ? ulist[lane] : __builtin_amdgcn_raw_buffer_load_b32(lrs, lane * 4, 0, 0);
  auto block_at = [&](int b) -> int {
    if (kPair && kDense) {
      const int bb = min(b, cnt - 1);
      return bb | ((bb <= qb ? 1 : 0) << kOwnShift) | ((has_b ? 2 : 0) << kOwnShift);
    }
    if (kDense) return b;
    if (b >= cnt - 1) return last_e;
    if (kPair) {
      if (b - chunk_base >= 64) {
        chunk_base = b;
        chunk = ulist[b + lane];  // past the list's end: LDS tile 6, never picked
      }
      return __builtin_amdgcn_readlane(chunk, b - chunk_base);
    }
    if (b - chunk_base >= 64) {
      chunk_base = b;
      chunk = __builtin_amdgcn_raw_buffer_load_b32(lrs, (b + lane) * 4, 0, 0);
      // Wait here, in the rare reload (a full s_waitcnt the compiler sees),
      // so that no load of `chunk` is pending at the lookups: otherwise the
      // compiler puts a vmcnt(0) before every readlane below, and that wait
      // also drains the K/V DMA in flight, which it cannot see.
      __builtin_amdgcn_s_waitcnt(0);
    }
    return min(max(__builtin_amdgcn_readlane(chunk, b - chunk_base), 0), qb - 1);
  };
  auto kb_of = [](int e) -> int { return kPair ? (e & 0xffff) : e; };
  // Whether this wave's block lists the entry's key block (always, with one block).
  auto own_of = [&](int e) -> bool { return kPair ? ((e >> (kOwnShift + half)) & 1) != 0 : true; };
  auto key0_of = [&](int e, int step) -> int { return kb_of(e) * kBlock + (step & 1) * kStep; };

  // The DMA is issued through inline asm so that the compiler does not
  // track it: it would otherwise wait for every outstanding LDS DMA before
  // the first LDS read of each step, whatever stage that read touches.
  // Ordering is explicit instead: each step ends with a vmcnt wait covering
  // the tiles the next step reads, then a barrier.
  const int wu = __builtin_amdgcn_readfirstlane(w);
  // One DMA instruction: rows R wu + 4 i .. +3 of the tile of step `step`.
  // `off` is the lane's byte offset for i = 0 when `imm` is set: the
  // instruction's immediate offset (1024 i) then moves both the global read
  // and the LDS destination.  Otherwise `off` is the lane's offset for i.
  auto dma1 = [&](__amdgpu_buffer_rsrc_t rs, int off, __bf16* stage, int kb, int step, int i, bool imm) {
    const int key0 = key0_of(kb, step);
    int soff = key0 * (kHeadDim * 2);
    // one wait state between writing M0 and the DMA that reads it
#define CRISP_DMA(OFF)                                                                        \
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen offset:" #OFF " lds" \
               :                                                                              \
               : "s"(lds_addr), "v"(off), "s"(rs), "s"(soff)                                  \
               : "memory", "m0")
    if (kRagged && key0 + kStep > p.n) {
      // a tile past row n-1: the whole row offset goes to the lane, clamped
      // to the last row (the lane's 16-byte chunk within its row is kept)
      const int off_i = imm ? off + 1024 * i : off;
      const int r = kRowsPerWave * w + 4 * i + (lane >> 4);
      off = min(key0 + r, p.n - 1) * (kHeadDim * 2) + (off_i & 255);
      soff = 0;
      const unsigned lds_addr =
          (unsigned)(uintptr_t)(__attribute__((address_space(3))) void*)(stage + (kRowsPerWave * wu + 4 * i) *
                                                                                    kHeadDim);
      CRISP_DMA(0);
      return;
    }
    if (imm) {
      const unsigned lds_addr =
          (unsigned)(uintptr_t)(__attribute__((address_space(3))) void*)(stage + kRowsPerWave * wu * kHeadDim);
      switch (i) {
        case 0: CRISP_DMA(0); break;
        case 1: CRISP_DMA(1024); break;
        case 2: CRISP_DMA(2048); break;
        default: CRISP_DMA(3072); break;
      }
    } else {
      const unsigned lds_addr =
          (unsigned)(uintptr_t)(__attribute__((address_space(3))) void*)(stage + (kRowsPerWave * wu + 4 * i) *
                                                                                    kHeadDim);
      CRISP_DMA(0);
    }
#undef CRISP_DMA
  };
  auto dma_k_tile = [&](__bf16* stage, int kb, int step) {
#pragma unroll
    for (int i = 0; i < kDmaPerTile; ++i) dma1(krs, dma_k[i], stage, kb, step, i, false);
  };
  auto dma_v_tile = [&](__bf16* stage, int kb, int step) {
#pragma unroll
    for (int i = 0; i < kDmaPerTile; ++i) dma1(vrs, dma_v, stage, kb, step, i, true);
  };

  // Row of the K operand fed by this lane: a permutation of 0..31 (see top).
  const int ia = l32 >> 3, ig = (l32 >> 2) & 1, ib = l32 & 3;
  const int krow = 16 * (ia >> 1) + 8 * ig + 4 * (ia & 1) + ib;
  // Byte offsets, from the start of the K stages, of this lane's K operand:
  // row 32 kb2 + krow, logical chunk 2 kk + lg; kb2 leaves swz_k unchanged
  // (+8 KiB).
  constexpr int kKBase = 2 * kStep * kHeadDim * 2;  // bytes of the two V stages
  int k_off[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) k_off[kk] = kKBase + krow * 256 + (((2 * kk + lg) ^ swz_k(krow)) << 4);
  // V^T operand through the transposing LDS read: within each 16-lane group
  // (gq = lane / 16, li = lane % 16) lane li receives element li % 4 of the
  // 4-element vectors addressed by lanes 4e + li / 4 (e = 0..3).  A lane
  // addresses row k0 + li / 4, columns d0 + 4 (li % 4) .. +3, so it gets
  // keys k0 .. k0+3 at column d0 + li.  For the A operand of O^T += V^T P^T
  // (row d = 32 db + l32, keys 32 kb2 + 16 mm + 8 lg + s) two reads
  // (s = 0..3, hh = 0, and s = 4..7, hh = 1) give the 8 slots.  Rows differ
  // by 4 hh + 16 mm + 32 kb2, none of which changes swz_v, so one base
  // offset per db covers every read.
  const int gq = lane >> 4, li = lane & 15;
  int v_base[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    const int r = 8 * (gq >> 1) + (li >> 2);
    const int d = 32 * db + 16 * (gq & 1) + 4 * (li & 3);
    v_base[db] = r * 256 + (((d >> 3) ^ swz_v(r)) << 4) + (d & 7) * 2;
  }
  auto v_off = [&](int db, int kb2, int mm, int hh) -> int {
    return v_base[db] + (32 * kb2 + 16 * mm + 4 * hh) * 256;
  };

  // Scores of the step whose K tile is in stage kst.
  auto qk = [&](int kst, f32x16 (&s)[2]) {
    const char* kb8 = (const char*)lds + kst * (kStep * kHeadDim * 2);
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
      for (int v = 0; v < 16; ++v) s[kb2][v] = 0.f;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const bf16x8 kf = as_bf16x8(*(const u32x4*)(kb8 + k_off[kk] + kb2 * 8192));
        s[kb2] = mfma32(kf, qf[kk], s[kb2]);
      }
    }
  };

  // One key half (keys key0 + 32 kb2 .. +31) of a step's scores, with the
  // K operand read from global memory in the layout the LDS path gives.
  auto qk_half_global = [&](int key0, int kb2) -> f32x16 {
    const int kr = key0 + 32 * kb2 + krow;
    const __bf16* krow_g = kg + (size_t)(kRagged ? min(kr, p.n - 1) : kr) * kHeadDim + 8 * lg;
    f32x16 s = {};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) s = mfma32(as_bf16x8(*(const u32x4*)(krow_g + 16 * kk)), qf[kk], s);
    return s;
  };

  // Iteration j of the software pipeline.  K_t lives in K stage t % 3 and
  // V_t in V stage t & 1 (`kst_in` = (j + 1) % 3 and `vpar_in` = j & 1,
  // compile-time constants in the main loop so that LDS read offsets become
  // instruction immediates); S_j arrives in `sc` already masked.  Iteration j
  //   - block 1: S_{j+1} = K_{j+1} Q^T (MFMA) beside exp / row sum / bf16
  //     packing of the second key half of S_j (VALU) against the current
  //     running max, and the DMA of V_{j+1} over V_{j-1} (read in iteration
  //     j-1),
  //   - raises the running max and redoes the exps when they grew too large
  //     (rare branch; the running max only needs to keep probabilities in
  //     range, any value works for exactness),
  //   - block 2: O += V_j P_j (MFMA) beside masking of S_{j+1} and the exps
  //     of its first key half, and the DMA of K_{j+3} over K_j (read in
  //     iteration j-1),
  //   - waits for all of its DMA but the K_{j+3} one, which has until the
  //     end of iteration j+1, and meets the other waves at one barrier.
  // The 8 DMA instructions of a wave are spread one per four MFMAs: issued
  // together right after the barrier, the 32 of a workgroup queue up in the
  // CU's address unit and stall the waves' in-order issue.
  // kCurMasked / kNextMasked: step j / j+1 is one of the two steps of the
  // diagonal block (sorted lists put it last); kKAhead: there is a step j+3;
  // kNext: j+1 is a step.  kb_c, kb_v, kb_k, kb_n: key blocks of steps j,
  // j+1, j+3, j+1; kst: stage of K_{j+1}.
  float neg_m = 0.f;
  // First-key-half probabilities of the next step (bf16 operands) and their
  // row sum, computed one iteration ahead.
  bf16x8 p_lo[2];
  float ls_lo = 0.f;
  // Row max across the two half-waves holding a query's keys: with both
  // operands equal, permlane32_swap returns lane l's value and that of lane
  // l ^ 32 in its two results.
  auto pair_max = [](float x) -> float {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  };
  // Row max of a step's scores, scaled: t = s * scale_log2 (> 0 keeps the
  // order, so the max is taken before scaling).
  auto row_max = [&](const f32x16 (&s)[2]) -> float {
    float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
    for (int v = 2; v < 16; v += 2) mx = fmaxf(mx, fmaxf(s[0][v], s[0][v + 1]));
#pragma unroll
    for (int v = 0; v < 16; v += 2) mx = fmaxf(mx, fmaxf(s[1][v], s[1][v + 1]));
    return pair_max(mx) * p.scale_log2;
  };
  // Raises the running max to at least `mxs` (a scaled row max), rescaling
  // O and the row sum; used on the first step and whenever a step's
  // probabilities grow past kSumLimit.
  auto raise_to = [&](float mxs) {
    const float m_new = fmaxf(m_run, mxs);
    const float alpha = fast_exp2(m_run - m_new);  // 0 while m_run is -inf
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) o[db][v] *= alpha;
    l_run *= alpha;
    m_run = m_new;
    neg_m = -m_new;
  };
  auto mask_scores = [&](f32x16 (&s)[2], int key0) {
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (key0 + 32 * kb2 + acc_key(v, lg) > qpos) s[kb2][v] = -INFINITY;
  };

  auto iter = [&](int j, int kb_c, int kb_v, int kb_k, int kb_n, auto kst_in, auto vpar_in, f32x16 (&sc)[2],
                  f32x16 (&sn)[2], auto cur_masked_tag, auto k_ahead_tag, auto next_masked_tag, auto next_tag) {
    const int kst = kst_in, vpar = vpar_in;
    // compile-time tags in the main loops, run-time flags in the two-block tail
    const bool kCurMasked = cur_masked_tag;
    const bool kKAhead = k_ahead_tag;
    const bool kNextMasked = next_masked_tag;
    const bool kNext = next_tag;
    // Two blocks: a step of a key block this wave's list lacks weighs
    // nothing: its exponents are taken against an infinite running max.
    // (Its products still run: leaving them out, per instruction or per
    // iteration, measured slower.)
    const float nm_c = own_of(kb_c) ? neg_m : -INFINITY;
    __bf16* vdst = vstage(vpar ^ 1);
    __bf16* kdst = kstage(kst == 0 ? 2 : kst - 1);

    // The two blocks are written out in issue order, one unit per MFMA, with
    // operand reads three MFMAs ahead through 4-entry register rings;
    // sched_barrier(0) keeps the units as written.  The exps of a step are
    // split over both blocks so that every MFMA has about the same VALU work
    // beside it: scores 0..15 of S_{j+1} (its first key half) in block 2 of
    // iteration j, scores 16..31 in block 1 of iteration j+1.
    // Block 1: MFMA t of S_{j+1} (key half t & 1, d slice t / 2) beside the
    // exp, row sum and bf16 packing of score 16 + t of S_j.
    const char* kb8 = (const char*)lds + kst * (kStep * kHeadDim * 2);
    auto kread = [&](int t) -> bf16x8 {
      return as_bf16x8(*(const u32x4*)(kb8 + k_off[t >> 1] + (t & 1) * 8192));
    };
    bf16x8 kr[4];
    if (kNext) {
      kr[0] = kread(0);
      kr[1] = kread(1);
      kr[2] = kread(2);
    }
    float e[16];
    // P_j operand f = 2 * key half + 16-key group (keys 16 f + 8 lg .. +7);
    // pb[0], pb[1] come from the previous iteration.
    bf16x8 pb[4] = {p_lo[0], p_lo[1], {}, {}};
    float ls = ls_lo;
    const f32x16 zero = {};
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      if (kNext) {
        sn[t & 1] = mfma32(kr[t & 3], qf[t >> 1], t < 2 ? zero : sn[t & 1]);
        if (t + 3 < 16) kr[(t + 3) & 3] = kread(t + 3);
        if ((t & (kDmaStride - 1)) == 0) dma1(vrs, dma_v, vdst, kb_v, j + 1, t / kDmaStride, true);
      }
      e[t] = fast_exp2(fmaf(sc[1][t], p.scale_log2, nm_c));
      if (t & 1) {  // pack each pair as soon as it is complete
        pb[2 + (t >> 3)][(t & 7) - 1] = (__bf16)e[t - 1];
        pb[2 + (t >> 3)][t & 7] = (__bf16)e[t];
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    ls = sum_rounded(pb[3], sum_rounded(pb[2], ls));
    // The running max is only raised when it was too low for this step:
    // some lane's probabilities sum past kSumLimit (+inf included).  Every
    // probability then stays at most kSumLimit, far inside bf16 / fp32 range.
    // On the fully visible steps S_j is recomputed from K_j in global memory
    // (its LDS stage may already be refilled by waves in block 2), one key
    // half at a time, once for the max and once for the exps, so that its
    // first key half need not stay live; the two diagonal steps keep their
    // masked scores instead.
    if (__any(!(ls <= kSumLimit))) {
      const int key0c = key0_of(kb_c, j);
      float mx = -INFINITY;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        const f32x16 sr = kCurMasked ? sc[kb2] : qk_half_global(key0c, kb2);
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sr[v]);
      }
      raise_to(pair_max(mx) * p.scale_log2);
      ls = 0.f;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        const f32x16 sr = kCurMasked ? sc[kb2] : qk_half_global(key0c, kb2);
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          float x[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) x[i] = fast_exp2(fmaf(sr[8 * f + i], p.scale_log2, neg_m));
          pb[2 * kb2 + f] = pack_bf16x8(x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]);
          ls = sum_rounded(pb[2 * kb2 + f], ls);
        }
      }
    }
    l_run += ls;

    // Block 2: MFMA u of O += V_j P_j (d slice u & 3, P operand u / 4) beside
    // masking of scores 2u, 2u+1 of S_{j+1} and the exp, row sum and packing
    // of its score u.
    __attribute__((address_space(3))) char* vb8 = (__attribute__((address_space(3))) char*)vstage(vpar);
    auto vread = [&](int u) -> bf16x8 {
      const int db = u & 3, f = u >> 2;
      const bf16x4 lo = __builtin_bit_cast(
          bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vb8 + v_off(db, f >> 1, f & 1, 0))));
      const bf16x4 hi = __builtin_bit_cast(
          bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vb8 + v_off(db, f >> 1, f & 1, 1))));
      return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    bf16x8 vr[4];
    vr[0] = vread(0);
    vr[1] = vread(1);
    vr[2] = vread(2);
    const int key0n = kNextMasked ? key0_of(kb_n, j + 1) : 0;
    const float nm_n = own_of(kb_n) ? neg_m : -INFINITY;
    float lsn = 0.f;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      o[u & 3] = mfma32(vr[u & 3], pb[u >> 2], o[u & 3]);
      if (u + 3 < 16) vr[(u + 3) & 3] = vread(u + 3);
      if (kKAhead && (u & (kDmaStride - 1)) == 0)
        dma1(krs, dma_k[u / kDmaStride], kdst, kb_k, j + 3, u / kDmaStride, false);
      if (kNext) {
        if (kNextMasked) {
          const int kbase = key0n + 32 * (u >> 3);
          if (kbase + acc_key((2 * u) & 15, lg) > qpos) sn[u >> 3][(2 * u) & 15] = -INFINITY;
          if (kbase + acc_key((2 * u + 1) & 15, lg) > qpos) sn[u >> 3][(2 * u + 1) & 15] = -INFINITY;
        }
        e[u] = fast_exp2(fmaf(sn[0][u], p.scale_log2, nm_n));
        if (u & 1) {
          p_lo[u >> 3][(u & 7) - 1] = (__bf16)e[u - 1];
          p_lo[u >> 3][u & 7] = (__bf16)e[u];
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (kNext) lsn = sum_rounded(p_lo[1], sum_rounded(p_lo[0], lsn));
    ls_lo = lsn;

    if (kKAhead) {
      if (kPair)
        wait_dma_but_2();
      else
        wait_dma_but_4();
    } else {
      wait_dma();
    }
    __syncthreads();
  };

  f32x16 sa[2], sb[2];
  int kb_cur = block_at(0), kb_nxt = block_at(1), kb_nn = block_at(2);
  dma_k_tile(kstage(0), kb_cur, 0);
  dma_v_tile(vstage(0), kb_cur, 0);
  dma_k_tile(kstage(1), kb_cur, 1);
  if (nsteps > 2) dma_k_tile(kstage(2), kb_nxt, 2);
  wait_dma();
  __syncthreads();
  qk(0, sa);
  if (kPair ? nsteps <= 4 : nsteps == 2) mask_scores(sa, key0_of(kb_cur, 0));
  raise_to(row_max(sa));
  const float nm0 = own_of(kb_cur) ? neg_m : -INFINITY;
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    float x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = fast_exp2(fmaf(sa[0][8 * f + i], p.scale_log2, nm0));
    p_lo[f] = pack_bf16x8(x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]);
    ls_lo = sum_rounded(p_lo[f], ls_lo);
  }
  __syncthreads();  // every wave has read K_0 before iteration 0 overwrites it

  // Steps 0 .. nsteps-3 cover the fully visible blocks, the last two the
  // diagonal block.  The main loop runs the iterations whose next step is
  // fully visible six at a time (3 K stages x 2 V stages / score buffers,
  // so every stage is known at compile time), a pair loop runs the 0-2
  // remaining pairs, and the tail runs the last four iterations (two when
  // the list holds only the diagonal block).
  using F = std::false_type;
  using T = std::true_type;
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  int j = 0, kst = 1;
  if constexpr (kPair) {
    // Two blocks: each of the last two key blocks (the last four steps) is
    // diagonal or past the rows for one of them.  The causal mask is exact
    // wherever it is applied, so it is applied to those four steps for both
    // blocks.  The same main and pair loops as below stop six steps short;
    // the tail takes its flags at run time.
    for (; j + 6 <= nsteps - 6; j += 6) {
      const int kb3 = block_at((j >> 1) + 3), kb4 = block_at((j >> 1) + 4);
      iter(j, kb_cur, kb_cur, kb_nxt, kb_cur, S1{}, S0{}, sa, sb, F{}, T{}, F{}, T{});
      iter(j + 1, kb_cur, kb_nxt, kb_nn, kb_nxt, S2{}, S1{}, sb, sa, F{}, T{}, F{}, T{});
      iter(j + 2, kb_nxt, kb_nxt, kb_nn, kb_nxt, S0{}, S0{}, sa, sb, F{}, T{}, F{}, T{});
      iter(j + 3, kb_nxt, kb_nn, kb3, kb_nn, S1{}, S1{}, sb, sa, F{}, T{}, F{}, T{});
      iter(j + 4, kb_nn, kb_nn, kb3, kb_nn, S2{}, S0{}, sa, sb, F{}, T{}, F{}, T{});
      iter(j + 5, kb_nn, kb3, kb4, kb3, S0{}, S1{}, sb, sa, F{}, T{}, F{}, T{});
      kb_cur = kb3;
      kb_nxt = kb4;
      kb_nn = block_at((j >> 1) + 5);
    }
    for (; j < nsteps - 6; j += 2) {
      iter(j, kb_cur, kb_cur, kb_nxt, kb_cur, kst, 0, sa, sb, F{}, T{}, F{}, T{});
      kst = kst == 2 ? 0 : kst + 1;
      iter(j + 1, kb_cur, kb_nxt, kb_nn, kb_nxt, kst, 1, sb, sa, F{}, T{}, F{}, T{});
      kst = kst == 2 ? 0 : kst + 1;
      kb_cur = kb_nxt;
      kb_nxt = kb_nn;
      kb_nn = block_at((j >> 1) + 3);
    }
    for (; j < nsteps; j += 2) {
      iter(j, kb_cur, kb_cur, kb_nxt, kb_cur, kst, 0, sa, sb, j >= nsteps - 4, j + 3 < nsteps, j + 1 >= nsteps - 4,
           true);
      kst = kst == 2 ? 0 : kst + 1;
      iter(j + 1, kb_cur, kb_nxt, kb_nn, kb_nxt, kst, 1, sb, sa, j + 1 >= nsteps - 4, j + 4 < nsteps,
           j + 2 >= nsteps - 4, j + 2 < nsteps);
      kst = kst == 2 ? 0 : kst + 1;
      kb_cur = kb_nxt;
      kb_nxt = kb_nn;
      kb_nn = block_at((j >> 1) + 3);
    }
  } else {
    if (nsteps >= 4) {
      for (; j + 6 <= nsteps - 4; j += 6) {
        // blocks of steps j .. j+8: kb_cur (j, j+1), kb_nxt (j+2, j+3), kb_nn (j+4, j+5), then two more
        const int kb3 = block_at((j >> 1) + 3), kb4 = block_at((j >> 1) + 4);
        iter(j, kb_cur, kb_cur, kb_nxt, kb_cur, S1{}, S0{}, sa, sb, F{}, T{}, F{}, T{});
        iter(j + 1, kb_cur, kb_nxt, kb_nn, kb_nxt, S2{}, S1{}, sb, sa, F{}, T{}, F{}, T{});
        iter(j + 2, kb_nxt, kb_nxt, kb_nn, kb_nxt, S0{}, S0{}, sa, sb, F{}, T{}, F{}, T{});
        iter(j + 3, kb_nxt, kb_nn, kb3, kb_nn, S1{}, S1{}, sb, sa, F{}, T{}, F{}, T{});
        iter(j + 4, kb_nn, kb_nn, kb3, kb_nn, S2{}, S0{}, sa, sb, F{}, T{}, F{}, T{});
        iter(j + 5, kb_nn, kb3, kb4, kb3, S0{}, S1{}, sb, sa, F{}, T{}, F{}, T{});
        kb_cur = kb3;
        kb_nxt = kb4;
        kb_nn = block_at((j >> 1) + 5);
      }
      for (; j < nsteps - 4; j += 2) {
        iter(j, kb_cur, kb_cur, kb_nxt, kb_cur, kst, 0, sa, sb, F{}, T{}, F{}, T{});
        kst = kst == 2 ? 0 : kst + 1;
        iter(j + 1, kb_cur, kb_nxt, kb_nn, kb_nxt, kst, 1, sb, sa, F{}, T{}, F{}, T{});
        kst = kst == 2 ? 0 : kst + 1;
        kb_cur = kb_nxt;
        kb_nxt = kb_nn;
        kb_nn = block_at((j >> 1) + 3);
      }
      // j = nsteps - 4: kb_cur is the last fully visible block, kb_nxt the diagonal one
      iter(j, kb_cur, kb_cur, kb_nxt, kb_cur, kst, 0, sa, sb, F{}, T{}, F{}, T{});
      kst = kst == 2 ? 0 : kst + 1;
      iter(j + 1, kb_cur, kb_nxt, kb_nxt, kb_nxt, kst, 1, sb, sa, F{}, F{}, T{}, T{});
      kst = kst == 2 ? 0 : kst + 1;
      j += 2;
      kb_cur = kb_nxt;
    }
    iter(j, kb_cur, kb_cur, kb_cur, kb_cur, kst, 0, sa, sb, T{}, F{}, T{}, T{});
    kst = kst == 2 ? 0 : kst + 1;
    iter(j + 1, kb_cur, kb_cur, kb_cur, kb_cur, kst, 1, sb, sa, T{}, F{}, F{}, F{});
  }

  loop_end();
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.f / l_tot;
  // The output goes through LDS (the K/V stages are idle after the last
  // barrier): each lane writes its row's values with 16-byte chunks
  // XOR-swizzled by the row, then the workgroup stores whole rows, a 16-byte
  // chunk per lane, consecutive lanes along a row.
  // With two blocks the 256 rows of blocks qb, qb + 1 are contiguous in out.
  constexpr int kRows = kPair ? 2 * kBlock : kBlock;
  constexpr int kThreads = kPair ? 512 : 256;
  constexpr bool kRowCheck = kRagged || kPair;
  char* ob = (char*)lds;
  const int orow_l = 32 * w + l32;  // row within the item's rows
  const size_t obase = ((size_t)h * p.n + (size_t)qb * kBlock) * kHeadDim;
  const int rows_out = kRowCheck ? min(kRows, p.n - qb * kBlock) : kRows;  // rows inside [0, n)
  if (p.out_fp32) {  // 512-byte rows, 32 chunks of 4 values
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        f32x4 r;
        r[0] = o[db][4 * a + 0] * inv;
        r[1] = o[db][4 * a + 1] * inv;
        r[2] = o[db][4 * a + 2] * inv;
        r[3] = o[db][4 * a + 3] * inv;
        const int c = 8 * db + 2 * a + lg;
        *(f32x4*)(ob + orow_l * 512 + ((c ^ (orow_l & 31)) << 4)) = r;
      }
    __syncthreads();
    float* out = (float*)p.out + obase;
#pragma unroll
    for (int i = 0; i < kRows * 32 / kThreads; ++i) {
      const int id = i * kThreads + tid, row = id >> 5, c = id & 31;
      if (!kRowCheck || row < rows_out)
        *(f32x4*)(out + row * kHeadDim + 4 * c) = *(const f32x4*)(ob + row * 512 + ((c ^ (row & 31)) << 4));
    }
  } else {  // 256-byte rows, 16 chunks of 8 values; a lane holds half a chunk
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        bf16x4 r;
        r[0] = (__bf16)(o[db][4 * a + 0] * inv);
        r[1] = (__bf16)(o[db][4 * a + 1] * inv);
        r[2] = (__bf16)(o[db][4 * a + 2] * inv);
        r[3] = (__bf16)(o[db][4 * a + 3] * inv);
        const int c = 4 * db + a;
        *(bf16x4*)(ob + orow_l * 256 + ((c ^ (orow_l & 15)) << 4) + 8 * lg) = r;
      }
    __syncthreads();
    __bf16* out = (__bf16*)p.out + obase;
#pragma unroll
    for (int i = 0; i < kRows * 16 / kThreads; ++i) {
      const int id = i * kThreads + tid, row = id >> 4, c = id & 15;
      if (!kRowCheck || row < rows_out)
        *(u32x4*)(out + row * kHeadDim + 8 * c) = *(const u32x4*)(ob + row * 256 + ((c ^ (row & 15)) << 4));
    }
  }
  if (p.lse != nullptr && lg == 0 && (!kRowCheck || qpos < p.n))
    p.lse[(size_t)h * p.n + qpos] = (m_run + fast_log2(l_tot)) * kLn2;
}

// Persistent workgroups (two per CU, or one with two blocks per item) take
// items from eight queues.  Queue x holds the item ids x, x+8, x+16, ... in
// increasing order, which the row map lays out so that the heads of a KV group
// stream the same K/V blocks side by side; a workgroup serves the queue of the
// XCD it runs on (so those heads share that XCD's L2) and, once it is empty,
// the others in turn.  Claiming items one at a time keeps every slot busy
// whatever the spread of list lengths: the hardware dispatcher, which places
// workgroups in order, leaves CUs idle behind a slow one, and XCDs that run
// slower than the rest hand their last items to the others.  The next item is
// claimed when the current one's main loop ends, so the claim's latency hides
// behind the output and items start in the order their slots free up, as under
// hardware dispatch.  (Claiming it when the current item starts reorders the
// items: heads of a group then stream their blocks further apart, which
// measured 2.6 times the L2 misses and a 5% lower clock.)  Every workgroup
// leaves once all eight counters have passed their queue ends.
template <bool kDense, bool kRagged, bool kPair, bool kRuns = false, typename LdsT>
__device__ __forceinline__ void run_items(const AttnArgs& p, LdsT& lds) {
  // The next item id passes through the first word of V stage 1, which an
  // item's first writes (list bitmaps and merged list, K stages 0-2 and V
  // stage 0) leave alone.
  int* const next_slot = (int*)lds[1];
  // Wave 0 claims (its first lane issues the atomic); the claim state is
  // wave-uniform and stays in scalar registers.
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const bool claimer = wave == 0;
  // The dispatcher deals workgroups to the XCDs round-robin, so workgroup b
  // runs on XCD b mod 8 and starts with that XCD's queue.
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
  if (claimer) {
    const int first = claim();
    if (opaque_lane() == 0) next_slot[0] = first;
  }
  __syncthreads();
  int item = next_slot[0];
  while (item >= 0) {
    int next = -1;
    int h, qb;
    map_row(p.map, item, &h, &qb);  // with two blocks: the pair index
    if constexpr (kRuns) qb = runs_of_16(qb, p.nblk);
    attend<kDense, kRagged, kPair>(p, lds, h, kPair ? 2 * qb : qb, wave, [&] {
      if (claimer) next = claim();
    });
    __syncthreads();
    if (claimer && opaque_lane() == 0) next_slot[0] = next;
    __syncthreads();
    item = next_slot[0];
  }
}

// Whether a launch runs the two-block kernel.  Walking the union of the
// lists of blocks 2p and 2p + 1 costs both blocks' waves one step per union
// block: 2U steps where the one-block kernel takes cA + cB.  In exchange each
// K/V tile is loaded once for both, which makes a step about 3.5% cheaper
// (dense causal attention at 512k: 1,747 -> 1,710 ms).  U is at most
// min(cA + cB, 2p + 2); with own = sum of cA + cB and bound = sum of that
// bound over the pairs, the two-block kernel runs when 2 bound <= 1.035 own.
// Dense lists of 32 blocks or more and near-dense ones meet this; lists
// that leave out a few percent of their blocks do not (pooled-estimation
// lists at gamma 0.95 measured no faster with two blocks: 3.8% more steps).
__host__ __device__ inline bool two_block_pays(unsigned long long own, unsigned long long bound) {
  return 2000ull * bound <= 1035ull * own;
}

// One-block kernel: four waves per (head, query block) item, two
// workgroups per CU.  A launch that the schedule hands to another kernel
// ends here.
template <bool kDense, bool kRagged>
__global__ __launch_bounds__(256, 2) void fa_fwd_kernel(AttnArgs p) {
  // 32 KiB of V stages (tiles 0-1) then 48 KiB of K stages (tiles 2-4): two
  // workgroups fill a CU's 160 KiB.  With V first, every stage offset of a
  // statically known stage fits the 16-bit immediate of an LDS read.
  __shared__ __attribute__((aligned(1024))) AttnLds lds;
  if (p.sched != nullptr && two_block_pays(p.sched[0], p.sched[1])) return;
  run_items<kDense, kRagged, false>(p, lds);
}

// The one-block kernel for short lists (64 listed tiles or fewer per item
// on average, as forced Vertical-Slash lists): the same items dealt to the
// XCDs in runs of 16 adjacent query blocks, so that the slash tiles of
// neighbouring blocks (shifted by one block from one to the next) meet in
// one L2 (19% fewer bytes fetched past L2 and 1.9% faster at 512k).  Long
// lists keep the interleaved deal: with runs, the items of an XCD stream
// the same tiles at the same moment, and a route-auto launch ran 7% slower.
template <bool kRagged>
__global__ __launch_bounds__(256, 2) void fa_runs_kernel(AttnArgs p) {
  __shared__ __attribute__((aligned(1024))) AttnLds lds;
  if (p.sched != nullptr && two_block_pays(p.sched[0], p.sched[1])) return;
  run_items<false, kRagged, false, true>(p, lds);
}

// The same scheduler over (head, pair of query blocks) items, one
// eight-wave workgroup per CU with 128 KiB of LDS.
template <bool kDense, bool kRagged>
__global__ __launch_bounds__(512, 1) void fa_pair_kernel(AttnArgs p) {
  __shared__ __attribute__((aligned(1024))) PairLds lds;
  if (p.sched != nullptr && !two_block_pays(p.sched[0], p.sched[1])) return;
  run_items<kDense, kRagged, true>(p, lds);
}

// Sums of the schedule choice over every (head, pair) item, with the counts
// clamped as the kernels read them.
__global__ __launch_bounds__(256) void sched_kernel(const int32_t* count, int hq, int nblk, unsigned long long* sums) {
  const int pairs = (nblk + 1) / 2;
  unsigned long long own = 0, bound = 0;
  for (int i = blockIdx.x * 256 + threadIdx.x; i < hq * pairs; i += gridDim.x * 256) {
    const int h = i / pairs, qa = 2 * (i - h * pairs);
    const int ca = min(max(count[(size_t)h * nblk + qa], 1), qa + 1);
    int cb = 0, u = ca;
    if (qa + 1 < nblk) {
      cb = min(max(count[(size_t)h * nblk + qa + 1], 1), qa + 2);
      u = min(ca + cb, qa + 2);
    }
    own += (unsigned long long)(ca + cb);
    bound += (unsigned long long)u;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    own += __shfl_xor(own, o);
    bound += __shfl_xor(bound, o);
  }
  // one pair of atomics per workgroup: those on one address serialise
  __shared__ unsigned long long part[2][4];
  if ((threadIdx.x & 63) == 0) {
    part[0][threadIdx.x >> 6] = own;
    part[1][threadIdx.x >> 6] = bound;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    atomicAdd(sums, part[0][0] + part[0][1] + part[0][2] + part[0][3]);
    atomicAdd(sums + 1, part[1][0] + part[1][1] + part[1][2] + part[1][3]);
  }
}

// Clears the 8 claim counters (words 0-7) and the schedule sums (words 16-19).
__global__ void clear_queue_kernel(int* queue) {
  if (threadIdx.x < 20) queue[threadIdx.x] = 0;
}

// One schedule for a sparse call, from the sums: each attention kernel reads
// its own pair of words through the test it applies to the sums (the
// one-block kernels run unless two_block_pays holds, the two-block kernel
// only if it does), so exactly one of them takes the items.
__global__ void decide_kernel(unsigned long long* sums, int items, int nblk) {
  if (threadIdx.x != 0) return;
  const unsigned long long own = sums[0], bound = sums[1];
  const bool two = two_block_pays(own, bound);
  const bool runs = !two && own <= 64ull * (unsigned long long)items && nblk % 128 == 0;
  const unsigned long long go[2] = {0ull, 1ull}, stop[2] = {1ull, 0ull};  // for the one-block test
  unsigned long long* d = sums + 2;  // [two-block][one-block][runs], two words each
  d[0] = two ? stop[0] : go[0];      // two_block_pays(1, 0) holds: the two-block kernel runs
  d[1] = two ? stop[1] : go[1];
  d[2] = (!two && !runs) ? go[0] : stop[0];
  d[3] = (!two && !runs) ? go[1] : stop[1];
  d[4] = runs ? go[0] : stop[0];
  d[5] = runs ? go[1] : stop[1];
}

}  // namespace

hipError_t launch_attention(const __bf16* q, const __bf16* k, const __bf16* v, const int32_t* count,
                            const int32_t* idx, void* out, int out_fp32, float* lse, int hq, int hkv, int n,
                            float scale, bool dense, int* queue, hipStream_t stream) {
  AttnArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.count = count;
  a.idx = idx;
  a.out = out;
  a.lse = lse;
  a.n = n;
  a.nblk = nblocks(n);
  a.qpg = hq / hkv;
  a.scale_log2 = scale * kLog2e;
  a.out_fp32 = out_fp32;
  a.map = make_row_map(hq, hkv, a.nblk);
  a.queue = queue;
  a.items = hq * a.nblk;
  a.sched = nullptr;
  const int pairs = (a.nblk + 1) / 2;
  AttnArgs b = a;  // the two-block kernel's items: (head, pair of blocks)
  b.map = make_row_map(hq, hkv, pairs);
  b.items = hq * pairs;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  cus = max(cus, 1);
  const unsigned grid = (unsigned)min(a.items, 2 * cus);
  const unsigned grid2 = (unsigned)min(b.items, cus);
  hipLaunchKernelGGL(clear_queue_kernel, dim3(1), dim3(64), 0, stream, queue);
  const bool ragged = n % kBlock != 0;
  bool one = true, two = true;
  if (dense) {
    // the rule the schedule pass applies to full lists, evaluated here
    unsigned long long own = 0, bound = 0;
    for (int pi = 0; pi < pairs; ++pi) {
      const int qa = 2 * pi;
      const bool hb = qa + 1 < a.nblk;
      own += (unsigned long long)(qa + 1 + (hb ? qa + 2 : 0));
      bound += (unsigned long long)(hb ? qa + 2 : qa + 1);
    }
    two = two_block_pays(own, bound);
    one = !two;
  } else {
    unsigned long long* sums = (unsigned long long*)(queue + 16);
    const int sblocks = (int)min(64LL, ((long long)b.items + 255) / 256);
    hipLaunchKernelGGL(sched_kernel, dim3(sblocks), dim3(256), 0, stream, count, hq, a.nblk, sums);
    hipLaunchKernelGGL(decide_kernel, dim3(1), dim3(64), 0, stream, sums, a.items, a.nblk);
    b.sched = sums + 2;
    a.sched = sums + 4;
  }
  if (two) {
    if (dense && ragged)
      hipLaunchKernelGGL((fa_pair_kernel<true, true>), dim3(grid2), dim3(512), 0, stream, b);
    else if (dense)
      hipLaunchKernelGGL((fa_pair_kernel<true, false>), dim3(grid2), dim3(512), 0, stream, b);
    else if (ragged)
      hipLaunchKernelGGL((fa_pair_kernel<false, true>), dim3(grid2), dim3(512), 0, stream, b);
    else
      hipLaunchKernelGGL((fa_pair_kernel<false, false>), dim3(grid2), dim3(512), 0, stream, b);
  }
  if (one) {
    if (dense && ragged)
      hipLaunchKernelGGL((fa_fwd_kernel<true, true>), dim3(grid), dim3(256), 0, stream, a);
    else if (dense)
      hipLaunchKernelGGL((fa_fwd_kernel<true, false>), dim3(grid), dim3(256), 0, stream, a);
    else if (ragged)
      hipLaunchKernelGGL((fa_fwd_kernel<false, true>), dim3(grid), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((fa_fwd_kernel<false, false>), dim3(grid), dim3(256), 0, stream, a);
  }
  if (!dense && a.nblk % 128 == 0) {
    AttnArgs r = a;
    r.sched = a.sched + 2;  // the runs decision
    if (ragged)
      hipLaunchKernelGGL((fa_runs_kernel<true>), dim3(grid), dim3(256), 0, stream, r);
    else
      hipLaunchKernelGGL((fa_runs_kernel<false>), dim3(grid), dim3(256), 0, stream, r);
  }
  return hipGetLastError();
}

}  // namespace crisp
