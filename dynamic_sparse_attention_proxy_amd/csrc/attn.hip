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

#include <type_traits>

#include "common.h"
#include "internal.h"

namespace crisp {

namespace {

constexpr int kStep = 64;              // keys per pipeline step
constexpr int kKsStride = kHeadDim + 8; // bf16 per K row in LDS (16 B pad)
constexpr int kVtStride = kStep + 8;    // bf16 per V^T row in LDS (16 B pad)
constexpr float kHeadroom = 8.f;        // log2 slack before the running max is raised

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
};

// Key index (0..31) held by accumulator register v of lane group lg.
__device__ __forceinline__ int acc_key(int v, int lg) { return (v < 8) ? (8 * lg + v) : (16 + 8 * lg + (v - 8)); }

template <bool kDense>
__global__ __launch_bounds__(256, 2) void fa_fwd_kernel(AttnArgs p) {
  __shared__ __attribute__((aligned(16))) __bf16 ks[2][kStep * kKsStride];
  __shared__ __attribute__((aligned(16))) __bf16 vt[2][kHeadDim * kVtStride];

  int h, qb;
  map_row(p.map, blockIdx.x, &h, &qb);
  const int g = h / p.qpg;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, lg = lane >> 5;

  const size_t nd = (size_t)p.n * kHeadDim;
  const __bf16* qh = p.q + (size_t)h * nd;
  const __bf16* kg = p.k + (size_t)g * nd;
  const __bf16* vg = p.v + (size_t)g * nd;

  int cnt;
  const int32_t* list = nullptr;
  if (kDense) {
    cnt = qb + 1;
  } else {
    // A malformed count or entry is clamped so that reads stay inside the
    // head's rows 0 .. 128(qb+1)-1; well-formed lists are unaffected.
    cnt = min(max(p.count[(size_t)h * p.nblk + qb], 1), qb + 1);
    list = p.idx + (size_t)h * ((size_t)p.nblk * (p.nblk + 1) / 2) + (size_t)qb * (qb + 1) / 2;
  }
  const int nsteps = 2 * cnt;

  // Q rows as the B operand of K.Q^T: query row 32w + l32, d = 16kk + 8lg + [0, 8).
  const int qpos = qb * kBlock + 32 * w + l32;
  bf16x8 qf[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk)
    qf[kk] = as_bf16x8(*(const u32x4*)(qh + (size_t)qpos * kHeadDim + 16 * kk + 8 * lg));

  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[db][v] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  // Global -> register staging of one step.
  // K: 64 rows x 16 chunks of 16 B; thread takes chunks tid + 256 i.
  // V: thread takes a 4-key x 8-d sub-block (keys 4*kq.., d 8*dc..).
  const int kq = tid >> 4, dc = tid & 15;
  u32x4 kreg[4], vreg[4];

  auto step_key0 = [&](int step) -> int {
    const int kb = kDense ? (step >> 1) : min(max(list[step >> 1], 0), qb);
    return kb * kBlock + (step & 1) * kStep;
  };

  auto load_step = [&](int step) {
    const int key0 = step_key0(step);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i;
      const int row = c >> 4, col = (c & 15) * 8;
      kreg[i] = *(const u32x4*)(kg + (size_t)(key0 + row) * kHeadDim + col);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) vreg[i] = *(const u32x4*)(vg + (size_t)(key0 + 4 * kq + i) * kHeadDim + 8 * dc);
  };

  auto store_step = [&](int stage) {
    __bf16* kdst = ks[stage];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i;
      const int row = c >> 4, col = (c & 15) * 8;
      *(u32x4*)(kdst + row * kKsStride + col) = kreg[i];
    }
    __bf16* vdst = vt[stage];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // d = 8dc + 2j (low halves) and 8dc + 2j + 1 (high halves) of keys 4kq..4kq+3
      u32x2 ev, od;
      ev[0] = (vreg[0][j] & 0xffffu) | (vreg[1][j] << 16);
      ev[1] = (vreg[2][j] & 0xffffu) | (vreg[3][j] << 16);
      od[0] = (vreg[0][j] >> 16) | (vreg[1][j] & 0xffff0000u);
      od[1] = (vreg[2][j] >> 16) | (vreg[3][j] & 0xffff0000u);
      *(u32x2*)(vdst + (8 * dc + 2 * j) * kVtStride + 4 * kq) = ev;
      *(u32x2*)(vdst + (8 * dc + 2 * j + 1) * kVtStride + 4 * kq) = od;
    }
  };

  // Row of the K operand fed by this lane: a permutation of 0..31 (see top).
  const int ia = l32 >> 3, ig = (l32 >> 2) & 1, ib = l32 & 3;
  const int krow = 16 * (ia >> 1) + 8 * ig + 4 * (ia & 1) + ib;

  // One pipeline step: keys key0 .. key0+63 from LDS stage `cur`, while the
  // next step's tiles are in flight to registers.  kMasked is only used for
  // the two steps of the diagonal block, which sorted lists put last.
  auto do_step = [&](int step, auto masked_tag) {
    constexpr bool kMasked = decltype(masked_tag)::value;
    const int cur = step & 1;
    const bool more = step + 1 < nsteps;
    if (more) load_step(step + 1);

    const int key0 = step_key0(step);
    const __bf16* kbuf = ks[cur];
    const __bf16* vbuf = vt[cur];

    f32x16 s[2];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
      for (int v = 0; v < 16; ++v) s[kb2][v] = 0.f;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const bf16x8 kf = as_bf16x8(*(const u32x4*)(kbuf + (32 * kb2 + krow) * kKsStride + 16 * kk + 8 * lg));
        s[kb2] = mfma32(kf, qf[kk], s[kb2]);
      }
    }

    if (kMasked) {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (key0 + 32 * kb2 + acc_key(v, lg) > qpos) s[kb2][v] = -INFINITY;
    }

    // Online softmax in base 2 on raw scores: t = s * scale_log2 (> 0 keeps
    // the order, so the row max is taken before scaling).  The running max
    // is only raised when a score exceeds it by more than kHeadroom, so
    // rescaling the accumulator is rare; probabilities stay below
    // 2^kHeadroom, well inside bf16 and fp32 range.
    float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
    for (int v = 2; v < 16; v += 2) mx = fmaxf(mx, fmaxf(s[0][v], s[0][v + 1]));
#pragma unroll
    for (int v = 0; v < 16; v += 2) mx = fmaxf(mx, fmaxf(s[1][v], s[1][v + 1]));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mxs = mx * p.scale_log2;
    if (__any(mxs > m_run + kHeadroom)) {
      const float m_new = fmaxf(m_run, mxs);
      const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[db][v] *= alpha;
      m_run = m_new;
    }
    const float neg_m = (m_run == -INFINITY) ? 0.f : -m_run;

    bf16x8 pb[2][2];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      float e[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        e[v] = fast_exp2(fmaf(s[kb2][v], p.scale_log2, neg_m));
        l_run += e[v];
      }
      pb[kb2][0] = pack_bf16x8(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]);
      pb[kb2][1] = pack_bf16x8(e[8], e[9], e[10], e[11], e[12], e[13], e[14], e[15]);
    }

#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const __bf16* vrow = vbuf + (32 * db + l32) * kVtStride + 8 * lg;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
          const bf16x8 vf = as_bf16x8(*(const u32x4*)(vrow + 32 * kb2 + 16 * mm));
          o[db] = mfma32(vf, pb[kb2][mm], o[db]);
        }
    }

    if (more) store_step(cur ^ 1);
    __syncthreads();
  };

  load_step(0);
  store_step(0);
  __syncthreads();
  // every block but the last (the diagonal) is fully visible to all rows
  for (int step = 0; step < nsteps - 2; ++step) do_step(step, std::false_type{});
  do_step(nsteps - 2, std::true_type{});
  do_step(nsteps - 1, std::true_type{});

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.f / l_tot;
  const size_t orow = ((size_t)h * p.n + qpos) * kHeadDim;
  if (p.out_fp32) {
    float* out = (float*)p.out + orow;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        f32x4 r;
        r[0] = o[db][4 * a + 0] * inv;
        r[1] = o[db][4 * a + 1] * inv;
        r[2] = o[db][4 * a + 2] * inv;
        r[3] = o[db][4 * a + 3] * inv;
        *(f32x4*)(out + 32 * db + 8 * a + 4 * lg) = r;
      }
  } else {
    __bf16* out = (__bf16*)p.out + orow;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        bf16x4 r;
        r[0] = (__bf16)(o[db][4 * a + 0] * inv);
        r[1] = (__bf16)(o[db][4 * a + 1] * inv);
        r[2] = (__bf16)(o[db][4 * a + 2] * inv);
        r[3] = (__bf16)(o[db][4 * a + 3] * inv);
        *(bf16x4*)(out + 32 * db + 8 * a + 4 * lg) = r;
      }
  }
  if (p.lse != nullptr && lg == 0) p.lse[(size_t)h * p.n + qpos] = (m_run + fast_log2(l_tot)) * kLn2;
}

}  // namespace

hipError_t launch_attention(const __bf16* q, const __bf16* k, const __bf16* v, const int32_t* count,
                            const int32_t* idx, void* out, int out_fp32, float* lse, int hq, int hkv, int n,
                            float scale, bool dense, hipStream_t stream) {
  AttnArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.count = count;
  a.idx = idx;
  a.out = out;
  a.lse = lse;
  a.n = n;
  a.nblk = n / kBlock;
  a.qpg = hq / hkv;
  a.scale_log2 = scale * kLog2e;
  a.out_fp32 = out_fp32;
  a.map = make_row_map(hq, hkv, a.nblk);
  const unsigned grid = (unsigned)hq * (unsigned)a.nblk;
  if (dense)
    hipLaunchKernelGGL(fa_fwd_kernel<true>, dim3(grid), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(fa_fwd_kernel<false>, dim3(grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace crisp
