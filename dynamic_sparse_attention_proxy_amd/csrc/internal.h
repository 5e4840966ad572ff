// Launchers of the CRISP kernels, called by the C ABI layer after argument
// validation.  All take device pointers and enqueue on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace crisp {

// Blocks of 128 positions, aligned at position 0; the last one holds
// n - 128 (N - 1) positions when 128 does not divide n.
__host__ __device__ inline int nblocks(int n) { return (n + 127) / 128; }

// Proxy: keys per workgroup of the two proxy passes.
constexpr int kProxyChunk = 1024;
inline int proxy_chunks(int n) { return (n + kProxyChunk - 1) / kProxyChunk; }
inline size_t proxy_scratch_bytes(int hq, int n) {
  // per (head, chunk, row): running max and sum; per (head, row): log2-sum-exp;
  // per (head, key block, row): the row's mass in the three slash bands of
  // the block and its running max (16 bytes); per (head, row): the row's
  // mass in key block N-2 that lies in the recency window
  return (size_t)hq * proxy_chunks(n) * 128 * 2 * sizeof(float) + (size_t)hq * 128 * sizeof(float) +
         (size_t)hq * nblocks(n) * 128 * 4 * sizeof(float) + (size_t)hq * 128 * sizeof(float);
}

// amap and/or mass (at least one non-null): the proxy map and the block
// masses [4][Hq][N] (per key block kb the mass in slash bands N-1-kb,
// N-2-kb, N-3-kb, and the mass on the last 128 keys).  colmass [Hq][n] (the
// column masses) may only be given with mass and without amap.
hipError_t launch_proxy(const __bf16* q, const __bf16* k, float* amap, float* mass, float* colmass, float* row_lse,
                        void* scratch, int hq, int hkv, int n, float scale, hipStream_t stream);

// From the column masses [Hq][n] (any widths).
hipError_t launch_route_cols(const float* colmass, float* c_struct, int32_t* route, int hq, int n, int sink_width,
                             int recency_width, float tau, int route_override, hipStream_t stream);

// From the block masses when mass != nullptr (widths of one block), else
// from the map.
hipError_t launch_route(const float* amap, const float* mass, float* c_struct, int32_t* route, int hq, int n,
                        int sink_width, int recency_width, float tau, int route_override, hipStream_t stream);

struct SelectBuffers {
  float* mass;    // [4][Hq][N] block masses summed from the proxy map
  float* vscore;  // [Hq][N]
  float* sscore;  // [Hq][N]
  float* floor_v; // [Hq]
  float* floor_s; // [Hq]
  int32_t* vmask; // [Hq][N]
  int32_t* smask; // [Hq][N]
  int32_t* n_v;   // [Hq]
  int32_t* n_s;   // [Hq]
  int32_t* kept;  // [2][Hq] kept blocks per direction (workspace only)
  float* kbar;    // [Hkv][N] pooled keys, 512 bytes each: bf16 hi[128] then lo[128]
};

size_t select_workspace_bytes(int hq, int hkv, int n);
SelectBuffers carve_select_workspace(void* ws, int hq, int hkv, int n);

// Token-granular vertical selection: column masses in, kept columns out.
struct TokenCols {
  const float* colmass;  // [Hq][n]
  int32_t* cols;         // [Hq][n]: kept columns past key block 0, ascending
  int32_t* ncols;        // [Hq]
  int32_t* col_below;    // [Hq][N]: kept columns below 128 qb
};

// use_gamma = false: noise floor on VS heads, gamma_pe on PE heads.
// use_gamma = true: gamma-cumulative on VS heads and `gamma` on PE heads.
// VS scores come from the block masses when mass != nullptr, else from a
// pass over the map.
hipError_t launch_select(const __bf16* q, const __bf16* k, const float* amap, const float* mass, const int32_t* route,
                         const SelectBuffers& b, int32_t* count, int32_t* idx, int hq, int hkv, int n, float scale,
                         float alpha, float gamma_pe, int kmin, int nf_stat, bool use_gamma, float gamma,
                         const TokenCols* tok, hipStream_t stream);

// JSD routing signal: workspace holds qbar [Hq][128] and the logits [Hq][N].
size_t jsd_workspace_bytes(int hq, int n);
hipError_t launch_route_jsd(const __bf16* q, const __bf16* k, const float* mass, float* js_dist, int32_t* route,
                            float* estimate, void* workspace, int hq, int hkv, int n, float scale, float tau_jsd,
                            hipStream_t stream);

// Kept single columns merged into the tile attention (out fp32 and lse are
// read and updated in place).
hipError_t launch_col_attention(const __bf16* q, const __bf16* k, const __bf16* v, const int32_t* count,
                                const int32_t* idx, const int32_t* cols, const int32_t* col_below, float* out,
                                float* lse, int hq, int hkv, int n, float scale, int* queue, hipStream_t stream);

hipError_t launch_attention(const __bf16* q, const __bf16* k, const __bf16* v, const int32_t* count,
                            const int32_t* idx, void* out, int out_fp32, float* lse, int hq, int hkv, int n,
                            float scale, bool dense, int* queue, hipStream_t stream);
// Device bytes of the attention kernels' work queues (the `queue` arguments
// of launch_attention and launch_col_attention).
constexpr size_t kAttnQueueBytes = 256;

}  // namespace crisp
