// C ABI of the CRISP library: argument validation, workspace carving and
// kernel dispatch.  Declarations and the contract of every entry point are
// in include/crisp.h.

#include <hip/hip_runtime.h>
#include <math.h>
#include <string.h>

#include "../../include/crisp.h"
#include "common.h"
#include "internal.h"

namespace {

constexpr int kMaxSeqLen = 524288;  // LDS sizing of the selection kernels (N <= 4096)
constexpr int kMaxDevices = 64;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Finite, decided on the bit pattern (exponent not all ones), so that a NaN
// or an infinity is rejected even where a compiler flag lets the compiler
// assume that floats are never NaN.
bool finite_bits(float x) {
  uint32_t b;
  memcpy(&b, &x, sizeof b);
  return (b & 0x7f800000u) != 0x7f800000u;
}
// lo <= x <= hi (or lo < x when lo_open), for finite x only.
bool in_range(float x, float lo, float hi, bool lo_open = false) {
  if (!finite_bits(x)) return false;
  return (lo_open ? x > lo : x >= lo) && x <= hi;
}

crisp_status check_dims(const crisp_dims* d) {
  if (d == nullptr) return CRISP_ERR_NULL;
  if (d->head_dim != 128 || d->block != 128) return CRISP_ERR_SHAPE;
  if (d->num_q_heads <= 0 || d->num_kv_heads <= 0) return CRISP_ERR_SHAPE;
  if (d->num_q_heads % d->num_kv_heads != 0) return CRISP_ERR_SHAPE;
  // any length: a partial last block holds the n - 128 (N-1) last positions
  if (d->seq_len < 2 * d->block || d->seq_len > kMaxSeqLen) return CRISP_ERR_SHAPE;
  // grid sizes (Hq * N workgroups) must fit the launch limits comfortably
  if ((long long)d->num_q_heads * crisp::nblocks(d->seq_len) > (1LL << 30)) return CRISP_ERR_SHAPE;
  if (!in_range(d->scale, 0.f, 3.0e38f, true)) return CRISP_ERR_PARAM;
  return CRISP_OK;
}

crisp_status check_cfg(const crisp_dims* d, const crisp_cfg* c) {
  if (c == nullptr) return CRISP_ERR_NULL;
  if (!in_range(c->tau, 0.f, 1.f)) return CRISP_ERR_PARAM;
  if (!in_range(c->alpha, 0.f, 3.0e38f, true)) return CRISP_ERR_PARAM;
  if (!in_range(c->gamma_pe, 0.f, 1.f, true)) return CRISP_ERR_PARAM;
  if (c->kmin_blocks < 1) return CRISP_ERR_PARAM;
  if (c->sink_width < 1 || c->sink_width > d->seq_len / 2) return CRISP_ERR_PARAM;
  if (c->recency_width < 1 || c->recency_width > d->seq_len / 2) return CRISP_ERR_PARAM;
  if (c->nf_stat != CRISP_NF_MEDIAN && c->nf_stat != CRISP_NF_MEAN) return CRISP_ERR_PARAM;
  if (c->route_override < CRISP_ROUTE_AUTO || c->route_override > CRISP_ROUTE_FORCE_PE) return CRISP_ERR_PARAM;
  return CRISP_OK;
}

crisp_status check_ptr(const void* p) {
  if (p == nullptr) return CRISP_ERR_NULL;
  if (!aligned16(p)) return CRISP_ERR_ALIGN;
  return CRISP_OK;
}

crisp_status check_opt(const void* p) { return (p == nullptr || aligned16(p)) ? CRISP_OK : CRISP_ERR_ALIGN; }

#define CRISP_TRY(expr)              \
  do {                               \
    crisp_status s_ = (expr);        \
    if (s_ != CRISP_OK) return s_;   \
  } while (0)

// 0 = unknown, 1 = gfx950, 2 = other
int g_device_kind[kMaxDevices];

crisp_status check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return CRISP_ERR_DEVICE;
  if (dev >= kMaxDevices) return CRISP_ERR_DEVICE;
  int kind = __atomic_load_n(&g_device_kind[dev], __ATOMIC_ACQUIRE);
  if (kind == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return CRISP_ERR_DEVICE;
    kind = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    __atomic_store_n(&g_device_kind[dev], kind, __ATOMIC_RELEASE);
  }
  return kind == 1 ? CRISP_OK : CRISP_ERR_DEVICE;
}

crisp_status launched(hipError_t e) { return e == hipSuccess ? CRISP_OK : CRISP_ERR_LAUNCH; }

// Selection workspace of crisp_select_noalloc: a file-scope device array,
// one copy per device, held from the module's load to the process's end.
// Host code never passes its name to a kernel (on the host it is only a
// stand-in for the symbol): the device address comes from
// hipGetSymbolAddress, once per device, and is kept in g_scratch_ptr.
static __device__ __align__(256) unsigned char scratch[CRISP_NOALLOC_SCRATCH_BYTES];
void* g_scratch_ptr[kMaxDevices];

// The current device's address of `scratch` (NULL if it cannot be had).
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* ptr = __atomic_load_n(&g_scratch_ptr[dev], __ATOMIC_ACQUIRE);
  if (ptr == nullptr) {
    // concurrent first calls on one device get the same address
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    __atomic_store_n(&g_scratch_ptr[dev], ptr, __ATOMIC_RELEASE);
  }
  return ptr;
}

// The proxy's output: the map, the block masses, or both; at least one.
crisp_status check_map_or_mass(const void* attn_map, const void* block_mass) {
  if (attn_map == nullptr && block_mass == nullptr) return CRISP_ERR_NULL;
  CRISP_TRY(check_opt(attn_map));
  return check_opt(block_mass);
}

crisp_status check_blocks(const crisp_blocks* out) {
  if (out == nullptr) return CRISP_ERR_NULL;
  CRISP_TRY(check_ptr(out->count));
  CRISP_TRY(check_ptr(out->idx));
  CRISP_TRY(check_opt(out->v_score));
  CRISP_TRY(check_opt(out->s_score));
  CRISP_TRY(check_opt(out->floor_v));
  CRISP_TRY(check_opt(out->floor_s));
  CRISP_TRY(check_opt(out->v_mask));
  CRISP_TRY(check_opt(out->s_mask));
  CRISP_TRY(check_opt(out->n_v));
  CRISP_TRY(check_opt(out->n_s));
  return CRISP_OK;
}

// Selection launch after validation: carves the workspace and points the
// optional diagnostics the caller gave at its own buffers.
crisp_status select_launch(const crisp_dims* dims, const crisp_cfg* cfg, bool use_gamma, float gamma, const void* q,
                           const void* k, const float* attn_map, const float* block_mass, const int32_t* route,
                           const crisp_blocks* out, void* workspace, const crisp::TokenCols* tok, void* stream) {
  const int hq = dims->num_q_heads, hkv = dims->num_kv_heads, n = dims->seq_len;
  crisp::SelectBuffers b = crisp::carve_select_workspace(workspace, hq, hkv, n);
  if (out->v_score) b.vscore = out->v_score;
  if (out->s_score) b.sscore = out->s_score;
  if (out->floor_v) b.floor_v = out->floor_v;
  if (out->floor_s) b.floor_s = out->floor_s;
  if (out->v_mask) b.vmask = out->v_mask;
  if (out->s_mask) b.smask = out->s_mask;
  if (out->n_v) b.n_v = out->n_v;
  if (out->n_s) b.n_s = out->n_s;
  return launched(crisp::launch_select((const __bf16*)q, (const __bf16*)k, attn_map, block_mass, route, b, out->count,
                                       out->idx,
                                       hq, hkv, n, dims->scale, cfg->alpha, cfg->gamma_pe, cfg->kmin_blocks,
                                       cfg->nf_stat, use_gamma, gamma, tok, (hipStream_t)stream));
}

crisp_status select_common(const crisp_dims* dims, const crisp_cfg* cfg, bool use_gamma, float gamma, const void* q,
                           const void* k, const float* attn_map, const float* block_mass, const int32_t* route,
                           const crisp_blocks* out, void* workspace, size_t workspace_bytes,
                           const crisp::TokenCols* tok, void* stream) {
  CRISP_TRY(check_dims(dims));
  CRISP_TRY(check_cfg(dims, cfg));
  if (use_gamma && !in_range(gamma, 0.f, 1.f, true)) return CRISP_ERR_PARAM;
  CRISP_TRY(check_blocks(out));
  CRISP_TRY(check_ptr(q));
  CRISP_TRY(check_ptr(k));
  CRISP_TRY(check_map_or_mass(attn_map, block_mass));
  CRISP_TRY(check_ptr(route));
  CRISP_TRY(check_ptr(workspace));
  if (workspace_bytes < crisp::select_workspace_bytes(dims->num_q_heads, dims->num_kv_heads, dims->seq_len))
    return CRISP_ERR_WORKSPACE;
  CRISP_TRY(check_device());
  return select_launch(dims, cfg, use_gamma, gamma, q, k, attn_map, block_mass, route, out, workspace, tok, stream);
}

// The one-call layer's workspace: the proxy scratch first (so that a buffer
// of this size also serves the step-by-step calls, the selection workspace
// starting at the proxy scratch rounded up to 256 bytes), then the selection
// workspace, then the block masses, C_struct and routes.
constexpr size_t kCarve = 256;
size_t round_carve(size_t x) { return (x + kCarve - 1) / kCarve * kCarve; }

struct PrefillCarve {
  void* partials;
  void* select_ws;
  float* mass;
  float* c_struct;
  int32_t* route;
  int* queue;
  size_t bytes;
};

PrefillCarve carve_prefill(void* ws, int hq, int hkv, int n) {
  PrefillCarve c;
  const size_t N = (size_t)crisp::nblocks(n);
  const uintptr_t p = (uintptr_t)ws;  // integer arithmetic: ws may be NULL when only the size is wanted
  size_t off = 0;
  c.partials = (void*)(p + off);
  off += round_carve(crisp::proxy_scratch_bytes(hq, n));
  c.select_ws = (void*)(p + off);
  off += round_carve(crisp::select_workspace_bytes(hq, hkv, n));
  c.mass = (float*)(p + off);
  off += round_carve(4 * (size_t)hq * N * sizeof(float));
  c.c_struct = (float*)(p + off);
  off += round_carve((size_t)hq * sizeof(float));
  c.route = (int32_t*)(p + off);
  off += round_carve((size_t)hq * sizeof(int32_t));
  c.queue = (int*)(p + off);
  off += round_carve(crisp::kAttnQueueBytes);
  c.bytes = off;
  return c;
}

crisp_status attn_common(const crisp_dims* dims, const void* q, const void* k, const void* v, const int32_t* count,
                         const int32_t* idx, void* out, int32_t out_is_fp32, float* lse, bool dense, void* workspace,
                         size_t workspace_bytes, void* stream) {
  CRISP_TRY(check_dims(dims));
  CRISP_TRY(check_ptr(q));
  CRISP_TRY(check_ptr(k));
  CRISP_TRY(check_ptr(v));
  if (!dense) {
    CRISP_TRY(check_ptr(count));
    CRISP_TRY(check_ptr(idx));
  }
  CRISP_TRY(check_ptr(out));
  CRISP_TRY(check_opt(lse));
  if (out_is_fp32 != 0 && out_is_fp32 != 1) return CRISP_ERR_PARAM;
  CRISP_TRY(check_ptr(workspace));
  if (workspace_bytes < crisp::kAttnQueueBytes) return CRISP_ERR_WORKSPACE;
  CRISP_TRY(check_device());
  return launched(crisp::launch_attention((const __bf16*)q, (const __bf16*)k, (const __bf16*)v, count, idx, out,
                                          out_is_fp32, lse, dims->num_q_heads, dims->num_kv_heads, dims->seq_len,
                                          dims->scale, dense, (int*)workspace, (hipStream_t)stream));
}

}  // namespace

extern "C" {

size_t crisp_proxy_scratch_bytes(const crisp_dims* dims) {
  if (check_dims(dims) != CRISP_OK) return 0;
  return crisp::proxy_scratch_bytes(dims->num_q_heads, dims->seq_len);
}

crisp_status crisp_proxy(const crisp_dims* dims, const void* q, const void* k, float* attn_map, float* block_mass,
                         float* row_lse, void* partials, size_t partials_bytes, void* stream) {
  CRISP_TRY(check_dims(dims));
  CRISP_TRY(check_ptr(q));
  CRISP_TRY(check_ptr(k));
  CRISP_TRY(check_map_or_mass(attn_map, block_mass));
  CRISP_TRY(check_opt(row_lse));
  CRISP_TRY(check_ptr(partials));
  if (partials_bytes < crisp::proxy_scratch_bytes(dims->num_q_heads, dims->seq_len)) return CRISP_ERR_WORKSPACE;
  CRISP_TRY(check_device());
  return launched(crisp::launch_proxy((const __bf16*)q, (const __bf16*)k, attn_map, block_mass, nullptr, row_lse,
                                      partials, dims->num_q_heads, dims->num_kv_heads, dims->seq_len, dims->scale,
                                      (hipStream_t)stream));
}

crisp_status crisp_proxy_cols(const crisp_dims* dims, const void* q, const void* k, float* block_mass,
                              float* col_mass, float* row_lse, void* partials, size_t partials_bytes, void* stream) {
  CRISP_TRY(check_dims(dims));
  CRISP_TRY(check_ptr(q));
  CRISP_TRY(check_ptr(k));
  CRISP_TRY(check_ptr(block_mass));
  CRISP_TRY(check_ptr(col_mass));
  CRISP_TRY(check_opt(row_lse));
  CRISP_TRY(check_ptr(partials));
  if (partials_bytes < crisp::proxy_scratch_bytes(dims->num_q_heads, dims->seq_len)) return CRISP_ERR_WORKSPACE;
  CRISP_TRY(check_device());
  return launched(crisp::launch_proxy((const __bf16*)q, (const __bf16*)k, nullptr, block_mass, col_mass, row_lse,
                                      partials, dims->num_q_heads, dims->num_kv_heads, dims->seq_len, dims->scale,
                                      (hipStream_t)stream));
}

crisp_status crisp_route(const crisp_dims* dims, const crisp_cfg* cfg, const float* attn_map, const float* block_mass,
                         float* c_struct, int32_t* route, void* stream) {
  CRISP_TRY(check_dims(dims));
  CRISP_TRY(check_cfg(dims, cfg));
  CRISP_TRY(check_map_or_mass(attn_map, block_mass));
  // block masses resolve whole key blocks only
  if (block_mass != nullptr && (cfg->sink_width != dims->block || cfg->recency_width != dims->block))
    return CRISP_ERR_PARAM;
  CRISP_TRY(check_ptr(c_struct));
  CRISP_TRY(check_ptr(route));
  CRISP_TRY(check_device());
  return launched(crisp::launch_route(attn_map, block_mass, c_struct, route, dims->num_q_heads, dims->seq_len,
                                      cfg->sink_width, cfg->recency_width, cfg->tau, cfg->route_override,
                                      (hipStream_t)stream));
}

crisp_status crisp_route_cols(const crisp_dims* dims, const crisp_cfg* cfg, const float* col_mass, float* c_struct,
                              int32_t* route, void* stream) {
  CRISP_TRY(check_dims(dims));
  CRISP_TRY(check_cfg(dims, cfg));
  CRISP_TRY(check_ptr(col_mass));
  CRISP_TRY(check_ptr(c_struct));
  CRISP_TRY(check_ptr(route));
  CRISP_TRY(check_device());
  return launched(crisp::launch_route_cols(col_mass, c_struct, route, dims->num_q_heads, dims->seq_len,
                                           cfg->sink_width, cfg->recency_width, cfg->tau, cfg->route_override,
                                           (hipStream_t)stream));
}

size_t crisp_route_jsd_workspace_bytes(const crisp_dims* dims) {
  if (check_dims(dims) != CRISP_OK) return 0;
  return crisp::jsd_workspace_bytes(dims->num_q_heads, dims->seq_len);
}

crisp_status crisp_route_jsd(const crisp_dims* dims, float tau_jsd, const void* q, const void* k,
                             const float* block_mass, float* js_dist, int32_t* route, float* estimate,
                             void* workspace, size_t workspace_bytes, void* stream) {
  CRISP_TRY(check_dims(dims));
  if (!in_range(tau_jsd, 0.f, 3.0e38f)) return CRISP_ERR_PARAM;
  CRISP_TRY(check_ptr(q));
  CRISP_TRY(check_ptr(k));
  CRISP_TRY(check_ptr(block_mass));
  CRISP_TRY(check_ptr(js_dist));
  CRISP_TRY(check_ptr(route));
  CRISP_TRY(check_opt(estimate));
  CRISP_TRY(check_ptr(workspace));
  if (workspace_bytes < crisp::jsd_workspace_bytes(dims->num_q_heads, dims->seq_len)) return CRISP_ERR_WORKSPACE;
  CRISP_TRY(check_device());
  return launched(crisp::launch_route_jsd((const __bf16*)q, (const __bf16*)k, block_mass, js_dist, route, estimate,
                                          workspace, dims->num_q_heads, dims->num_kv_heads, dims->seq_len,
                                          dims->scale, tau_jsd, (hipStream_t)stream));
}

crisp_status crisp_select(const crisp_dims* dims, const crisp_cfg* cfg, const void* q, const void* k,
                          const float* attn_map, const float* block_mass, const int32_t* route,
                          const crisp_blocks* out, void* workspace, size_t workspace_bytes, void* stream) {
  return select_common(dims, cfg, false, 0.f, q, k, attn_map, block_mass, route, out, workspace, workspace_bytes,
                       nullptr, stream);
}

crisp_status crisp_select_noalloc(const crisp_dims* dims, const crisp_cfg* cfg, const void* q, const void* k,
                                  const float* attn_map, const float* block_mass, const int32_t* route,
                                  const crisp_blocks* out, void* stream) {
  CRISP_TRY(check_dims(dims));
  CRISP_TRY(check_cfg(dims, cfg));
  CRISP_TRY(check_blocks(out));
  CRISP_TRY(check_ptr(q));
  CRISP_TRY(check_ptr(k));
  CRISP_TRY(check_map_or_mass(attn_map, block_mass));
  CRISP_TRY(check_ptr(route));
  if (crisp::select_workspace_bytes(dims->num_q_heads, dims->num_kv_heads, dims->seq_len) >
      (size_t)CRISP_NOALLOC_SCRATCH_BYTES)
    return CRISP_ERR_WORKSPACE;
  CRISP_TRY(check_device());
  void* ws = scratch_ptr();
  if (ws == nullptr) return CRISP_ERR_DEVICE;
  return select_launch(dims, cfg, false, 0.f, q, k, attn_map, block_mass, route, out, ws, nullptr, stream);
}

crisp_status crisp_select_tokens(const crisp_dims* dims, const crisp_cfg* cfg, const void* q, const void* k,
                                 const float* block_mass, const float* col_mass, const int32_t* route,
                                 const crisp_blocks* out, int32_t* cols, int32_t* ncols, int32_t* col_below,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  CRISP_TRY(check_ptr(block_mass));
  CRISP_TRY(check_ptr(col_mass));
  CRISP_TRY(check_ptr(cols));
  CRISP_TRY(check_ptr(ncols));
  CRISP_TRY(check_ptr(col_below));
  crisp::TokenCols tc;
  tc.colmass = col_mass;
  tc.cols = cols;
  tc.ncols = ncols;
  tc.col_below = col_below;
  return select_common(dims, cfg, false, 0.f, q, k, nullptr, block_mass, route, out, workspace, workspace_bytes, &tc,
                       stream);
}

crisp_status crisp_select_gamma(const crisp_dims* dims, const crisp_cfg* cfg, float gamma, const void* q,
                                const void* k, const float* attn_map, const float* block_mass, const int32_t* route,
                                const crisp_blocks* out, void* workspace, size_t workspace_bytes, void* stream) {
  return select_common(dims, cfg, true, gamma, q, k, attn_map, block_mass, route, out, workspace, workspace_bytes,
                       nullptr, stream);
}

size_t crisp_select_workspace_bytes(const crisp_dims* dims) {
  if (check_dims(dims) != CRISP_OK) return 0;
  return crisp::select_workspace_bytes(dims->num_q_heads, dims->num_kv_heads, dims->seq_len);
}

size_t crisp_list_capacity(const crisp_dims* dims) {
  if (check_dims(dims) != CRISP_OK) return 0;
  const size_t N = (size_t)crisp::nblocks(dims->seq_len);
  return (size_t)dims->num_q_heads * (N * (N + 1) / 2);
}

size_t crisp_attn_workspace_bytes(const crisp_dims* dims) {
  if (check_dims(dims) != CRISP_OK) return 0;
  return crisp::kAttnQueueBytes;
}

crisp_status crisp_sparse_attn(const crisp_dims* dims, const void* q, const void* k, const void* v,
                               const int32_t* count, const int32_t* idx, void* out, int32_t out_is_fp32, float* lse,
                               void* workspace, size_t workspace_bytes, void* stream) {
  return attn_common(dims, q, k, v, count, idx, out, out_is_fp32, lse, false, workspace, workspace_bytes, stream);
}

crisp_status crisp_sparse_attn_cols(const crisp_dims* dims, const void* q, const void* k, const void* v,
                                    const int32_t* count, const int32_t* idx, const int32_t* cols,
                                    const int32_t* col_below, float* out, float* lse, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  CRISP_TRY(check_dims(dims));
  CRISP_TRY(check_ptr(q));
  CRISP_TRY(check_ptr(k));
  CRISP_TRY(check_ptr(v));
  CRISP_TRY(check_ptr(count));
  CRISP_TRY(check_ptr(idx));
  CRISP_TRY(check_ptr(cols));
  CRISP_TRY(check_ptr(col_below));
  CRISP_TRY(check_ptr(out));
  CRISP_TRY(check_ptr(lse));
  CRISP_TRY(check_ptr(workspace));
  if (workspace_bytes < crisp::kAttnQueueBytes) return CRISP_ERR_WORKSPACE;
  CRISP_TRY(check_device());
  return launched(crisp::launch_col_attention((const __bf16*)q, (const __bf16*)k, (const __bf16*)v, count, idx, cols,
                                              col_below, out, lse, dims->num_q_heads, dims->num_kv_heads,
                                              dims->seq_len, dims->scale, (int*)workspace, (hipStream_t)stream));
}

crisp_status crisp_dense_attn(const crisp_dims* dims, const void* q, const void* k, const void* v, void* out,
                              int32_t out_is_fp32, float* lse, void* workspace, size_t workspace_bytes,
                              void* stream) {
  return attn_common(dims, q, k, v, nullptr, nullptr, out, out_is_fp32, lse, true, workspace, workspace_bytes,
                     stream);
}

size_t crisp_prefill_workspace_bytes(const crisp_dims* dims) {
  if (check_dims(dims) != CRISP_OK) return 0;
  return carve_prefill(nullptr, dims->num_q_heads, dims->num_kv_heads, dims->seq_len).bytes;
}

crisp_status crisp_prefill(const crisp_dims* dims, const crisp_cfg* cfg, int32_t dense_below, const void* q,
                           const void* k, const void* v, const crisp_blocks* blocks, float* block_mass,
                           float* c_struct, int32_t* route, void* out, int32_t out_is_fp32, float* lse,
                           void* workspace, size_t workspace_bytes, void* stream) {
  CRISP_TRY(check_dims(dims));
  CRISP_TRY(check_cfg(dims, cfg));
  // routing reads the block masses, which resolve whole key blocks only
  if (cfg->sink_width != dims->block || cfg->recency_width != dims->block) return CRISP_ERR_PARAM;
  CRISP_TRY(check_ptr(q));
  CRISP_TRY(check_ptr(k));
  CRISP_TRY(check_ptr(v));
  CRISP_TRY(check_blocks(blocks));
  CRISP_TRY(check_opt(block_mass));
  CRISP_TRY(check_opt(c_struct));
  CRISP_TRY(check_opt(route));
  CRISP_TRY(check_ptr(out));
  CRISP_TRY(check_opt(lse));
  if (out_is_fp32 != 0 && out_is_fp32 != 1) return CRISP_ERR_PARAM;
  CRISP_TRY(check_ptr(workspace));
  const int hq = dims->num_q_heads, hkv = dims->num_kv_heads, n = dims->seq_len;
  const PrefillCarve w = carve_prefill(workspace, hq, hkv, n);
  if (workspace_bytes < w.bytes) return CRISP_ERR_WORKSPACE;
  CRISP_TRY(check_device());
  const int gate = dense_below < 0 ? CRISP_DENSE_BELOW_DEFAULT : dense_below;
  const hipStream_t st = (hipStream_t)stream;
  if (n < gate)
    return launched(crisp::launch_attention((const __bf16*)q, (const __bf16*)k, (const __bf16*)v, nullptr, nullptr,
                                            out, out_is_fp32, lse, hq, hkv, n, dims->scale, true, w.queue, st));
  float* mass = block_mass ? block_mass : w.mass;
  float* cs = c_struct ? c_struct : w.c_struct;
  int32_t* rt = route ? route : w.route;
  CRISP_TRY(launched(crisp::launch_proxy((const __bf16*)q, (const __bf16*)k, nullptr, mass, nullptr, nullptr,
                                         w.partials, hq, hkv, n, dims->scale, st)));
  CRISP_TRY(launched(crisp::launch_route(nullptr, mass, cs, rt, hq, n, cfg->sink_width, cfg->recency_width, cfg->tau,
                                         cfg->route_override, st)));
  CRISP_TRY(select_launch(dims, cfg, false, 0.f, q, k, nullptr, mass, rt, blocks, w.select_ws, nullptr, stream));
  return launched(crisp::launch_attention((const __bf16*)q, (const __bf16*)k, (const __bf16*)v, blocks->count,
                                          blocks->idx, out, out_is_fp32, lse, hq, hkv, n, dims->scale, false, w.queue,
                                          st));
}

const char* crisp_status_string(crisp_status status) {
  switch (status) {
    case CRISP_OK: return "ok";
    case CRISP_ERR_NULL: return "a required pointer is NULL";
    case CRISP_ERR_SHAPE: return "unsupported dimensions (need d = 128, block = 128, 256 <= n <= 524288, Hq % Hkv == 0)";
    case CRISP_ERR_PARAM: return "a method parameter is out of range";
    case CRISP_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case CRISP_ERR_WORKSPACE: return "workspace or scratch buffer too small";
    case CRISP_ERR_DEVICE: return "no gfx950 device is current";
    case CRISP_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

int32_t crisp_abi_version(void) { return (5 << 16) | 1; }

}  // extern "C"
