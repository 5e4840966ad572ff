/*
 * crisp.h - C ABI of the CRISP sparse prefill attention library (gfx950).
 *
 * Method: "CRISP: Cliff-awaRe Input-adaptive Sparse Prefilling with
 * Structural-Mass-Motivated Routing" (arXiv 2609.01925).  Per attention head
 * the prefill path makes two runtime decisions, which sparse pattern to use
 * and how many blocks to keep (ai.info summary, "Methodology in Plain
 * English"), then runs exact softmax attention over what it kept (ai.info
 * summary, "Why This Matters").  The four calls below are those steps, in
 * order, plus a dense causal kernel (the speedup denominator) and a
 * gamma-cumulative selector (the FlexPrefill-style budget rule the paper
 * compares against, "Main Findings").
 *
 * Conventions shared by every entry point
 *   - Tensors are device pointers to contiguous, head-major arrays:
 *       q        [Hq][n][d]   bf16, rotary embedding already applied
 *       k, v     [Hkv][n][d]  bf16, rotary embedding already applied (k)
 *     Query head h reads KV head h / (Hq / Hkv) (consecutive heads share).
 *   - Supported shapes: d = 128, block = 128, 256 <= n <= 524288, Hq a
 *     multiple of Hkv.  Anything else is CRISP_ERR_SHAPE.
 *   - Blocks: N = ceil(n / 128) blocks of 128 positions from position 0;
 *     when 128 does not divide n the last block holds the n - 128 (N-1)
 *     last positions, and every quantity below covers only the positions
 *     that exist (a partial block has fewer keys, query rows and offsets;
 *     its pooled mean is over its rows).
 *   - Every pointer must be 16-byte aligned (CRISP_ERR_ALIGN otherwise).
 *   - The caller owns every buffer; the library allocates nothing.  Its
 *     global state is write-once per device: whether the device is a gfx950,
 *     and the address of the static scratch of crisp_select_noalloc.  Every
 *     other call is reentrant.
 *   - Arguments are validated on the host before anything is launched; a
 *     failed validation returns an error and leaves all outputs untouched.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t, NULL for
 *     the default stream).  No call synchronises; outputs are valid once
 *     the stream has completed.  A launch error is CRISP_ERR_LAUNCH.
 *   - The device must be a gfx950 (CRISP_ERR_DEVICE otherwise).
 */
#ifndef CRISP_H
#define CRISP_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define CRISP_API __attribute__((visibility("default")))
#else
#define CRISP_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum crisp_status {
  CRISP_OK = 0,
  CRISP_ERR_NULL = 1,      /* a required pointer is NULL */
  CRISP_ERR_SHAPE = 2,     /* unsupported dimensions */
  CRISP_ERR_PARAM = 3,     /* a method parameter is out of range */
  CRISP_ERR_ALIGN = 4,     /* a pointer is not 16-byte aligned */
  CRISP_ERR_WORKSPACE = 5, /* workspace smaller than crisp_select_workspace_bytes */
  CRISP_ERR_DEVICE = 6,    /* no device, or the current device is not gfx950 */
  CRISP_ERR_LAUNCH = 7     /* a kernel launch failed */
} crisp_status;

/* Route codes written by crisp_route (per query head). */
#define CRISP_ROUTE_PE 0 /* Pooled-Estimation path */
#define CRISP_ROUTE_VS 1 /* Vertical-Slash path */

/* crisp_cfg.route_override */
#define CRISP_ROUTE_AUTO 0     /* C_struct >= tau picks VS, else PE */
#define CRISP_ROUTE_FORCE_VS 1 /* every head VS (exercises the noise floor) */
#define CRISP_ROUTE_FORCE_PE 2 /* every head PE */

/* crisp_cfg.nf_stat: statistic of the background block mass */
#define CRISP_NF_MEDIAN 0 /* lower median of the non-retained blocks (default) */
#define CRISP_NF_MEAN 1   /* their mean (the literal "expected background mass") */

typedef struct crisp_dims {
  int32_t num_q_heads;  /* Hq */
  int32_t num_kv_heads; /* Hkv, divides Hq */
  int32_t seq_len;      /* n, 2 * block .. 524288 (any length) */
  int32_t head_dim;     /* d, must be 128 */
  int32_t block;        /* B, must be 128 */
  float scale;          /* softmax scale applied to q.k, > 0 (normally 1/sqrt(d)) */
} crisp_dims;

/* Method parameters (ai.info summary, "Methodology in Plain English":
 * block 128, k_min = 8 blocks per direction, gamma = 0.95 on PE only,
 * alpha in {1.0, 1.25} on VS; "Key Contributions": 128-token sink and
 * recency windows). */
typedef struct crisp_cfg {
  float tau;             /* route threshold on C_struct, in [0, 1] */
  float alpha;           /* noise-floor multiple, > 0 */
  float gamma_pe;        /* coverage target on PE heads, in (0, 1] */
  int32_t kmin_blocks;   /* minimum blocks kept per VS direction, >= 1 */
  int32_t sink_width;    /* first columns counted by C_struct, 1..n/2 */
  int32_t recency_width; /* last columns counted by C_struct, 1..n/2 */
  int32_t nf_stat;       /* CRISP_NF_MEDIAN or CRISP_NF_MEAN */
  int32_t route_override;/* CRISP_ROUTE_AUTO / _FORCE_VS / _FORCE_PE */
} crisp_cfg;

/* Selection output.  With N = ceil(n / 128) blocks, the key-block list of query
 * block qb of head h is idx[h * N(N+1)/2 + qb(qb+1)/2 + t], t < count[h*N+qb],
 * ascending, always holding qb (the diagonal).  Optional diagnostics may be
 * NULL; for PE heads the VS diagnostics are written as zeros. */
typedef struct crisp_blocks {
  int32_t* count;   /* [Hq][N], required */
  int32_t* idx;     /* [Hq][N(N+1)/2], required (crisp_list_capacity entries) */
  float* v_score;   /* [Hq][N] pooled vertical mass, optional */
  float* s_score;   /* [Hq][N] pooled slash mass, optional */
  float* floor_v;   /* [Hq] threshold used on v (alpha * statistic), optional */
  float* floor_s;   /* [Hq] threshold used on s, optional */
  int32_t* v_mask;  /* [Hq][N] 1 = vertical block kept, optional */
  int32_t* s_mask;  /* [Hq][N] 1 = slash block kept, optional */
  int32_t* n_v;     /* [Hq] kept vertical blocks, optional */
  int32_t* n_s;     /* [Hq] kept slash blocks, optional */
} crisp_blocks;

/* Step 1 - proxy attention map (ai.info summary, "Key Contributions" item 2:
 * C_struct is read off a proxy attention map the method already computes).
 * The proxy rows are the last 128 query positions of each head, attending
 * causally to all keys:
 *   attn_map[h][r][j] = softmax_j(scale * q[h][n-128+r] . k[g(h)][j]), j <= n-128+r,
 *   and 0 for j > n-128+r.                                 [Hq][128][n] fp32
 * block_mass: the map summed per key block kb over all 128 rows, split by
 * slash band and with the recency window apart:              [4][Hq][N] fp32
 *   entry (r, j) lies at offset o = n-128+r-j, in slash band o / 128
 *   block_mass[0][h][kb] = mass of key block kb in band N-1-kb
 *   block_mass[1][h][kb] = mass of key block kb in band N-2-kb
 *   block_mass[2][h][kb] = mass of key block kb in band N-3-kb
 *   block_mass[3][h][kb] = mass of key block kb on keys j >= n-128
 * No other band is reachable.  With 128 | n, entry (r, 128 kb + c) is at
 * offset 128(N-1-kb) + r - c, so planes 0 and 1 are the tile's mass on/below
 * (r >= c) and above its diagonal, plane 2 is zero and plane 3 is the total
 * of block N-1.  Every quantity routing and selection read from the map
 * follows from these (ai.info summary, "Methodology in Plain English":
 * vertical mass per key block, slash mass per offset band): the vertical
 * score of kb is its three band planes summed over 128, the slash score of
 * band b is planes 0, 1, 2 of key blocks N-1-b, N-2-b, N-3-b over 128, and
 * C_struct with one-block sink and recency widths is (block 0's bands +
 * plane 3 of blocks N-2 and N-1) / 128.
 * Either output may be NULL, not both; computing only block_mass skips the
 * 4 * 128 * n * Hq bytes of the map.
 * row_lse (optional, [Hq][128] fp32): natural log of each row's sum of
 * exp(scale * q.k).  `partials` is scratch of crisp_proxy_scratch_bytes
 * bytes (caller-owned device memory). */
CRISP_API crisp_status crisp_proxy(const crisp_dims* dims, const void* q, const void* k, float* attn_map,
                         float* block_mass, float* row_lse, void* partials, size_t partials_bytes, void* stream);

CRISP_API size_t crisp_proxy_scratch_bytes(const crisp_dims* dims);

/* Step 2 - structural-mass routing (ai.info summary, "Key Contributions"
 * item 2 and "Methodology in Plain English"; ai-feeds summary, method
 * module 1).  C_struct[h] is the mass of the proxy map on the first
 * sink_width and the last recency_width key columns, averaged over the 128
 * proxy rows, so it lies in [0, 1]; route[h] = VS when C_struct >= tau, PE
 * otherwise, unless cfg->route_override forces one path.
 * Reads block_mass when it is non-NULL (then both widths must be 128,
 * CRISP_ERR_PARAM otherwise), else attn_map.  For other widths without the
 * map, crisp_route_cols reads the column masses of crisp_proxy_cols.
 * c_struct [Hq] fp32, route [Hq] int32. */
CRISP_API crisp_status crisp_route(const crisp_dims* dims, const crisp_cfg* cfg, const float* attn_map,
                         const float* block_mass, float* c_struct, int32_t* route, void* stream);

/* Step 2 from the column masses (same pages as crisp_route): C_struct[h] =
 * sum of col_mass[h][j] over the first sink_width and the last
 * recency_width columns, any widths in 1..n/2 (cfg is checked as for
 * crisp_route); route as crisp_route.  col_mass [Hq][n] fp32: the column
 * masses crisp_proxy_cols writes (the map's column sums over its 128 rows,
 * divided by 128).  c_struct [Hq] fp32, route [Hq] int32; all device
 * pointers, 16-byte aligned. */
CRISP_API crisp_status crisp_route_cols(const crisp_dims* dims, const crisp_cfg* cfg, const float* col_mass,
                                        float* c_struct, int32_t* route, void* stream);

/* Step 3 - block selection (ai.info summary, "Methodology in Plain English";
 * ai-feeds summary, method module 2).
 *   VS heads: pooled vertical scores v[kb] (column mass of key block kb) and
 *   slash scores s[b] (mass at query-key offsets 128b..128b+127) from the
 *   proxy map; per direction the floor is alpha times the lower median (or
 *   mean) of blocks 1..N-1 (block 0 - the sink, or the local window - is
 *   always kept and excluded from the estimate); every block above the floor
 *   is kept, topped up to kmin_blocks by score (ties to the lower index).
 *   The list of qb is {kept vertical kb <= qb} U {qb-b, qb-b-1 : kept slash b},
 *   clipped to [0, qb].
 *   PE heads: mean-pool q and k over 128-token blocks, softmax of
 *   scale * qbar[qb] . kbar[kb] over kb <= qb, keep the shortest prefix of the
 *   descending order whose mass reaches gamma_pe, plus qb.
 * q, k, attn_map, block_mass: as above (the VS scores come from block_mass
 * when it is non-NULL, else from a pass over attn_map; at least one is
 * needed); route: [Hq] from crisp_route.  `workspace` must hold
 * crisp_select_workspace_bytes(dims) bytes of device memory. */
CRISP_API crisp_status crisp_select(const crisp_dims* dims, const crisp_cfg* cfg, const void* q, const void* k,
                          const float* attn_map, const float* block_mass, const int32_t* route,
                          const crisp_blocks* out, void* workspace, size_t workspace_bytes, void* stream);

/* Comparison chain - gamma-cumulative coverage on both paths (ai.info
 * summary, "Main Findings": the budget rule CRISP replaces on VS heads,
 * and the routing-only ablation).  Same as crisp_select except that each VS
 * direction keeps the shortest prefix of its blocks (block 0 included) in
 * descending score order whose mass reaches `gamma`, then block 0 and the
 * kmin top-up; PE heads use `gamma` instead of cfg->gamma_pe.
 * gamma in (0, 1]. */
CRISP_API crisp_status crisp_select_gamma(const crisp_dims* dims, const crisp_cfg* cfg, float gamma, const void* q,
                                const void* k, const float* attn_map, const float* block_mass,
                                const int32_t* route, const crisp_blocks* out, void* workspace,
                                size_t workspace_bytes, void* stream);

CRISP_API size_t crisp_select_workspace_bytes(const crisp_dims* dims);

/* crisp_select without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP stream capture, tight serving
 * loops, harnesses that forbid allocation.  Arguments, results and errors
 * are those of crisp_select.  The workspace is a static per-device buffer
 * inside the library of CRISP_NOALLOC_SCRATCH_BYTES (32 MiB), held on every
 * device the library runs on until the process ends; a layer whose
 * crisp_select_workspace_bytes exceeds it is CRISP_ERR_WORKSPACE (every
 * layer up to 524288 tokens with up to 64 query and 8 KV heads fits).  The
 * call allocates nothing and needs no zeroed memory: every kernel writes the
 * scratch it reads.  The buffer is shared by every call on a device and
 * keeps the last call's contents, so calls that overlap on one device (two
 * streams, or two threads) race: serialise them. */
#define CRISP_NOALLOC_SCRATCH_BYTES (32u << 20)

CRISP_API crisp_status crisp_select_noalloc(const crisp_dims* dims, const crisp_cfg* cfg, const void* q,
                                            const void* k, const float* attn_map, const float* block_mass,
                                            const int32_t* route, const crisp_blocks* out, void* stream);

/* Number of int32 entries crisp_blocks.idx must hold: Hq * N(N+1)/2. */
CRISP_API size_t crisp_list_capacity(const crisp_dims* dims);

/* Step 4 - exact block-sparse causal attention (ai.info summary, "Why This
 * Matters": exact softmax attention over the selected blocks).  For a query
 * i in block qb the keys are every j <= i lying in a key block of qb's list:
 *   out[h][i] = sum_j softmax_j(scale * q[h][i] . k[g][j]) v[g][j]
 * count/idx: the lists produced by crisp_select (entries must satisfy
 * 0 <= kb <= qb, strictly ascending, last entry qb; count >= 1).  A list
 * that breaks this is read defensively: count is clamped to [1, qb+1], the
 * last entry is taken as qb whatever it holds, and every other entry is
 * clamped to [0, qb-1].  So no key after a query is ever weighted and every
 * read stays inside the head's rows; the result is only meaningful for a
 * well-formed list (a repeated entry counts its keys twice, or once when
 * the call takes the two-block schedule described below).
 * Schedule: the call sums, over every head and pair of query blocks
 * (2p, 2p+1), own = cA + cB and bound = min(cA + cB, 2p + 2) on the size
 * of the union of the two lists.  When 2 sum(bound) <= 1.035 sum(own)
 * (dense and near-dense lists) one workgroup walks the union of a pair's
 * lists for both blocks and loads each K/V tile once; otherwise each
 * (head, query block) is an item of its own, dealt to the XCDs in runs of
 * 16 adjacent query blocks when the lists hold at most 64 tiles per item on
 * average and N is a multiple of 128.  Either way the result is the same
 * exact attention, up to rounding.
 * out: [Hq][n][d], bf16 when out_is_fp32 = 0, fp32 otherwise.
 * lse (optional, [Hq][n] fp32): natural log of each row's sum of exp.
 * workspace: crisp_attn_workspace_bytes(dims) bytes of device memory, any
 * contents; it holds the work queue the kernel's workgroups take items
 * from and the schedule sums, cleared by the call on `stream` (so two calls
 * in flight at once need two workspaces).  Smaller: CRISP_ERR_WORKSPACE. */
CRISP_API crisp_status crisp_sparse_attn(const crisp_dims* dims, const void* q, const void* k, const void* v,
                               const int32_t* count, const int32_t* idx, void* out, int32_t out_is_fp32,
                               float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* Dense causal attention with the same kernels and output conventions
 * (every key block 0..qb): the exact baseline the speedups are measured
 * against (ai.info summary, "Main Findings").  It takes the schedule
 * crisp_sparse_attn takes for full lists (two blocks per workgroup from 32
 * blocks on), so the two agree bit for bit on full lists.  workspace: as
 * crisp_sparse_attn. */
CRISP_API crisp_status crisp_dense_attn(const crisp_dims* dims, const void* q, const void* k, const void* v, void* out,
                              int32_t out_is_fp32, float* lse, void* workspace, size_t workspace_bytes,
                              void* stream);

/* Bytes of the workspace crisp_sparse_attn, crisp_dense_attn and
 * crisp_sparse_attn_cols take (0 for unsupported dims). */
CRISP_API size_t crisp_attn_workspace_bytes(const crisp_dims* dims);

/* Token-granular Vertical-Slash (ai-feeds summary, method module 2: keep
 * the tokens whose mass stands clearly above the noise floor; ai.info
 * summary, "Methodology in Plain English": k_min = 1024 tokens).  Vertical
 * columns are selected one by one; slash bands keep the block rule (kept
 * single offsets far from the diagonal scatter over nearly every band).
 * The chain is crisp_proxy_cols -> crisp_route -> crisp_select_tokens ->
 * crisp_sparse_attn (fp32 out, with lse) -> crisp_sparse_attn_cols. */

/* Proxy with the block masses (as crisp_proxy) and the column masses:
 *   col_mass[h][j] = (1/128) sum_r attn_map[h][r][j]          [Hq][n] fp32
 * without writing the map.  Arguments otherwise as crisp_proxy. */
CRISP_API crisp_status crisp_proxy_cols(const crisp_dims* dims, const void* q, const void* k, float* block_mass,
                              float* col_mass, float* row_lse, void* partials, size_t partials_bytes,
                              void* stream);

/* Selection as crisp_select (block_mass required), except the vertical
 * direction of VS heads: columns 0..127 (the sink tile) are always kept and
 * excluded from the floor; the floor is alpha times the lower median (or
 * mean) of col_mass over columns 128..n-1; every column above it is kept,
 * topped up to kmin_blocks * 128 columns in all by the best remaining ones
 * (descending mass, ties to the lower index).  The tile lists then hold key
 * block 0, the slash bands' tiles and the diagonal; out->v_mask is block 0
 * only, out->floor_v the column floor and out->n_v the kept columns in all.
 *   cols      [Hq][n] int32: kept columns >= 128 of head h, ascending, in
 *             cols[h][0 .. ncols[h]) (0 for PE heads)
 *   ncols     [Hq] int32
 *   col_below [Hq][N] int32: how many of them lie below 128 qb
 * The column floor, the top-up cut and the compaction are exact and
 * deterministic (radix selects and in-order scans). */
CRISP_API crisp_status crisp_select_tokens(const crisp_dims* dims, const crisp_cfg* cfg, const void* q, const void* k,
                                 const float* block_mass, const float* col_mass, const int32_t* route,
                                 const crisp_blocks* out, int32_t* cols, int32_t* ncols, int32_t* col_below,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* Adds the kept columns to a tile attention already in `out` (fp32,
 * [Hq][n][d]) and `lse` ([Hq][n], natural log), as written by
 * crisp_sparse_attn on the same count/idx.  For query i in block qb the
 * key set becomes the listed tiles (keys j <= i) plus the columns
 * cols[h][0 .. col_below[h][qb]) that lie outside the listed tiles; the two
 * softmaxes are merged exactly and out/lse updated in place.  Column
 * entries are clamped to [0, 128 qb - 1] and counts to [0, n]; entries must
 * be distinct for the result to mean anything.  workspace: as
 * crisp_sparse_attn (crisp_attn_workspace_bytes bytes, any contents). */
CRISP_API crisp_status crisp_sparse_attn_cols(const crisp_dims* dims, const void* q, const void* k, const void* v,
                                    const int32_t* count, const int32_t* idx, const int32_t* cols,
                                    const int32_t* col_below, float* out, float* lse, void* workspace,
                                    size_t workspace_bytes, void* stream);

/* Comparison routing signal - FlexPrefill's Jensen-Shannon routing, the one
 * C_struct replaces (ai.info summary, "Key Contributions" items 1 and 2:
 * C_struct drops its pooled matmul and KL divergence and reproduces its
 * decisions; "Methodology in Plain English": a pooled attention estimate is
 * compared with the per-query attention to decide whether a head is
 * concentrated).  The pages give no formula; this computes, per query head h
 * of KV group g:
 *   qbar       = mean of q[h] rows n-128 .. n-1 (the proxy rows)
 *   kbar[kb]   = mean of k[g] rows 128kb .. min(128kb+127, n-1)
 *   est[kb]    = softmax over all N key blocks of scale * qbar . kbar[kb]
 *   a[kb]      = (block_mass[0][h][kb] + [1][h][kb] + [2][h][kb]) / 128, the
 *                proxy map summed per key block and averaged over its rows
 *   js_dist[h] = sqrt(JSD(a, est)), natural log (0 .. sqrt(ln 2))
 *   route[h]   = CRISP_ROUTE_VS when js_dist >= tau_jsd, else CRISP_ROUTE_PE.
 * block_mass: [4][Hq][N] from crisp_proxy.  js_dist [Hq] fp32, route [Hq]
 * int32; estimate (optional, [Hq][N] fp32) receives est.  tau_jsd >= 0,
 * finite (CRISP_ERR_PARAM otherwise).  `workspace` must hold
 * crisp_route_jsd_workspace_bytes(dims) bytes of device memory.  Reads all
 * of K once: this is the extra pass C_struct does without. */
CRISP_API crisp_status crisp_route_jsd(const crisp_dims* dims, float tau_jsd, const void* q, const void* k,
                             const float* block_mass, float* js_dist, int32_t* route, float* estimate,
                             void* workspace, size_t workspace_bytes, void* stream);

CRISP_API size_t crisp_route_jsd_workspace_bytes(const crisp_dims* dims);

/* One layer in one call, with the context-length gate (ai.info summary,
 * "Main Findings": the point where sparse prefill starts to pay lies between
 * 8K and 64K tokens; "Why This Matters": gate sparse prefill on a
 * context-length threshold).
 *   n <  gate: crisp_dense_attn alone (blocks, block_mass, c_struct and route
 *              are then not written);
 *   n >= gate: crisp_proxy (block masses only) -> crisp_route (from the block
 *              masses) -> crisp_select -> crisp_sparse_attn, in that order on
 *              `stream`.
 * gate = dense_below, or CRISP_DENSE_BELOW_DEFAULT when dense_below < 0;
 * dense_below = 0 always runs the sparse chain.  The default is the length
 * from which the route-auto chain recovers its proxy, routing and selection
 * cost on MI355X (Llama-3.1-8B-shaped layers: 0.90x of the dense kernel at
 * 8K tokens, 1.00x or better from 16K on).
 * cfg: as crisp_route / crisp_select; sink_width and recency_width must be
 * 128 (routing reads the block masses; CRISP_ERR_PARAM otherwise).
 * blocks: as crisp_select (count and idx required, diagnostics optional).
 * block_mass ([4][Hq][N] fp32), c_struct ([Hq] fp32), route ([Hq] int32):
 * optional copies of the intermediate results (NULL: kept in the workspace).
 * out, out_is_fp32, lse: as crisp_sparse_attn.
 * workspace: crisp_prefill_workspace_bytes(dims) bytes of device memory.
 * That size is at least crisp_proxy_scratch_bytes rounded up to a multiple
 * of 256 plus crisp_select_workspace_bytes, so one buffer can also serve the
 * step-by-step calls (proxy scratch at its start, selection workspace at
 * that rounded offset).
 * Every argument is validated before anything is launched, whichever branch
 * the gate takes.  A launch failure part-way returns CRISP_ERR_LAUNCH with
 * the earlier steps already enqueued. */
#define CRISP_DENSE_BELOW_DEFAULT 16384

CRISP_API crisp_status crisp_prefill(const crisp_dims* dims, const crisp_cfg* cfg, int32_t dense_below,
                                     const void* q, const void* k, const void* v, const crisp_blocks* blocks,
                                     float* block_mass, float* c_struct, int32_t* route, void* out,
                                     int32_t out_is_fp32, float* lse, void* workspace, size_t workspace_bytes,
                                     void* stream);

CRISP_API size_t crisp_prefill_workspace_bytes(const crisp_dims* dims);

/* Static description of a status code. */
CRISP_API const char* crisp_status_string(crisp_status status);

/* ABI version, (major << 16) | minor. */
CRISP_API int32_t crisp_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CRISP_H */
