"""Plain fp64 CPU oracle for CRISP's sparse prefill attention path.

TEST INFRASTRUCTURE ONLY.  This module is the slow, obviously-correct
definition that the HIP path is checked against.  Only the test suite, the
package's smoke check and the benchmark's CPU-baseline leg may import it; the
product path never does, and this module imports nothing from the product
(no kernels, headers, helpers or constants are shared).

Source: "CRISP: Cliff-awaRe Input-adaptive Sparse Prefilling with
Structural-Mass-Motivated Routing" (arXiv 2609.01925) as summarised on
  * the ai.info AI-summary page (sections "Key Contributions",
    "Methodology in Plain English", "Main Findings", "Why This Matters"),
  * the ai-feeds.com summary page (section "方法" / method, modules 1 and 2,
    and section "局限" / limitations),
  * the authors' abstract (reproduced on every page).

All arithmetic is float64.  Inputs arrive as float64 arrays that hold the
exact values of the bf16 tensors the GPU sees.  Array conventions:
  q  : [Hq][n][d]      k, v : [Hkv][n][d]
  GQA group of query head h is g(h) = h * Hkv // Hq (consecutive heads share).
  B  : block size (128); N = ceil(n / B) blocks, aligned at position 0.
       When B does not divide n the last block holds the n - B (N-1) last
       positions (reading R29); every quantity below stays defined token by
       token, so a partial block only has fewer keys, rows or offsets.

Where the pages leave a step open, the reading used here is named in the
function's docstring with its tag (R1..R29); the same tags are listed with
their justification in the repository's design notes.

Parity pins: every function below is pinned by tests that do not reuse its
own formula (closed forms, invariants, brute force on tiny inputs); see
tests/test_oracle_pins.py.  The one thing left unpinned is agreement with the
paper's own accuracy/latency numbers, which need trained models and an H100.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np

ROUTE_PE = 0
ROUTE_VS = 1

OVERRIDE_AUTO = 0
OVERRIDE_FORCE_VS = 1
OVERRIDE_FORCE_PE = 2

NF_MEDIAN = 0
NF_MEAN = 1


@dataclass
class OracleConfig:
    """Method constants.

    Defaults follow the ai.info summary, "Methodology in Plain English":
    block size 128, k_min of 1024 tokens (8 blocks) per direction, gamma 0.95
    on the Pooled-Estimation path, alpha in {1.0, 1.25} on the Vertical-Slash
    path; sink and recency windows of 128 tokens ("Key Contributions", item 2).
    tau defaults to the 0.5 of the synthetic workloads (the paper's universal
    setting is 0.2; reading R3).  alpha defaults to 1.25 (reading R8).
    """

    block: int = 128
    tau: float = 0.5
    alpha: float = 1.25
    gamma_pe: float = 0.95
    kmin_blocks: int = 8
    sink_width: int = 128
    recency_width: int = 128
    nf_stat: int = NF_MEDIAN
    route_override: int = OVERRIDE_AUTO


# ---------------------------------------------------------------------------
# Step 1: proxy attention map (ai.info "Key Contributions" item 2 and
# "Methodology in Plain English": C_struct reads a proxy attention map the
# method already computes).  Reading R1: the proxy rows are the last B query
# positions, causally masked.
# ---------------------------------------------------------------------------


def proxy_map(q_last: np.ndarray, k: np.ndarray, scale: float):
    """Softmax attention of the last B queries of one head against all keys.

    q_last : [B][d]  query rows at positions n-B .. n-1
    k      : [n][d]  keys of the head's GQA group
    Returns (A [B][n], lse [B]); A[r, j] = 0 for j > n - B + r (causal).
    lse is the natural log of the row's sum of exp(logit).
    """
    B = q_last.shape[0]
    n = k.shape[0]
    s = scale * (q_last @ k.T)  # [B][n], a library matmul as one step
    for r in range(B):
        i = n - B + r
        s[r, i + 1:] = -np.inf
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    l = e.sum(axis=1)
    A = e / l[:, None]
    lse = m + np.log(l)
    return A, lse


# ---------------------------------------------------------------------------
# Step 2: C_struct and routing (ai.info "Key Contributions" item 2,
# "Methodology in Plain English"; ai-feeds "方法", module 1).
# ---------------------------------------------------------------------------


def c_struct(A: np.ndarray, sink_width: int = 128, recency_width: int = 128) -> float:
    """Structural mass: row-mean of the proxy mass on the first `sink_width`
    and the last `recency_width` key columns (reading R2: absolute columns,
    normalised by the number of proxy rows so that C lies in [0, 1])."""
    B, n = A.shape
    total = A[:, :sink_width].sum() + A[:, n - recency_width:].sum()
    return float(total / B)


def route(c: float, tau: float, override: int = OVERRIDE_AUTO) -> int:
    """Vertical-Slash when C_struct >= tau, else Pooled-Estimation
    (reading R3; ties go to VS).  The override forces one path."""
    if override == OVERRIDE_FORCE_VS:
        return ROUTE_VS
    if override == OVERRIDE_FORCE_PE:
        return ROUTE_PE
    return ROUTE_VS if c >= tau else ROUTE_PE


# ---------------------------------------------------------------------------
# Step 3: Vertical-Slash scores.  Columns (vertical) and fixed query-key
# offsets (slash) of the proxy map (abstract: mass at Vertical-Slash
# compatible positions).  Readings R4, R5, R22.
# ---------------------------------------------------------------------------


def token_scores(A: np.ndarray):
    """Token-level vertical and slash mass of one head's proxy map.

    c[j]  = (1/B) * sum_r A[r, j]                     (column mass)
    dg[o] = (1/B) * sum_{r : i_r - o >= 0} A[r, i_r - o]   (offset mass)
    with i_r = n - B + r the absolute position of proxy row r.
    """
    B, n = A.shape
    c = A.sum(axis=0) / B
    dg = np.zeros(n, dtype=np.float64)
    for r in range(B):
        i = n - B + r
        # offsets o = 0..i map to keys j = i - o, i.e. the row read backwards
        dg[: i + 1] += A[r, i::-1]
    dg /= B
    return c, dg


def pooled_scores(c: np.ndarray, dg: np.ndarray, block: int = 128):
    """Block-pooled scores: v[kb] sums columns of key block kb; sl[s] sums
    offsets 128s .. 128s+127 (reading R5).  A partial last block or band
    sums the entries it has (reading R29)."""
    n = c.shape[0]
    N = -(-n // block)
    v = np.array([c[b * block:(b + 1) * block].sum() for b in range(N)])
    sl = np.array([dg[b * block:(b + 1) * block].sum() for b in range(N)])
    return v, sl


def block_masses(A: np.ndarray, block: int = 128, recency_width: int = 128):
    """Per key block kb, how the proxy map's mass in that block splits over
    the slash bands, and how much of it lies in the recency window.

    Reading R5 pools offsets in bands of 128: proxy row r (position
    i_r = n - B + r) against key j lies at offset o = i_r - j, in band
    o // 128.  Within key block kb every visible entry falls in band
    N-1-kb, N-2-kb or N-3-kb (the last only when 128 does not divide n,
    reading R29).  Returns four [N] arrays:
      lo[kb]  = mass of block kb in band N-1-kb,
      up[kb]  = mass of block kb in band N-2-kb,
      up2[kb] = mass of block kb in band N-3-kb,
      rec[kb] = mass of block kb on keys j >= n - recency_width.
    lo + up + up2 is the block's vertical mass; with 128 | n, up2 = 0, lo is
    the tile's mass on and below its diagonal (r >= column) and up the rest,
    and rec is nonzero in block N-1 only."""
    B, n = A.shape
    N = -(-n // block)
    planes = np.zeros(3 * N, dtype=np.float64)
    rec = np.zeros(N, dtype=np.float64)
    for r in range(B):
        i = n - B + r
        j = np.arange(i + 1)           # the keys row r sees
        kb = j // block
        d = (N - 1 - kb) - (i - j) // block
        a = A[r, : i + 1]
        planes += np.bincount(d * N + kb, weights=a, minlength=3 * N)
        inw = j >= n - recency_width
        rec += np.bincount(kb[inw], weights=a[inw], minlength=N)
    return planes[:N], planes[N:2 * N], planes[2 * N:], rec


# ---------------------------------------------------------------------------
# Step 4a: sink-aware noise-floor selection on Vertical-Slash heads
# (ai.info "Methodology in Plain English": expected background mass over the
# blocks that are not always retained, keep each block above alpha times it;
# ai-feeds "方法" module 2: floor e.g. the median of the background level).
# Readings R6, R7, R9, R10.
# ---------------------------------------------------------------------------


def lower_median(x: Sequence[float]) -> float:
    """Element at index floor((m-1)/2) of the ascending order (reading R7)."""
    xs = sorted(float(t) for t in x)
    return xs[(len(xs) - 1) // 2]


def _order_desc(x: np.ndarray, items: Sequence[int]) -> List[int]:
    """Items sorted by descending score, ties to the lower index."""
    return sorted(items, key=lambda i: (-float(x[i]), i))


def noise_floor_select(x: np.ndarray, alpha: float, kmin: int, stat: int = NF_MEDIAN):
    """Noise-floor selection over one direction's block scores.

    Block 0 (the sink for vertical, the local window for slash) is always
    retained and excluded from the floor estimate (R6).  The floor mu is the
    lower median (or the mean, for the ablation) of the remaining N-1 scores
    (R7); threshold T = alpha * mu; keep every candidate with x > T (R9).
    If fewer than min(kmin, N) blocks are kept (block 0 counts), add the
    best unselected candidates, ties to the lower index (R10).
    Returns (mask [N] bool, T).
    """
    N = x.shape[0]
    cand = list(range(1, N))
    if stat == NF_MEDIAN:
        mu = lower_median([x[b] for b in cand])
    else:
        mu = float(np.mean([x[b] for b in cand]))
    T = alpha * mu
    sel = {0}
    for b in cand:
        if x[b] > T:
            sel.add(b)
    want = min(kmin, N)
    if len(sel) < want:
        for b in _order_desc(x, [b for b in cand if b not in sel]):
            if len(sel) >= want:
                break
            sel.add(b)
    mask = np.zeros(N, dtype=bool)
    mask[sorted(sel)] = True
    return mask, T


# ---------------------------------------------------------------------------
# Step 4b: gamma-cumulative coverage (ai.info "Main Findings" and
# "Methodology in Plain English": accumulate the largest masses until the
# fixed coverage gamma is reached; kept by CRISP on the PE path only, and
# the comparison selector here).  Reading R11.
# ---------------------------------------------------------------------------


def gamma_prefix(x: np.ndarray, gamma: float, items: Optional[Sequence[int]] = None) -> List[int]:
    """Shortest prefix of the (descending score, ascending index) order whose
    fp64 running sum reaches gamma; all items if it never does."""
    if items is None:
        items = range(x.shape[0])
    order = _order_desc(x, list(items))
    taken = []
    acc = 0.0
    for i in order:
        taken.append(i)
        acc += float(x[i])
        if acc >= gamma:
            break
    return taken


def vs_gamma_select(x: np.ndarray, gamma: float, kmin: int):
    """gamma-cumulative selection on one VS direction for the comparison
    chain: prefix over all N blocks (block 0 included, which is what lets a
    heavy sink end the selection early), then block 0 and the k_min top-up,
    so that only the threshold rule differs from noise_floor_select (R11)."""
    N = x.shape[0]
    sel = set(gamma_prefix(x, gamma))
    sel.add(0)
    want = min(kmin, N)
    if len(sel) < want:
        for b in _order_desc(x, [b for b in range(N) if b not in sel]):
            if len(sel) >= want:
                break
            sel.add(b)
    mask = np.zeros(N, dtype=bool)
    mask[sorted(sel)] = True
    return mask


# ---------------------------------------------------------------------------
# Step 4c: Pooled-Estimation path (ai.info "Key Contributions" item 2 and
# "Methodology in Plain English": a pooled attention estimate; gamma = 0.95 on
# this path only).  Reading R12: mean-pool Q and K over 128-token blocks,
# block-causal softmax per query block, gamma prefix, plus the diagonal block.
# ---------------------------------------------------------------------------


def pe_pool(x: np.ndarray, block: int = 128) -> np.ndarray:
    """Mean of each block of `block` consecutive rows: [n][d] -> [N][d].
    A partial last block is the mean of the rows it has (reading R29)."""
    n, d = x.shape
    N = -(-n // block)
    return np.stack([x[b * block:(b + 1) * block].mean(axis=0) for b in range(N)])


def pe_row_probs(qbar: np.ndarray, kbar: np.ndarray, qb: int, scale: float) -> np.ndarray:
    """Softmax over kb in [0, qb] of scale * <Qbar[qb], Kbar[kb]>."""
    e = scale * (kbar[: qb + 1] @ qbar[qb])
    e = e - e.max()
    p = np.exp(e)
    return p / p.sum()


def pe_row_select(qbar: np.ndarray, kbar: np.ndarray, qb: int, scale: float, gamma: float) -> List[int]:
    """Key-block list of query block qb on a PE head (ascending)."""
    p = pe_row_probs(qbar, kbar, qb, scale)
    sel = set(gamma_prefix(p, gamma))
    sel.add(qb)
    return sorted(sel)


# ---------------------------------------------------------------------------
# Step 5: expansion of the Vertical-Slash sets into per-query-block key-block
# lists (ai-feeds "方法": the output is a per-head sparse mask used in
# prefill).  Reading R5: slash block s covers key blocks qb-s and qb-s-1.
# ---------------------------------------------------------------------------


def vs_list_row(vmask: np.ndarray, smask: np.ndarray, qb: int) -> List[int]:
    """Key-block list of query block qb: the kept vertical blocks up to qb
    and the two key blocks each kept slash band covers, ascending."""
    N = vmask.shape[0]
    sel = set()
    for kb in range(qb + 1):
        if vmask[kb]:
            sel.add(kb)
    for s in range(N):
        if smask[s]:
            for kb in (qb - s, qb - s - 1):
                if 0 <= kb <= qb:
                    sel.add(kb)
    return sorted(sel)


def vs_lists(vmask: np.ndarray, smask: np.ndarray) -> List[List[int]]:
    return [vs_list_row(vmask, smask, qb) for qb in range(vmask.shape[0])]


def dense_lists(N: int) -> List[List[int]]:
    return [list(range(qb + 1)) for qb in range(N)]


# ---------------------------------------------------------------------------
# Step 6: exact softmax attention over the selected blocks (ai.info "Why This
# Matters": exact softmax over the blocks it selects).  Reading R13: the
# diagonal block is always present, so no row is empty.
# ---------------------------------------------------------------------------


def attention_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, lists: Sequence[Sequence[int]],
                   scale: float, qbs: Sequence[int], block: int = 128):
    """Block-sparse causal attention of one head for the query blocks `qbs`.

    For query i in block qb the key set is the union of the listed key
    blocks, restricted to keys j <= i.  Returns {qb: (O [rows][d], lse [rows])}
    over the block's rows (fewer than `block` in a partial last block).
    """
    out = {}
    for qb in qbs:
        n = q.shape[0]
        kbs = sorted(set(int(t) for t in lists[qb]))
        keys = np.concatenate([np.arange(kb * block, min((kb + 1) * block, n)) for kb in kbs])
        rows = np.arange(qb * block, min((qb + 1) * block, n))
        s = scale * (q[rows] @ k[keys].T)
        s[keys[None, :] > rows[:, None]] = -np.inf
        m = s.max(axis=1)
        e = np.exp(s - m[:, None])
        l = e.sum(axis=1)
        O = (e @ v[keys]) / l[:, None]
        out[qb] = (O, m + np.log(l))
    return out


# ---------------------------------------------------------------------------
# Whole layer.
# ---------------------------------------------------------------------------


@dataclass
class HeadResult:
    c_struct: float
    route: int
    lse_proxy: np.ndarray
    v: np.ndarray
    sl: np.ndarray
    vmask: Optional[np.ndarray]
    smask: Optional[np.ndarray]
    floor_v: float
    floor_s: float
    lists: List[List[int]]
    attn: Dict[int, tuple] = field(default_factory=dict)
    A: Optional[np.ndarray] = None


def select_head(q_h: np.ndarray, k_g: np.ndarray, cfg: OracleConfig, scale: float,
                gamma: Optional[float] = None, keep_map: bool = False) -> HeadResult:
    """Proxy, route and selection of one query head.

    gamma=None runs CRISP (noise floor on VS heads, gamma_pe on PE heads);
    a float runs the gamma-cumulative comparison chain with that gamma on
    both paths (ai.info "Main Findings": the routing-only ablation).
    """
    B = cfg.block
    n = k_g.shape[0]
    A, lse = proxy_map(q_h[n - B:], k_g, scale)
    c = c_struct(A, cfg.sink_width, cfg.recency_width)
    rt = route(c, cfg.tau, cfg.route_override)
    ct, dg = token_scores(A)
    v, sl = pooled_scores(ct, dg, B)
    vmask = smask = None
    fv = fs = float("nan")
    if rt == ROUTE_VS:
        if gamma is None:
            vmask, fv = noise_floor_select(v, cfg.alpha, cfg.kmin_blocks, cfg.nf_stat)
            smask, fs = noise_floor_select(sl, cfg.alpha, cfg.kmin_blocks, cfg.nf_stat)
        else:
            vmask = vs_gamma_select(v, gamma, cfg.kmin_blocks)
            smask = vs_gamma_select(sl, gamma, cfg.kmin_blocks)
        lists = vs_lists(vmask, smask)
    else:
        g = cfg.gamma_pe if gamma is None else gamma
        qbar = pe_pool(q_h, B)
        kbar = pe_pool(k_g, B)
        lists = [pe_row_select(qbar, kbar, qb, scale, g) for qb in range(-(-n // B))]
    return HeadResult(c, rt, lse, v, sl, vmask, smask, fv, fs, lists, A=A if keep_map else None)


def run_layer(q: np.ndarray, k: np.ndarray, v: np.ndarray, cfg: OracleConfig,
              scale: Optional[float] = None, heads: Optional[Sequence[int]] = None,
              attn_qbs: Optional[Sequence[int]] = None, gamma: Optional[float] = None,
              keep_map: bool = False) -> Dict[int, HeadResult]:
    """The whole path for the listed heads (all by default); attention is
    evaluated on the query blocks `attn_qbs` (all by default)."""
    Hq, n, d = q.shape
    Hkv = k.shape[0]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if heads is None:
        heads = range(Hq)
    N = -(-n // cfg.block)
    qbs = list(range(N)) if attn_qbs is None else list(attn_qbs)
    res = {}
    for h in heads:
        g = h * Hkv // Hq
        hr = select_head(q[h], k[g], cfg, scale, gamma=gamma, keep_map=keep_map)
        if qbs:
            hr.attn = attention_rows(q[h], k[g], v[g], hr.lists, scale, qbs, cfg.block)
        res[h] = hr
    return res


# ---------------------------------------------------------------------------
# Comparison: FlexPrefill's routing signal, the one C_struct replaces
# (ai.info "Key Contributions" items 1 and 2: C_struct drops the pooled
# matmul and the KL divergence that JSD routing needs, and reproduces its
# decisions; "Methodology in Plain English": an extra pooled attention
# estimate is compared by Jensen-Shannon divergence with the per-query
# attention to decide whether a head is concentrated).  Readings R23-R25.
# ---------------------------------------------------------------------------


def jsd_estimate(q_last: np.ndarray, k: np.ndarray, scale: float, block: int = 128) -> np.ndarray:
    """Pooled attention estimate of the last query block over the N key
    blocks (reading R23): softmax over kb of scale * <qbar, kbar[kb]>, with
    qbar the mean of the B proxy query rows and kbar[kb] the mean of the
    keys of block kb.  Every key block is visible to the last query block,
    so no block is masked."""
    qbar = q_last.mean(axis=0)
    kbar = pe_pool(k, block)
    e = scale * (kbar @ qbar)
    p = np.exp(e - e.max())
    return p / p.sum()


def jsd_actual(A: np.ndarray, block: int = 128) -> np.ndarray:
    """The per-query attention of the proxy rows, summed over each key block
    and averaged over the rows: a distribution over the N key blocks."""
    B, n = A.shape
    N = -(-n // block)
    return np.array([A[:, b * block:(b + 1) * block].sum() for b in range(N)]) / B


def js_divergence(p: np.ndarray, q: np.ndarray) -> float:
    """Jensen-Shannon divergence in nats: the mean of KL(p || m) and
    KL(q || m), m the midpoint of p and q, with 0 log 0 = 0."""
    m = 0.5 * (p + q)

    def kl(a):
        nz = a > 0
        return float(np.sum(a[nz] * np.log(a[nz] / m[nz])))

    return 0.5 * kl(p) + 0.5 * kl(q)


def jsd_route(p_est: np.ndarray, a_bar: np.ndarray, tau_jsd: float):
    """Jensen-Shannon distance sqrt(JSD) between the block-summed proxy and
    the pooled estimate, and the route it implies (reading R24): a head whose
    attention the pooled estimate misses by at least tau_jsd is concentrated
    and goes Vertical-Slash; otherwise Pooled-Estimation.  Ties go to VS."""
    d = math.sqrt(max(js_divergence(a_bar, p_est), 0.0))
    return d, (ROUTE_VS if d >= tau_jsd else ROUTE_PE)


# ---------------------------------------------------------------------------
# Token-granular Vertical-Slash selection (ai-feeds "方法", module 2: keep the
# tokens whose mass stands clearly above the noise floor; ai.info
# "Methodology in Plain English": k_min = 1024 tokens per direction).
# Readings R26-R28.
# ---------------------------------------------------------------------------


def token_noise_floor_select(x: np.ndarray, alpha: float, kmin_tokens: int, retained: int = 128,
                             stat: int = NF_MEDIAN):
    """Noise floor over one direction's token scores (reading R26).

    Entries 0 .. retained-1 (the sink columns for vertical, the local
    offsets for slash) are always kept and excluded from the floor estimate.
    The floor is the lower median (or the mean) of the other entries; every
    other entry above alpha times the floor is kept.  If fewer than
    min(kmin_tokens, n) entries are kept in all, the best unkept entries
    (descending score, ties to the lower index) are added until there are.
    Returns (mask [n] bool, T)."""
    n = x.shape[0]
    cand = list(range(retained, n))
    if stat == NF_MEDIAN:
        mu = lower_median([x[j] for j in cand])
    else:
        mu = float(np.mean([x[j] for j in cand]))
    T = alpha * mu
    sel = set(range(retained))
    for j in cand:
        if x[j] > T:
            sel.add(j)
    want = min(kmin_tokens, n)
    if len(sel) < want:
        for j in _order_desc(x, [j for j in cand if j not in sel]):
            if len(sel) >= want:
                break
            sel.add(j)
    mask = np.zeros(n, dtype=bool)
    mask[sorted(sel)] = True
    return mask, T


@dataclass
class TokenPlan:
    vmask: np.ndarray       # [n] kept vertical columns
    floor_v: float          # token floor of the vertical direction
    smask: np.ndarray       # [N] kept slash bands (block-level rule)
    floor_s: float
    cols: List[int]         # kept columns outside key block 0, ascending
    lists: List[List[int]]  # per query block: listed key blocks (tiles)


def token_vs_plan(c: np.ndarray, sl: np.ndarray, alpha: float, kmin_tokens: int, kmin_blocks: int,
                  block: int = 128, stat: int = NF_MEDIAN) -> TokenPlan:
    """What a Vertical-Slash head computes under token-granular vertical
    selection.

    Reading R26: the vertical direction keeps columns by the token floor
    over the column masses c.  Reading R27: the slash direction keeps its
    block rule on the band scores sl (offsets far from the diagonal carry
    background mass only, so kept single offsets would scatter over nearly
    every band and a tile cover of them would be almost dense).  Key block 0
    holds the retained sink columns and is always a tile.  Reading R28:
    every kept column outside key block 0 is read one by one, by every query
    block past it, on top of the tiles."""
    N = -(-c.shape[0] // block)
    vmask, Tv = token_noise_floor_select(c, alpha, kmin_tokens, block, stat)
    smask, Ts = noise_floor_select(sl, alpha, kmin_blocks, stat)
    vblocks = np.zeros(N, dtype=bool)
    vblocks[0] = True
    cols = [int(j) for j in np.nonzero(vmask)[0] if j >= block]
    return TokenPlan(vmask, Tv, smask, Ts, cols, vs_lists(vblocks, smask))


def attention_rows_mixed(q: np.ndarray, k: np.ndarray, v: np.ndarray, lists: Sequence[Sequence[int]],
                         cols: Sequence[int], scale: float, qbs: Sequence[int], block: int = 128):
    """Causal attention of one head over listed tiles plus single key
    columns: for query i in block qb the key set is every key j <= i that
    lies in a listed key block of qb or is one of `cols`.  Each key counts
    once.  Returns {qb: (O [block][d], lse [block])}."""
    out = {}
    n = q.shape[0]
    col_set = set(int(j) for j in cols)
    for qb in qbs:
        keys = set()
        for kb in lists[qb]:
            keys.update(range(int(kb) * block, min((int(kb) + 1) * block, n)))
        keys.update(j for j in col_set if j < (qb + 1) * block)
        keys = np.array(sorted(keys), dtype=np.int64)
        rows = np.arange(qb * block, min((qb + 1) * block, n))
        s = scale * (q[rows] @ k[keys].T)
        s[keys[None, :] > rows[:, None]] = -np.inf
        m = s.max(axis=1)
        e = np.exp(s - m[:, None])
        l = e.sum(axis=1)
        O = (e @ v[keys]) / l[:, None]
        out[qb] = (O, m + np.log(l))
    return out
