"""Comparators between the HIP path and the fp64 oracle.

Tolerances (applied element by element):
  * route: exact, unless C_struct is within 1e-3 relative of tau;
  * C_struct: 1e-4 relative;
  * selected sets: exact, except blocks whose oracle score lies within 1e-3
    relative of the decision boundary (the floor, the k_min cut, or the
    gamma cut); a gamma prefix may differ in length by one when the oracle's
    running sum crosses gamma within 1e-3 relative;
  * attention: max-abs 1e-2 and mean-abs 1e-3 against fp64, on identical lists.
  * attention lse: the kernels sum the bf16-rounded probabilities that enter
    the PV product (so a row is an exact weighted mean of V rows); each is
    within a relative 2^-8 of the exact one, so the log of the sum is within
    ln(1 + 2^-8) < 2^-8 of the oracle's, plus 2e-5 for the fp32 parts.
  * JSD routing signal: the pooled estimate 1e-4 relative per key block
    (fp32 logits, errors of order 1e-6 in the exponent); the divergence
    JSD = dist^2 within 2e-6 absolute plus 1e-4 relative (the kernel reads
    the block masses, each within about 1e-5 relative of the oracle's, and
    JSD moves by at most ln(2)/2 per unit of mass moved); the route as
    above, with the distance in place of C_struct.
"""
from __future__ import annotations

import math
from typing import List, Sequence

import numpy as np
import torch

from oracle import crisp_oracle as O

REL_SEL = 1e-3
REL_CSTRUCT = 1e-4
ATTN_MAXABS = 1e-2
ATTN_MEANABS = 1e-3
LSE_ABS = 2.0 ** -8 + 2e-5
REL_JSD_EST = 1e-4
JSD_ABS = 2e-6
JSD_REL = 1e-4


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def gpu_lists(count: np.ndarray, idx: np.ndarray, h: int, N: int) -> List[List[int]]:
    base = h * (N * (N + 1) // 2)
    out = []
    for qb in range(N):
        s = base + qb * (qb + 1) // 2
        out.append(idx[s:s + int(count[h, qb])].tolist())
    return out


def near(x: float, ref: float, rel: float = REL_SEL) -> bool:
    return abs(x - ref) <= rel * abs(ref)


def check_route(c_oracle: float, tau: float, route_gpu: int, route_oracle: int):
    if route_gpu != route_oracle:
        assert near(c_oracle, tau), f"route differs with C_struct={c_oracle} far from tau={tau}"


def check_noise_floor_mask(x: np.ndarray, alpha: float, kmin: int, stat: int, mask_gpu: np.ndarray,
                           floor_gpu: float):
    mask_o, T = O.noise_floor_select(x, alpha, kmin, stat)
    assert near(floor_gpu, T), f"floor {floor_gpu} vs oracle {T}"
    N = x.shape[0]
    cand = list(range(1, N))
    order = O._order_desc(x, cand)
    bounds = [T]
    want = min(kmin, N)
    if want - 1 >= 1:
        bounds.append(float(x[order[want - 2]]))
    diff = np.nonzero(mask_o != mask_gpu.astype(bool))[0]
    for b in diff:
        assert b != 0, "block 0 must always be kept"
        assert any(near(float(x[b]), t) for t in bounds), (
            f"block {b} (score {x[b]}) differs away from the boundaries {bounds}")
    return mask_o


def check_token_cols(c: np.ndarray, alpha: float, kmin_tokens: int, stat: int, cols_gpu: Sequence[int],
                     floor_gpu: float, retained: int = 128):
    """Kept columns past the retained ones: exact, except columns whose
    oracle mass lies within REL_SEL of the floor or of the k_min cut."""
    mask_o, T = O.token_noise_floor_select(c, alpha, kmin_tokens, retained, stat)
    assert near(floor_gpu, T), f"column floor {floor_gpu} vs oracle {T}"
    n = c.shape[0]
    got = np.zeros(n, dtype=bool)
    got[:retained] = True
    cols = np.asarray(cols_gpu, dtype=np.int64)
    assert np.all(np.diff(cols) > 0), "kept columns must be ascending without repeats"
    assert cols.size == 0 or cols[0] >= retained
    got[cols] = True
    bounds = [T]
    want = min(kmin_tokens, n)
    if want - retained >= 1:
        order = O._order_desc(c, list(range(retained, n)))
        bounds.append(float(c[order[want - retained - 1]]))
    diff = np.nonzero(mask_o != got)[0]
    for j in diff:
        assert any(near(float(c[j]), t) for t in bounds), (
            f"column {j} (mass {c[j]}) differs away from the boundaries {bounds}")
    return mask_o


def gamma_candidates(x: np.ndarray, items: Sequence[int], gamma: float):
    """Prefix lengths the GPU may legitimately take, with the cut score of each."""
    order = O._order_desc(x, list(items))
    cums = np.cumsum(x[order])
    K = len(O.gamma_prefix(x, gamma, items))
    ks = {K}
    if K >= 2 and cums[K - 2] >= gamma * (1 - REL_SEL):
        ks.add(K - 1)
    if K < len(order) and cums[K - 1] <= gamma * (1 + REL_SEL):
        ks.add(K + 1)
    return order, sorted(ks)


def check_gamma_set(x: np.ndarray, items: Sequence[int], gamma: float, got: set, always: set,
                    extra_fill: int = 0):
    """`got` must equal some admissible prefix (plus `always`, plus a k_min
    fill to `extra_fill` blocks) up to swaps of near-equal scores at the cut."""
    order, ks = gamma_candidates(x, items, gamma)
    errs = []
    for K in ks:
        ref = set(order[:K]) | set(always)
        pos = K
        while len(ref) < extra_fill and pos < len(order):
            ref.add(order[pos])
            pos += 1
        cut_scores = [float(x[order[K - 1]])]
        if pos > K:
            cut_scores.append(float(x[order[pos - 1]]))
        diff = (ref ^ got) - set(always)
        bad = [b for b in diff if not any(near(float(x[b]), c) for c in cut_scores)]
        if not bad:
            return
        errs.append((K, sorted(bad)[:8]))
    raise AssertionError(f"gamma set differs beyond the near-cut exemption: {errs}")


def check_pe_lists(qbar: np.ndarray, kbar: np.ndarray, scale: float, gamma: float, lists_gpu, qbs=None):
    N = qbar.shape[0]
    qbs = range(N) if qbs is None else qbs
    for qb in qbs:
        p = O.pe_row_probs(qbar, kbar, qb, scale)
        got = set(lists_gpu[qb])
        assert lists_gpu[qb] == sorted(got), "lists must be ascending without repeats"
        assert qb in got
        check_gamma_set(p, range(qb + 1), gamma, got, {qb})


def check_lse(lse_gpu: np.ndarray, lse_ref: np.ndarray, what: str = ""):
    err = np.abs(np.asarray(lse_gpu, dtype=np.float64) - lse_ref)
    assert err.max() <= LSE_ABS, f"{what} lse max-abs {err.max()}"


def check_attention(out_gpu: np.ndarray, out_ref: np.ndarray, what: str = ""):
    err = np.abs(out_gpu - out_ref)
    assert err.max() <= ATTN_MAXABS, f"{what} max-abs {err.max()}"
    assert err.mean() <= ATTN_MEANABS, f"{what} mean-abs {err.mean()}"
    return float(err.max()), float(err.mean())
