"""Pins of the fp64 oracle against closed forms, invariants and brute force.

None of these re-types the oracle's own formula: each check derives the
expected value another way (a closed form for a planted input, an identity
between two independently computed quantities, or exhaustive search), so a
dropped term, a wrong sign or index, or a transposed operand fails one.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import crisp_oracle as O

B = 128
HERE = os.path.dirname(os.path.abspath(__file__))


def _rng(seed):
    return np.random.default_rng(seed)


# --------------------------------------------------------------------------
# constants printed on the pages
# --------------------------------------------------------------------------


def test_constants_match_pages():
    with open(os.path.join(HERE, "golden", "crisp_constants.json")) as f:
        g = json.load(f)
    cfg = O.OracleConfig()
    assert cfg.block == g["block_size"]["value"]
    assert cfg.kmin_blocks * cfg.block == g["kmin_tokens"]["value"]
    assert cfg.kmin_blocks == g["kmin_blocks"]["value"]
    assert cfg.gamma_pe == g["gamma_pe"]["value"]
    assert cfg.alpha in g["alpha_vs"]["value"]
    assert cfg.sink_width == g["sink_width"]["value"]
    assert cfg.recency_width == g["recency_width"]["value"]
    # the synthetic workloads use tau = 0.5; the paper's universal value is kept on record
    assert g["tau_proxy_paper"]["value"] == 0.2


# --------------------------------------------------------------------------
# proxy map
# --------------------------------------------------------------------------


def test_proxy_rows_sum_to_one_and_causal():
    rng = _rng(1)
    n, d = 640, 128
    q = rng.standard_normal((B, d))
    k = rng.standard_normal((n, d))
    A, lse = O.proxy_map(q, k, 1 / math.sqrt(d))
    assert A.shape == (B, n)
    np.testing.assert_allclose(A.sum(axis=1), 1.0, rtol=0, atol=1e-13)
    for r in range(B):
        assert np.all(A[r, n - B + r + 1:] == 0.0)
        assert np.all(A[r, : n - B + r + 1] > 0.0)


def test_proxy_zero_query_closed_form():
    # Q = 0: every visible logit is 0, so row r is uniform over i_r + 1 keys.
    rng = _rng(2)
    n, d = 512, 64
    k = rng.standard_normal((n, d))
    A, lse = O.proxy_map(np.zeros((B, d)), k, 0.3)
    for r in range(B):
        i = n - B + r
        np.testing.assert_allclose(A[r, : i + 1], 1.0 / (i + 1), rtol=1e-14)
        assert lse[r] == pytest.approx(math.log(i + 1), rel=1e-14)


def test_proxy_two_level_closed_form():
    # Keys in S are t*u, the rest are orthogonal to u; queries are s*u.
    # A visible key in S has weight e^x / Z, any other 1 / Z, with
    # x = scale * s * t and Z = |S_i| e^x + (i + 1 - |S_i|).
    rng = _rng(3)
    n, d = 768, 32
    scale = 1 / math.sqrt(d)
    s_amp, t_amp = 2.0, 3.5
    u = np.zeros(d)
    u[0] = 1.0
    k = rng.standard_normal((n, d))
    k[:, 0] = 0.0
    S = np.sort(rng.choice(n, 40, replace=False))
    k[S] = t_amp * u
    q = np.tile(s_amp * u, (B, 1))
    A, _ = O.proxy_map(q, k, scale)
    x = scale * s_amp * t_amp
    inS = np.zeros(n, bool)
    inS[S] = True
    for r in range(B):
        i = n - B + r
        cnt = int(inS[: i + 1].sum())
        Z = cnt * math.exp(x) + (i + 1 - cnt)
        exp_row = np.where(inS[: i + 1], math.exp(x) / Z, 1.0 / Z)
        np.testing.assert_allclose(A[r, : i + 1], exp_row, rtol=1e-12)


# --------------------------------------------------------------------------
# C_struct and routing
# --------------------------------------------------------------------------


def test_cstruct_equals_hand_sum_of_slices():
    rng = _rng(4)
    n, d = 384, 128
    q = rng.standard_normal((B, d))
    k = rng.standard_normal((n, d))
    k[:4] += 6.0 * q.mean(axis=0) / np.linalg.norm(q.mean(axis=0))
    A, _ = O.proxy_map(q, k, 1 / math.sqrt(d))
    hand = 0.0
    for r in range(B):
        for j in range(128):
            hand += A[r, j]
        for j in range(n - 128, n):
            hand += A[r, j]
    assert O.c_struct(A) == pytest.approx(hand / B, rel=1e-13)


def test_cstruct_zero_query_closed_form():
    # Q = 0: row r holds 128 sink keys and r + 1 recency keys out of n - 127 + r.
    for n in (256, 1024, 4096):
        A, _ = O.proxy_map(np.zeros((B, 16)), np.ones((n, 16)), 1.0)
        closed = sum((129 + r) / (n - 127 + r) for r in range(B)) / B
        assert O.c_struct(A) == pytest.approx(closed, rel=1e-13)
    # near the midpoint approximation 192.5 / (n - 63.5) (convexity of 1/x
    # puts the exact mean slightly below it)
    assert closed == pytest.approx(192.5 / (4096 - 63.5), rel=2e-3)
    assert closed < 192.5 / (4096 - 63.5)


def test_cstruct_identity_with_pooled_vertical_scores():
    # With 128-wide windows, C = v[0] + v[N-1]: two independent code paths.
    rng = _rng(5)
    n, d = 1024, 64
    A, _ = O.proxy_map(rng.standard_normal((B, d)), rng.standard_normal((n, d)), 0.2)
    c, dg = O.token_scores(A)
    v, sl = O.pooled_scores(c, dg)
    assert O.c_struct(A) == pytest.approx(v[0] + v[-1], rel=1e-13)


def test_route_rule():
    assert O.route(0.5, 0.5) == O.ROUTE_VS
    assert O.route(0.4999, 0.5) == O.ROUTE_PE
    assert O.route(0.9, 0.5, O.OVERRIDE_FORCE_PE) == O.ROUTE_PE
    assert O.route(0.0, 0.5, O.OVERRIDE_FORCE_VS) == O.ROUTE_VS


# --------------------------------------------------------------------------
# vertical / slash scores
# --------------------------------------------------------------------------


def test_scores_sum_to_one_and_tile_triangle_identity():
    # Pooled slash scores from the per-tile total T and lower triangle L:
    # row r (position 128(N-1)+r) against key 128kb+c has offset
    # 128(N-1-kb) + (r-c), so r >= c lands in slash block N-1-kb, r < c in N-2-kb.
    rng = _rng(6)
    n, d = 1280, 64
    A, _ = O.proxy_map(rng.standard_normal((B, d)), rng.standard_normal((n, d)), 0.25)
    c, dg = O.token_scores(A)
    v, sl = O.pooled_scores(c, dg)
    assert v.sum() == pytest.approx(1.0, abs=1e-13)
    assert sl.sum() == pytest.approx(1.0, abs=1e-13)
    N = n // B
    lower = np.tril(np.ones((B, B), bool))  # r >= c
    sl_t = np.zeros(N)
    for kb in range(N):
        tile = A[:, kb * B:(kb + 1) * B]
        T = tile.sum()
        L = tile[lower].sum()
        U = tile[~lower].sum()  # = T - L
        np.testing.assert_allclose(v[kb], T / B, rtol=1e-12)
        sl_t[N - 1 - kb] += L / B
        if N - 2 - kb >= 0:
            sl_t[N - 2 - kb] += U / B
        else:
            assert U == 0.0  # the masked upper triangle of the diagonal tile
    np.testing.assert_allclose(sl, sl_t, rtol=1e-12, atol=1e-18)


@pytest.mark.parametrize("n", [1536, 1499, 300, 257])
def test_block_masses_give_vertical_slash_and_c_struct(n):
    # block_masses is pinned by quantities computed along other routes: the
    # column sums (v), the diagonal loop (sl) and the slice sums (C_struct).
    # 1499, 300 and 257 leave a partial last block (43, 44 and 1 positions).
    rng = _rng(16)
    d = 64
    A, _ = O.proxy_map(rng.standard_normal((B, d)), rng.standard_normal((n, d)), 0.3)
    lo, up, up2, rec = O.block_masses(A)
    v, sl = O.pooled_scores(*O.token_scores(A))
    N = -(-n // B)
    assert len(lo) == N
    np.testing.assert_allclose((lo + up + up2) / B, v, rtol=1e-12)
    sl_b = np.zeros(N)
    for s in range(N):
        sl_b[s] = lo[N - 1 - s] + (up[N - 2 - s] if s <= N - 2 else 0.0) + (up2[N - 3 - s] if s <= N - 3 else 0.0)
    np.testing.assert_allclose(sl_b / B, sl, rtol=1e-12, atol=1e-18)
    # with 128 | n the tile splits at its diagonal only; with a partial last
    # block its neighbour N-2 is fully visible and holds part of the window
    if n % B == 0:
        assert np.all(up2 == 0.0)
        assert up[N - 1] == 0.0  # the masked half of the diagonal tile
        assert np.all(rec[: N - 1] == 0.0)
    else:
        assert up2[: N - 2].sum() > 0.0
        assert rec[N - 2] > 0.0
    assert np.all(rec[: N - 2] == 0.0)
    np.testing.assert_allclose(rec[N - 1], lo[N - 1] + up[N - 1] + up2[N - 1], rtol=1e-12)
    c = (lo[0] + up[0] + up2[0] + rec.sum()) / B
    assert c == pytest.approx(O.c_struct(A), rel=1e-12)


@pytest.mark.parametrize("n", [768, 700])
def test_block_masses_closed_form_at_zero_query(n):
    # Q = 0: row r (position i_r = n - 128 + r) is uniform, 1/(i_r + 1), on
    # keys 0..i_r.  With t = n - 128 (N-1) positions in the last block, a
    # fully visible tile has entry (r, column c) at offset
    # 128 (N-1-kb) + (r + t - 128 - c): band N-1-kb for c <= r + t - 128,
    # N-2-kb for r + t - 128 < c <= r + t, N-3-kb above.  Counting columns:
    N = -(-n // B)
    t = n - B * (N - 1)
    A, _ = O.proxy_map(np.zeros((B, 16)), _rng(17).standard_normal((n, 16)), 1.0)
    lo, up, up2, rec = O.block_masses(A)
    r = np.arange(B)
    inv = 1.0 / (n - B + r + 1)
    n_lo = np.clip(r + t - B + 1, 0, B)
    n_up = np.clip(r + t + 1, 0, B) - n_lo
    n_up2 = B - n_lo - n_up
    full = range(N - 2) if t < B else range(N - 1)
    for kb in full:
        assert lo[kb] == pytest.approx(float((n_lo * inv).sum()), rel=1e-12)
        assert up[kb] == pytest.approx(float((n_up * inv).sum()), rel=1e-12)
        assert up2[kb] == pytest.approx(float((n_up2 * inv).sum()), rel=1e-12, abs=1e-300)
    # the last block: row r sees its first r + t - 127 keys, all in band 0
    vis = np.clip(r + t - B + 1, 0, t)
    assert lo[N - 1] == pytest.approx(float((vis * inv).sum()), rel=1e-12)
    assert up[N - 1] == 0.0 and up2[N - 1] == 0.0
    # recency window: keys n-128 .. i_r, r + 1 of them per row
    assert rec.sum() == pytest.approx(float(((r + 1) * inv).sum()), rel=1e-12)


def test_periodic_slash_closed_form():
    # One-hot Q_i = a e_{i mod 128}, K_j = a e_{(j + o*) mod 128}:
    # logit x only where (i - j) = o* (mod 128).  Closed forms for c[j], dg[o].
    n, d, a, ostar = 640, 128, 1.7, 37
    scale = 1 / math.sqrt(d)
    pos = np.arange(n)
    k = np.zeros((n, d))
    k[pos, (pos + ostar) % d] = a
    qlast = np.zeros((B, d))
    rows = np.arange(n - B, n)
    qlast[np.arange(B), rows % d] = a
    A, _ = O.proxy_map(qlast, k, scale)
    c, dg = O.token_scores(A)
    ex = math.exp(scale * a * a)
    Z = []
    for r in range(B):
        i = n - B + r
        cnt = (i - ostar) // 128 + 1 if i >= ostar else 0
        Z.append(cnt * ex + (i + 1 - cnt))
    c_cf = np.zeros(n)
    dg_cf = np.zeros(n)
    for r in range(B):
        i = n - B + r
        for j in range(i + 1):
            w = (ex if (i - j) % 128 == ostar else 1.0) / Z[r]
            c_cf[j] += w / B
            dg_cf[i - j] += w / B
    np.testing.assert_allclose(c, c_cf, rtol=1e-12, atol=1e-18)
    np.testing.assert_allclose(dg, dg_cf, rtol=1e-12, atol=1e-18)
    # the planted offset is the heaviest slash position; vertical mass is flat-ish
    assert int(np.argmax(dg)) == ostar


# --------------------------------------------------------------------------
# noise floor
# --------------------------------------------------------------------------


@pytest.mark.parametrize("m", [1, 2, 3, 7, 8, 31, 64, 4095])
def test_lower_median_by_counting(m):
    rng = _rng(100 + m)
    x = rng.integers(0, 5, size=m).astype(float)  # many ties
    med = O.lower_median(x)
    kidx = (m - 1) // 2
    assert np.sum(x < med) <= kidx
    assert np.sum(x <= med) >= kidx + 1


def test_lower_median_hand_examples():
    assert O.lower_median([3, 1, 2, 4]) == 2
    assert O.lower_median([5, 1, 3]) == 3
    assert O.lower_median([2, 2, 1, 1]) == 1


def _cliff(N, Ms, k, msig, rng):
    x = np.empty(N)
    mbg = (1.0 - Ms - k * msig) / (N - 1 - k)
    x[:] = mbg
    x[0] = Ms
    planted = np.sort(rng.choice(np.arange(1, N), k, replace=False))
    x[planted] = msig
    return x, planted, mbg


def test_mass_cliff_noise_floor_flat_and_gamma_linear():
    """The O(n) claim in closed form: the noise floor keeps {0} + planted at
    every N, gamma keeps 1 + k + ceil((gamma - Ms - k msig) / mbg)."""
    rng = _rng(7)
    Ms, k, gamma = 0.30, 8, 0.95
    nf_counts, g_counts = [], []
    for N in (32, 64, 128, 256, 512, 1024, 2048, 4096):
        msig = 0.02 if N >= 64 else 0.03
        x, planted, mbg = _cliff(N, Ms, k, msig, rng)
        assert msig > 1.25 * mbg
        mask, T = O.noise_floor_select(x, 1.25, 8)
        assert T == pytest.approx(1.25 * mbg, rel=1e-12)
        assert sorted(np.nonzero(mask)[0].tolist()) == [0] + planted.tolist()
        nf_counts.append(int(mask.sum()))
        need = (gamma - Ms - k * msig) / mbg
        assert abs(need - round(need)) > 1e-6
        closed = 1 + k + max(0, math.ceil(need))
        taken = O.gamma_prefix(x, gamma)
        assert len(taken) == closed
        g_counts.append(len(taken))
    assert len(set(nf_counts)) == 1
    assert all(b > a for a, b in zip(g_counts[2:], g_counts[3:]))
    # linear growth: doubling N roughly doubles the background blocks taken
    assert g_counts[-1] / g_counts[-2] == pytest.approx(2.0, rel=0.02)


def test_sink_only_collapse():
    # Sink mass above gamma: the gamma prefix stops inside the sink and the
    # k_min top-up fills with the next best blocks, while the noise floor
    # still finds the planted blocks.
    N = 256
    x = np.full(N, 0.0)
    x[0] = 0.96
    planted = [17, 90, 200]
    rest = 0.04 - 3 * 0.004
    x[1:] = rest / (N - 4)
    x[planted] = 0.004
    assert O.gamma_prefix(x, 0.95) == [0]
    gm = O.vs_gamma_select(x, 0.95, 8)
    assert gm.sum() == 8 and gm[0] and all(gm[p] for p in planted)
    nf, _ = O.noise_floor_select(x, 1.25, 1)
    assert sorted(np.nonzero(nf)[0].tolist()) == [0] + planted
    # k_min: top-up to 8 uses the lowest indices among equal background scores
    nf8, _ = O.noise_floor_select(x, 1.25, 8)
    assert sorted(np.nonzero(nf8)[0].tolist()) == [0, 1, 2, 3, 4, 17, 90, 200]


def test_noise_floor_mean_variant():
    x = np.array([0.5, 0.1, 0.1, 0.1, 0.2])
    mask, T = O.noise_floor_select(x, 1.0, 1, O.NF_MEAN)
    assert T == pytest.approx(0.125)
    assert mask.tolist() == [True, False, False, False, True]
    mask, T = O.noise_floor_select(x, 1.0, 1, O.NF_MEDIAN)
    assert T == pytest.approx(0.1)
    assert mask.tolist() == [True, False, False, False, True]


# --------------------------------------------------------------------------
# gamma-cumulative coverage
# --------------------------------------------------------------------------


@pytest.mark.parametrize("seed", range(12))
def test_gamma_prefix_is_minimum_cardinality(seed):
    rng = _rng(200 + seed)
    N = int(rng.integers(3, 13))
    x = rng.dirichlet(np.ones(N) * 0.7)
    gamma = float(rng.uniform(0.5, 0.99))
    taken = O.gamma_prefix(x, gamma)
    best = None
    for size in range(1, N + 1):
        if any(sum(x[list(c)]) >= gamma for c in itertools.combinations(range(N), size)):
            best = size
            break
    assert len(taken) == best
    assert sum(x[taken]) >= gamma


def test_gamma_prefix_tie_rule_hand_example():
    x = np.array([0.2, 0.3, 0.2, 0.3])
    assert O.gamma_prefix(x, 0.7) == [1, 3, 0]
    assert O.gamma_prefix(x, 1.0) == [1, 3, 0, 2]


# --------------------------------------------------------------------------
# expansion to key-block lists
# --------------------------------------------------------------------------


@pytest.mark.parametrize("seed", range(4))
def test_vs_lists_equal_token_level_cover(seed):
    rng = _rng(300 + seed)
    N = 7
    n = N * B
    vmask = rng.random(N) < 0.35
    smask = rng.random(N) < 0.35
    vmask[0] = smask[0] = True
    lists = O.vs_lists(vmask, smask)
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    cover = (j <= i) & (vmask[j // B] | smask[np.clip((i - j) // B, 0, N - 1)] & (i >= j))
    touched = [set() for _ in range(N)]
    ii, jj = np.nonzero(cover)
    for a, b in zip(ii // B, jj // B):
        touched[a].add(int(b))
    for qb in range(N):
        assert lists[qb] == sorted(touched[qb])
        assert lists[qb][0] == 0 and lists[qb][-1] == qb


# --------------------------------------------------------------------------
# pooled estimation
# --------------------------------------------------------------------------


def test_pe_uniform_closed_form():
    n, d = 40 * B, 8
    q = np.ones((n, d))
    k = np.ones((n, d))
    qbar, kbar = O.pe_pool(q), O.pe_pool(k)
    gamma = 0.95
    for qb in range(40):
        if abs(gamma * (qb + 1) - round(gamma * (qb + 1))) < 1e-9:
            continue
        K = math.ceil(gamma * (qb + 1))
        lst = O.pe_row_select(qbar, kbar, qb, 0.3, gamma)
        assert lst == sorted(set(range(K)) | {qb})


def test_pe_two_level_closed_form():
    # Block means are t*u on planted key blocks, 0 elsewhere; Qbar = s*u.
    rng = _rng(8)
    N, d = 50, 16
    n = N * B
    u = np.zeros(d)
    u[3] = 1.0
    k = np.zeros((n, d))
    planted = [0, 7, 21, 33]
    for kb in planted:
        k[kb * B:(kb + 1) * B] = 2.0 * u + rng.standard_normal((B, d)) * 0  # exact means
    q = np.tile(1.5 * u, (n, 1))
    qbar, kbar = O.pe_pool(q), O.pe_pool(k)
    np.testing.assert_allclose(kbar[7], 2.0 * u)
    scale = 0.5
    x = scale * 1.5 * 2.0
    qb = 45
    p = O.pe_row_probs(qbar, kbar, qb, scale)
    Z = 4 * math.exp(x) + (qb + 1 - 4)
    for kb in range(qb + 1):
        assert p[kb] == pytest.approx((math.exp(x) if kb in planted else 1.0) / Z, rel=1e-12)
    mass_planted = 4 * math.exp(x) / Z
    gamma = 0.95
    need = (gamma - mass_planted) * Z
    closed = 4 + math.ceil(need)
    lst = O.pe_row_select(qbar, kbar, qb, scale, gamma)
    others = [kb for kb in range(qb + 1) if kb not in planted][: math.ceil(need)]
    assert lst == sorted(set(planted) | set(others) | {qb})
    assert len(O.gamma_prefix(p, gamma)) == closed


@pytest.mark.parametrize("n", [4 * B, 3 * B + 29])
def test_pe_pool_means(n):
    rng = _rng(9)
    x = rng.standard_normal((n, 5))
    m = O.pe_pool(x)
    assert m.shape == (4, 5)
    for b in range(4):
        acc = np.zeros(5)
        cnt = 0
        for t in range(B):
            if b * B + t < n:
                acc += x[b * B + t]
                cnt += 1
        np.testing.assert_allclose(m[b], acc / cnt, rtol=1e-13)


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------


def _brute_dense(q, k, v, scale):
    n = q.shape[0]
    out = np.zeros_like(q[:, : v.shape[1]])
    lse = np.zeros(n)
    for i in range(n):
        logits = [scale * float(np.dot(q[i], k[j])) for j in range(i + 1)]
        m = max(logits)
        w = [math.exp(t - m) for t in logits]
        z = sum(w)
        out[i] = sum(wj * v[j] for wj, j in zip(w, range(i + 1))) / z
        lse[i] = m + math.log(z)
    return out, lse


@pytest.mark.parametrize("n", [3 * B, 2 * B + 57])
def test_all_blocks_equal_brute_force_dense(n):
    rng = _rng(10)
    d = 16
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    scale = 0.37
    res = O.attention_rows(q, k, v, O.dense_lists(3), scale, range(3))
    ref, ref_lse = _brute_dense(q, k, v, scale)
    for qb in range(3):
        Ob, lb = res[qb]
        assert Ob.shape[0] == min(B, n - qb * B)
        np.testing.assert_allclose(Ob, ref[qb * B:(qb + 1) * B], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(lb, ref_lse[qb * B:(qb + 1) * B], rtol=1e-12)


def test_zero_query_gives_cumulative_mean():
    rng = _rng(11)
    n, d = 2 * B, 8
    v = rng.standard_normal((n, d))
    res = O.attention_rows(np.zeros((n, d)), rng.standard_normal((n, d)), v,
                           O.dense_lists(2), 1.0, range(2))
    cm = np.cumsum(v, axis=0) / np.arange(1, n + 1)[:, None]
    for qb in range(2):
        np.testing.assert_allclose(res[qb][0], cm[qb * B:(qb + 1) * B], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(res[qb][1], np.log(np.arange(qb * B, (qb + 1) * B) + 1), rtol=1e-13)


def test_constant_values_and_order_invariance():
    rng = _rng(12)
    n, d = 5 * B, 16
    q, k = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    v = np.full((n, d), 2.5)
    lists = [[0, qb] if qb else [0] for qb in range(5)]
    lists[4] = [4, 0, 2]
    res = O.attention_rows(q, k, v, lists, 0.25, range(5))
    for qb in range(5):
        np.testing.assert_allclose(res[qb][0], 2.5, rtol=1e-13)
    v2 = rng.standard_normal((n, d))
    a = O.attention_rows(q, k, v2, {4: [0, 2, 4]}, 0.25, [4])[4][0]
    b = O.attention_rows(q, k, v2, {4: [4, 2, 0, 2]}, 0.25, [4])[4][0]
    np.testing.assert_array_equal(a, b)


def test_diagonal_only_is_local_window():
    rng = _rng(13)
    n, d = 3 * B, 16
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    scale = 0.3
    res = O.attention_rows(q, k, v, [[0], [1], [2]], scale, [1, 2])
    for qb in (1, 2):
        for a in (0, 5, 127):
            i = qb * B + a
            js = range(qb * B, i + 1)
            logit = np.array([scale * q[i] @ k[j] for j in js])
            w = np.exp(logit - logit.max())
            expect = (w[:, None] * v[list(js)]).sum(0) / w.sum()
            np.testing.assert_allclose(res[qb][0][a], expect, rtol=1e-11, atol=1e-13)
    # first query of the sequence attends only to itself
    r0 = O.attention_rows(q, k, v, [[0]], scale, [0])[0]
    np.testing.assert_allclose(r0[0][0], v[0], rtol=1e-14)
    assert r0[1][0] == pytest.approx(scale * q[0] @ k[0], rel=1e-13)


# --------------------------------------------------------------------------
# the O(n) claim on structured inputs through the whole selection
# --------------------------------------------------------------------------


def test_structured_inputs_gamma_grows_noise_floor_flat():
    """Planted sink and needle blocks seen through the proxy map: the noise
    floor keeps the same blocks at every n, gamma = 0.95 keeps more as n grows
    (the O(n) background accumulation)."""
    d = 64
    cfg = O.OracleConfig(route_override=O.OVERRIDE_FORCE_VS, tau=0.5, alpha=1.25, kmin_blocks=1)
    scale = 1 / math.sqrt(d)
    nf_v, g_v = [], []
    for n in (2048, 4096, 8192):
        rng = _rng(14)
        u = np.zeros(d)
        u[0] = 1.0
        k = rng.standard_normal((n, d)) * 0.5
        k[:, 0] = 0.0
        q = rng.standard_normal((n, d)) * 0.5
        q[:, 0] = 0.0
        q[:, 0] += 4.0
        k[:4, 0] = 6.0  # sink
        for j0 in (640, 1280):  # two needle bands, 16 keys each
            k[j0:j0 + 16, 0] = 4.0
        hr = O.select_head(q, k, cfg, scale)
        gm = O.vs_gamma_select(hr.v, 0.95, cfg.kmin_blocks)
        nf_v.append(sorted(np.nonzero(hr.vmask)[0].tolist()))
        g_v.append(int(gm.sum()))
    # sink block 0 and the two needle blocks 640/128 = 5, 1280/128 = 10
    assert all(s == [0, 5, 10] for s in nf_v)
    assert g_v[0] < g_v[1] < g_v[2]
    assert g_v[2] / g_v[0] > 3.0  # roughly proportional to n


# --------------------------------------------------------------------------
# JSD routing signal (the comparison C_struct replaces)
# --------------------------------------------------------------------------


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_js_divergence_matches_scipy_distance(seed):
    from scipy.spatial.distance import jensenshannon

    r = _rng(seed)
    for n in (2, 7, 300):
        p = r.random(n)
        q = r.random(n) ** 4
        q[r.random(n) < 0.2] = 0.0  # zero entries exercise 0 log 0
        q[0] = 0.5
        p /= p.sum()
        q /= q.sum()
        d = jensenshannon(p, q)  # natural log by default
        assert math.isclose(O.js_divergence(p, q), d * d, rel_tol=1e-12, abs_tol=1e-15)


def test_js_divergence_two_point_entropy_form():
    # JSD = H(midpoint) - (H(p) + H(q)) / 2 with the binary entropy H
    def h(a):
        return -sum(x * math.log(x) for x in (a, 1 - a) if x > 0)

    for a, b in [(0.1, 0.9), (0.5, 0.5), (0.0, 1.0), (0.3, 0.31), (1.0, 0.25)]:
        p = np.array([a, 1 - a])
        q = np.array([b, 1 - b])
        want = h((a + b) / 2) - (h(a) + h(b)) / 2
        assert math.isclose(O.js_divergence(p, q), want, rel_tol=1e-12, abs_tol=1e-15)


def test_js_divergence_limits():
    r = _rng(5)
    p = r.random(50)
    p /= p.sum()
    q = r.random(50)
    q /= q.sum()
    assert O.js_divergence(p, p) == 0.0
    assert O.js_divergence(p, q) == pytest.approx(O.js_divergence(q, p), rel=1e-14)
    # disjoint supports reach the bound ln 2
    a = np.array([0.2, 0.8, 0.0, 0.0])
    b = np.array([0.0, 0.0, 0.6, 0.4])
    assert O.js_divergence(a, b) == pytest.approx(math.log(2.0), rel=1e-15)
    assert 0.0 < O.js_divergence(p, q) < math.log(2.0)


def test_jsd_actual_is_row_mean_of_block_sums():
    r = _rng(7)
    n, Bq = 4 * B, B
    A = r.random((Bq, n))
    A /= A.sum(axis=1, keepdims=True)
    got = O.jsd_actual(A, B)
    assert got.sum() == pytest.approx(1.0, abs=1e-12)
    for kb in range(n // B):
        hand = 0.0
        for row in range(Bq):
            for j in range(kb * B, (kb + 1) * B):
                hand += A[row, j]
        assert got[kb] == pytest.approx(hand / Bq, rel=1e-12)


def test_jsd_estimate_brute_force():
    r = _rng(8)
    n, d = 3 * B, 16
    ql = r.standard_normal((B, d))
    k = r.standard_normal((n, d))
    scale = 0.3
    qbar = [sum(ql[i, c] for i in range(B)) / B for c in range(d)]
    logits = []
    for kb in range(n // B):
        kbar = [sum(k[j, c] for j in range(kb * B, (kb + 1) * B)) / B for c in range(d)]
        logits.append(scale * sum(qbar[c] * kbar[c] for c in range(d)))
    z = sum(math.exp(x) for x in logits)
    want = [math.exp(x) / z for x in logits]
    np.testing.assert_allclose(O.jsd_estimate(ql, k, scale, B), want, rtol=1e-12)


def test_pooled_estimate_exact_for_block_constant_keys():
    # With one query vector for every proxy row and keys constant within each
    # block, unmasked per-row attention summed per block equals the pooled
    # softmax: the divergence vanishes.  A wrong pooling axis, a dropped
    # scale or a per-row normalisation error breaks the equality.
    r = _rng(9)
    N, d = 5, 8
    kb_vecs = r.standard_normal((N, d))
    k = np.repeat(kb_vecs, B, axis=0)
    q1 = r.standard_normal(d)
    ql = np.tile(q1, (B, 1))
    scale = 0.7
    s = scale * (ql @ k.T)
    A = np.exp(s - s.max(axis=1, keepdims=True))
    A /= A.sum(axis=1, keepdims=True)
    p_est = O.jsd_estimate(ql, k, scale, B)
    a_bar = O.jsd_actual(A, B)
    np.testing.assert_allclose(p_est, a_bar, rtol=1e-12)
    assert O.js_divergence(a_bar, p_est) == pytest.approx(0.0, abs=1e-15)
    # scaling the query changes the estimate unless the scale goes with it
    assert not np.allclose(O.jsd_estimate(ql, k, 2 * scale, B), a_bar, rtol=1e-6)


def test_jsd_route_direction_and_tie():
    u = np.full(8, 1.0 / 8)
    one_hot = np.zeros(8)
    one_hot[0] = 1.0
    # a head whose mass sits on one block, against a flat estimate: VS
    d, rt = O.jsd_route(u, one_hot, 0.1)
    # midpoint: 9/16 on block 0, 1/16 elsewhere
    want = math.sqrt(0.5 * math.log(16 / 9) + 0.5 * (1 / 8) * math.log(2 / 9) + 0.5 * (7 / 8) * math.log(2.0))
    assert d == pytest.approx(want, rel=1e-12)
    assert rt == O.ROUTE_VS
    # the estimate matches the attention: PE
    d0, rt0 = O.jsd_route(u, u, 0.1)
    assert d0 == 0.0 and rt0 == O.ROUTE_PE
    # a distance equal to the threshold goes VS
    assert O.jsd_route(u, one_hot, d)[1] == O.ROUTE_VS


# --------------------------------------------------------------------------
# token-granular Vertical-Slash selection
# --------------------------------------------------------------------------


@pytest.mark.parametrize("seed", [0, 1])
def test_token_floor_with_one_retained_is_the_block_rule(seed):
    # one retained entry is exactly the block-level rule with block 0 kept
    r = _rng(seed)
    x = r.random(40) ** 3
    for alpha, kmin, stat in [(1.25, 8, O.NF_MEDIAN), (1.0, 3, O.NF_MEDIAN), (2.0, 12, O.NF_MEAN)]:
        got, T1 = O.token_noise_floor_select(x, alpha, kmin, retained=1, stat=stat)
        want, T2 = O.noise_floor_select(x, alpha, kmin, stat)
        np.testing.assert_array_equal(got, want)
        assert T1 == T2


def test_token_floor_planted_spikes():
    # background 1.0 everywhere, spikes of 5 at three columns, first 4 retained:
    # median 1, floor alpha = 1.25 -> exactly the spikes; k_min 10 adds the
    # lowest-index background columns (ties to the lower index)
    n = 64
    x = np.ones(n)
    spikes = [9, 30, 61]
    x[spikes] = 5.0
    x[:4] = 0.0  # retained entries do not enter the median
    m, T = O.token_noise_floor_select(x, 1.25, 7, retained=4)
    assert T == 1.25
    assert sorted(np.nonzero(m)[0].tolist()) == [0, 1, 2, 3] + spikes
    m2, _ = O.token_noise_floor_select(x, 1.25, 10, retained=4)
    assert sorted(np.nonzero(m2)[0].tolist()) == [0, 1, 2, 3, 4, 5, 6, 9, 30, 61]
    # the mean statistic: (3 * 5 + 57) / 60 = 1.2 -> floor 1.5
    _, Tm = O.token_noise_floor_select(x, 1.25, 7, retained=4, stat=O.NF_MEAN)
    assert Tm == pytest.approx(1.25 * 72 / 60, rel=1e-15)


def test_token_plan_columns_and_lists():
    n, blk = 8 * 16, 16  # N = 8 blocks of 16 tokens
    c = np.ones(n)
    c[[5, 40, 41, 100]] = 9.0    # 5 is a sink column (block 0): a tile, not gathered
    sl = np.ones(8)
    sl[[2, 6]] = 9.0             # slash bands 2 and 6 (band 0 always)
    p = O.token_vs_plan(c, sl, 1.25, 1, 1, blk)
    assert p.cols == [40, 41, 100]
    assert np.nonzero(p.smask)[0].tolist() == [0, 2, 6]
    # query block 7 reads block 0, bands 0, 2 -> 7, 6, 5, 4; band 6 -> 1, 0
    assert p.lists[7] == [0, 1, 4, 5, 6, 7]
    assert p.lists[0] == [0]
    assert p.lists[3] == [0, 1, 2, 3]
    # only block 0 and the bands make tiles: query block 5 lists 0, then
    # bands 0 and 2 -> 5, 4, 3, 2
    assert p.lists[5] == [0, 2, 3, 4, 5]


def _mixed_brute(q, k, v, lists, cols, scale, qb, block):
    outs = []
    for i in range(qb * block, (qb + 1) * block):
        keys = [j for j in range(i + 1) if (j // block) in set(lists[qb]) or j in set(cols)]
        s = [scale * float(np.dot(q[i], k[j])) for j in keys]
        mx = max(s)
        w = [math.exp(t - mx) for t in s]
        z = sum(w)
        outs.append(sum(wi * v[j] for wi, j in zip(w, keys)) / z)
    return np.array(outs)


def test_mixed_attention_brute_force_and_reductions():
    r = _rng(11)
    blk, N, d = 8, 6, 4
    n = blk * N
    q = r.standard_normal((n, d))
    k = r.standard_normal((n, d))
    v = r.standard_normal((n, d))
    lists = [[0], [0, 1], [1, 2], [0, 3], [2, 4], [0, 4, 5]]
    cols = [3, 9, 17, 18, 33, 46]  # some inside listed tiles, one in a later block
    res = O.attention_rows_mixed(q, k, v, lists, cols, 0.5, range(N), blk)
    for qb in range(N):
        np.testing.assert_allclose(res[qb][0], _mixed_brute(q, k, v, lists, cols, 0.5, qb, blk), rtol=1e-12,
                                   atol=1e-12)
    # no columns: the tile-only attention
    tiles = O.attention_rows(q, k, v, lists, 0.5, range(N), blk)
    none = O.attention_rows_mixed(q, k, v, lists, [], 0.5, range(N), blk)
    for qb in range(N):
        np.testing.assert_array_equal(none[qb][0], tiles[qb][0])
    # every column plus the diagonal tile: dense causal attention
    dense = O.attention_rows(q, k, v, O.dense_lists(N), 0.5, range(N), blk)
    allc = O.attention_rows_mixed(q, k, v, [[qb] for qb in range(N)], list(range(n)), 0.5, range(N), blk)
    for qb in range(N):
        np.testing.assert_allclose(allc[qb][0], dense[qb][0], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(allc[qb][1], dense[qb][1], rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# whole layer: the per-head loop and the GQA head -> KV group map
# --------------------------------------------------------------------------


def _gqa_layer(hq, hkv, n, d, beta):
    """KV group 0 carries a sink (keys 0..3 = 8u, every other key 0) and
    constant values 3; its query heads have every row = beta u.  KV group
    1 has zero keys and values whose coordinate 0 is 10 + position (the
    rest 10); its query heads are zero.  Further groups repeat group 1 with
    values shifted by 100 g."""
    u = np.zeros(d)
    u[1] = 1.0
    q = np.zeros((hq, n, d))
    k = np.zeros((hkv, n, d))
    v = np.zeros((hkv, n, d))
    qpg = hq // hkv
    k[0, :4] = 8.0 * u
    v[0] = 3.0
    for h in range(qpg):  # consecutive heads share a group (the configs' GQA reading)
        q[h] = beta * u
    for g in range(1, hkv):
        v[g] = 10.0 + 100.0 * (g - 1)
        v[g, :, 0] += np.arange(n)
    return q, k, v


@pytest.mark.parametrize("hq,hkv", [(8, 2), (14, 2), (12, 3)])
def test_run_layer_maps_heads_to_groups_and_blocks(hq, hkv):
    n, d, scale, beta = 4 * B, 16, 0.25, 4.0
    q, k, v = _gqa_layer(hq, hkv, n, d, beta)
    qpg = hq // hkv
    # gamma_pe = 1 and kmin >= N keep every block on either route, so every
    # output has a closed form whatever the route
    cfg = O.OracleConfig(tau=0.5, gamma_pe=1.0, kmin_blocks=8)
    qbs = [3, 1]
    heads = list(range(hq))[::-1]
    res = O.run_layer(q, k, v, cfg, scale=scale, heads=heads, attn_qbs=qbs)
    assert sorted(res) == list(range(hq))
    e8 = math.exp(scale * beta * 8.0)  # sink logit 8 for group-0 heads
    # group 0: 4 sink keys of weight e8, every other visible key weight 1;
    # C_struct = mean over rows of (4 e8 + 124 + (r + 1)) / (4 e8 + i_r - 3)
    c_sink = sum((4 * e8 + 124 + r + 1) / (4 * e8 + (n - B + r) - 3) for r in range(B)) / B
    # zero queries: uniform rows, C_struct = mean of (129 + r) / (n - 127 + r)
    c_flat = sum((129 + r) / (n - 127 + r) for r in range(B)) / B
    assert c_sink > 0.9 and c_flat < 0.5
    for h in range(hq):
        g = h // qpg
        hr = res[h]
        assert sorted(hr.attn) == sorted(qbs)
        if g == 0:
            assert hr.route == O.ROUTE_VS
            assert hr.c_struct == pytest.approx(c_sink, rel=1e-12)
        else:
            assert hr.route == O.ROUTE_PE
            assert hr.c_struct == pytest.approx(c_flat, rel=1e-12)
        assert hr.lists == O.dense_lists(4)
        for qb in qbs:
            out, lse = hr.attn[qb]
            rows = np.arange(qb * B, (qb + 1) * B)
            if g == 0:
                np.testing.assert_allclose(out, 3.0, rtol=1e-13)
                # the row's logits: 8 on the sink keys, 0 elsewhere
                want_lse = np.log(4 * e8 + (rows + 1 - 4))
            else:
                # zero queries: the running mean of the group's values
                want = np.full((B, d), 10.0 + 100.0 * (g - 1))
                want[:, 0] += rows / 2.0
                np.testing.assert_allclose(out, want, rtol=1e-13)
                want_lse = np.log(rows + 1.0)
            np.testing.assert_allclose(lse, want_lse, rtol=1e-13)
    # a subset of heads and no attention
    sub = O.run_layer(q, k, v, cfg, scale=scale, heads=[qpg - 1, qpg], attn_qbs=[])
    assert sorted(sub) == [qpg - 1, qpg]
    assert sub[qpg - 1].route == O.ROUTE_VS and sub[qpg].route == O.ROUTE_PE
    assert sub[qpg].attn == {}
