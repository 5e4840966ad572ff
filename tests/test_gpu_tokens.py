"""GPU parity of token-granular Vertical-Slash selection and of the mixed
tile-plus-column attention against the fp64 oracle (needs an MI355X).

Every call goes through the C ABI; the oracle sees the same bf16 bits."""
import numpy as np
import pytest
import torch

from dynamic_sparse_attention_proxy_amd import binding as B
from dynamic_sparse_attention_proxy_amd import synth
from oracle import crisp_oracle as O
from parity import (REL_CSTRUCT, check_attention, check_lse, check_noise_floor_mask, check_pe_lists, check_route,
                    check_token_cols, gpu_lists, to64)

pytestmark = pytest.mark.gpu

BLK = 128


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    yield
    torch.cuda.synchronize()


def _inputs(hq, hkv, n, seed):
    print(f"[gen] tokens {hq}x{hkv} n={n} seed={seed}", flush=True)
    if hq == 1:
        return synth.make_inputs(synth.workload(0), device="cuda")
    return synth.make_inputs(synth.custom(hq, hkv, n, seed=seed, needles=8), device="cuda")


def _token_chain(x, cfg):
    hq, hkv, n = x.q.shape[0], x.k.shape[0], x.q.shape[1]
    dims = B.make_dims(hq, hkv, n)
    bufs = B.CrispBuffers(dims, tokens=True)
    B.crisp_prefill_tokens(dims, cfg, x.q, x.k, x.v, bufs)
    torch.cuda.synchronize()
    return dims, bufs


def test_column_masses_match_oracle_and_block_masses_agree():
    for hq, hkv, n in [(1, 1, 4096), (8, 2, 4480), (2, 1, 3030), (2, 2, 1090)]:
        x = _inputs(hq, hkv, n, 41)
        dims = B.make_dims(hq, hkv, n)
        N = B.num_blocks(n)
        mass = torch.empty((4, hq, N), dtype=torch.float32, device="cuda")
        mass_ref = torch.empty_like(mass)
        cm = torch.empty((hq, n), dtype=torch.float32, device="cuda")
        part = torch.empty(B.crisp_proxy_scratch_bytes(dims), dtype=torch.uint8, device="cuda")
        B.crisp_proxy_cols(dims, x.q, x.k, mass, cm, None, part)
        B.crisp_proxy(dims, x.q, x.k, None, partials=part, block_mass=mass_ref)
        torch.cuda.synchronize()
        # the column variant forms the masses in the second pass, the masses-only
        # proxy in the first one (per-row parts against the running max)
        np.testing.assert_allclose(mass.cpu().numpy(), mass_ref.cpu().numpy(), rtol=1e-5, atol=1e-10)
        cg = cm.cpu().numpy().astype(np.float64)
        for h in range(hq):
            g = h * hkv // hq
            A, _ = O.proxy_map(to64(x.q[h, n - BLK:]), to64(x.k[g]), dims.scale)
            c, _ = O.token_scores(A)
            np.testing.assert_allclose(cg[h], c, rtol=1e-4, atol=1e-10, err_msg=f"head {h}")


@pytest.mark.parametrize("hq,hkv,n", [(8, 2, 4096), (8, 2, 3030)])
def test_route_from_column_masses_any_width(hq, hkv, n):
    """crisp_route_cols on the column masses of crisp_proxy_cols: C_struct
    of every head of the graded-structure family, for sink and recency
    widths from one column to n/2, within 1e-4 of the oracle's C_struct on
    the map, routes alike away from tau; at 128/128 it matches crisp_route
    on the block masses."""
    x = synth.make_routing_family(seq_len=n, num_q_heads=hq, num_kv_heads=hkv, device="cuda")
    dims = B.make_dims(hq, hkv, n)
    N = B.num_blocks(n)
    mass = torch.empty((4, hq, N), dtype=torch.float32, device="cuda")
    cm = torch.empty((hq, n), dtype=torch.float32, device="cuda")
    part = torch.empty(B.crisp_proxy_scratch_bytes(dims), dtype=torch.uint8, device="cuda")
    B.crisp_proxy_cols(dims, x.q, x.k, mass, cm, None, part)
    maps = []
    for h in range(hq):
        A, _ = O.proxy_map(to64(x.q[h, n - BLK:]), to64(x.k[h * hkv // hq]), dims.scale)
        maps.append(A)
    for ws, wr in ((1, 1), (64, 200), (128, 128), (300, 1000), (n // 2, n // 2), (5, n // 2)):
        cfg = B.make_cfg(tau=0.3)
        cfg.sink_width, cfg.recency_width = ws, wr
        c = torch.empty(hq, dtype=torch.float32, device="cuda")
        r = torch.empty(hq, dtype=torch.int32, device="cuda")
        print(f"[route cols] n={n} widths {ws}/{wr}", flush=True)
        B.crisp_route_cols(dims, cfg, cm, c, r)
        torch.cuda.synchronize()
        cg, rg = c.cpu().numpy(), r.cpu().numpy()
        for h in range(hq):
            c_o = O.c_struct(maps[h], ws, wr)
            assert abs(cg[h] - c_o) <= REL_CSTRUCT * c_o + 1e-7, (ws, wr, h, cg[h], c_o)
            check_route(c_o, cfg.tau, int(rg[h]), O.route(c_o, cfg.tau))
        if (ws, wr) == (128, 128):
            cb = torch.empty_like(c)
            rb = torch.empty_like(r)
            B.crisp_route(dims, cfg, None, cb, rb, block_mass=mass)
            torch.cuda.synchronize()
            np.testing.assert_allclose(cb.cpu().numpy(), cg, rtol=1e-5)


@pytest.mark.parametrize("alpha,stat,kmin", [(1.25, B.NF_MEDIAN, 8), (1.0, B.NF_MEDIAN, 8), (1.25, B.NF_MEAN, 8),
                                             (3.0, B.NF_MEDIAN, 20)])
def test_token_selection_matches_oracle(alpha, stat, kmin):
    """Forced VS on a GQA layer with needles: the kept columns, the column
    floor and the slash bands, and the tile lists from them.  alpha = 3 with
    k_min = 20 blocks makes the top-up decide most columns."""
    hq, hkv, n = 4, 2, 8192
    x = _inputs(hq, hkv, n, 43)
    cfg = B.make_cfg(alpha=alpha, nf_stat=stat, kmin_blocks=kmin, route_override=B.ROUTE_FORCE_VS)
    dims, bufs = _token_chain(x, cfg)
    N = B.num_blocks(n)
    cols = bufs.cols.cpu().numpy()
    ncols = bufs.ncols.cpu().numpy()
    below = bufs.col_below.cpu().numpy()
    count = bufs.blocks["count"].cpu().numpy()
    idx = bufs.blocks["idx"].cpu().numpy()
    smask = bufs.blocks["s_mask"].cpu().numpy()
    vmask = bufs.blocks["v_mask"].cpu().numpy()
    floor_v = bufs.blocks["floor_v"].cpu().numpy()
    floor_s = bufs.blocks["floor_s"].cpu().numpy()
    n_v = bufs.blocks["n_v"].cpu().numpy()
    for h in range(hq):
        g = h * hkv // hq
        A, _ = O.proxy_map(to64(x.q[h, n - BLK:]), to64(x.k[g]), dims.scale)
        c, dg = O.token_scores(A)
        _, sl = O.pooled_scores(c, dg)
        kept = cols[h, :ncols[h]]
        check_token_cols(c, alpha, kmin * BLK, stat, kept, float(floor_v[h]))
        assert n_v[h] == BLK + ncols[h]
        check_noise_floor_mask(sl, alpha, kmin, stat, smask[h], float(floor_s[h]))
        assert vmask[h].tolist() == [1] + [0] * (N - 1)
        # per query block: kept columns below it, and the tile lists
        for qb in range(N):
            assert below[h, qb] == int(np.sum(kept < qb * BLK)), (h, qb)
        lists = gpu_lists(count, idx, h, N)
        vb = np.zeros(N, dtype=bool)
        vb[0] = True
        assert lists == O.vs_lists(vb, smask[h].astype(bool)), f"head {h} tile lists"


def test_token_chain_attention_matches_oracle():
    hq, hkv, n = 4, 2, 8192
    x = _inputs(hq, hkv, n, 47)
    cfg = B.make_cfg(route_override=B.ROUTE_FORCE_VS)
    dims, bufs = _token_chain(x, cfg)
    N = B.num_blocks(n)
    cols = bufs.cols.cpu().numpy()
    ncols = bufs.ncols.cpu().numpy()
    count = bufs.blocks["count"].cpu().numpy()
    idx = bufs.blocks["idx"].cpu().numpy()
    out = bufs.out.cpu().numpy()
    lse = bufs.lse.cpu().numpy()
    qbs = [0, 1, 2, 17, 40, N - 2, N - 1]
    for h in (0, hq - 1):
        g = h * hkv // hq
        q, k, v = to64(x.q[h]), to64(x.k[g]), to64(x.v[g])
        lists = gpu_lists(count, idx, h, N)
        ref = O.attention_rows_mixed(q, k, v, lists, cols[h, :ncols[h]].tolist(), dims.scale, qbs)
        for qb in qbs:
            rows = slice(qb * BLK, (qb + 1) * BLK)
            check_attention(out[h, rows], ref[qb][0], f"head {h} qb {qb}")
            check_lse(lse[h, rows], ref[qb][1])


@pytest.mark.parametrize("ncol,n,hq,hkv", [(1, 2048, 4, 2), (64, 2048, 4, 2), (200, 2176, 4, 2), (3000, 8192, 4, 2),
                                           (2500, 16384, 16, 4)])
def test_column_kernel_on_given_lists_and_columns(ncol, n, hq, hkv):
    """crisp_sparse_attn_cols on random tile lists and random columns: some
    inside listed tiles, counts that leave partial 64-column steps, an odd
    number of query blocks (a pair with one block), more columns than one
    staged index chunk (2048), and more (head, pair) items than CUs, so that
    each persistent workgroup takes several and queues drain unevenly; a
    workspace left full of garbage gives the same result."""
    N = B.num_blocks(n)
    x = _inputs(hq, hkv, n, 53 + ncol)
    dims = B.make_dims(hq, hkv, n)
    rng = np.random.default_rng(ncol)
    lists_all, cols_all = [], []
    for h in range(hq):
        lists = [sorted(set(rng.choice(qb + 1, size=int(rng.integers(1, qb + 2)), replace=False).tolist()) | {qb})
                 for qb in range(N)]
        lists_all.append(lists)
        cols_all.append(np.sort(rng.choice(np.arange(BLK, n), size=ncol, replace=False)).astype(np.int32))
    count = np.zeros((hq, N), np.int32)
    idx = np.zeros(hq * N * (N + 1) // 2, np.int32)
    cols = np.zeros((hq, n), np.int32)
    below = np.zeros((hq, N), np.int32)
    for h in range(hq):
        base = h * N * (N + 1) // 2
        for qb, l in enumerate(lists_all[h]):
            count[h, qb] = len(l)
            s = base + qb * (qb + 1) // 2
            idx[s:s + len(l)] = l
            below[h, qb] = int(np.sum(cols_all[h] < qb * BLK))
        cols[h, :ncol] = cols_all[h]
    cd, idd, cold, bd = (torch.from_numpy(a).cuda() for a in (count, idx, cols, below))
    out = torch.empty((hq, n, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((hq, n), dtype=torch.float32, device="cuda")
    print(f"[cols] hq={hq} n={n} ncol={ncol} items={hq * ((N + 1) // 2)}", flush=True)
    B.crisp_sparse_attn(dims, x.q, x.k, x.v, cd, idd, out, lse)
    out2, lse2 = out.clone(), lse.clone()
    B.crisp_sparse_attn_cols(dims, x.q, x.k, x.v, cd, idd, cold, bd, out, lse)
    junk = torch.full((B.crisp_attn_workspace_bytes(dims),), 0xFF, dtype=torch.uint8, device="cuda")
    B.crisp_sparse_attn_cols(dims, x.q, x.k, x.v, cd, idd, cold, bd, out2, lse2, workspace=junk)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    og, lg = out.cpu().numpy(), lse.cpu().numpy()
    for h in range(hq):
        g = h * hkv // hq
        q, k, v = to64(x.q[h]), to64(x.k[g]), to64(x.v[g])
        qbs = range(N) if N <= 20 else [0, 1, 2, 3, 30, 31, N - 2, N - 1]
        ref = O.attention_rows_mixed(q, k, v, lists_all[h], cols_all[h].tolist(), dims.scale, qbs)
        for qb in qbs:
            rows = slice(qb * BLK, (qb + 1) * BLK)
            check_attention(og[h, rows], ref[qb][0], f"head {h} qb {qb}")
            check_lse(lg[h, rows], ref[qb][1])


def test_token_chain_is_deterministic():
    hq, hkv, n = 4, 2, 8192
    x = _inputs(hq, hkv, n, 59)
    cfg = B.make_cfg(route_override=B.ROUTE_FORCE_VS)
    _, b1 = _token_chain(x, cfg)
    _, b2 = _token_chain(x, cfg)
    for name in ("col_mass", "ncols", "col_below", "out", "lse"):
        assert torch.equal(getattr(b1, name), getattr(b2, name)), name
    for h in range(hq):
        k = int(b1.ncols[h])
        assert torch.equal(b1.cols[h, :k], b2.cols[h, :k])


@pytest.mark.parametrize("hq,hkv,n", [(2, 1, 256), (2, 1, 384), (4, 2, 1152), (2, 1, 700), (4, 2, 3100),
                                     (2, 2, 2049)])
def test_token_chain_small_layers(hq, hkv, n):
    """The shortest layers (two and three key blocks, an odd block count):
    fewer candidate columns than k_min, so the top-up decides, and query
    block pairs with a missing second block; then lengths with a partial
    last block (60, 28 and 1 positions)."""
    x = _inputs(hq, hkv, n, 61 + n)
    cfg = B.make_cfg(route_override=B.ROUTE_FORCE_VS)
    dims, bufs = _token_chain(x, cfg)
    N = B.num_blocks(n)
    cols = bufs.cols.cpu().numpy()
    ncols = bufs.ncols.cpu().numpy()
    count = bufs.blocks["count"].cpu().numpy()
    idx = bufs.blocks["idx"].cpu().numpy()
    smask = bufs.blocks["s_mask"].cpu().numpy()
    out = bufs.out.cpu().numpy()
    for h in range(hq):
        g = h * hkv // hq
        q, k, v = to64(x.q[h]), to64(x.k[g]), to64(x.v[g])
        A, _ = O.proxy_map(q[n - BLK:], k, dims.scale)
        c, dg = O.token_scores(A)
        _, sl = O.pooled_scores(c, dg)
        kept = cols[h, :ncols[h]]
        # min(1024, n) columns in all: every candidate is kept when n <= 1024
        check_token_cols(c, cfg.alpha, 8 * BLK, 0, kept, float(bufs.blocks["floor_v"][h]))
        if n <= 8 * BLK:
            assert ncols[h] == n - BLK
        lists = gpu_lists(count, idx, h, N)
        vb = np.zeros(N, dtype=bool)
        vb[0] = True
        assert lists == O.vs_lists(vb, smask[h].astype(bool))
        ref = O.attention_rows_mixed(q, k, v, lists, kept.tolist(), dims.scale, range(N))
        for qb in range(N):
            check_attention(out[h, qb * BLK:min((qb + 1) * BLK, n)], ref[qb][0], f"n {n} head {h} qb {qb}")


def test_token_chain_with_mixed_routes():
    """Route auto on the graded-structure family (tau 0.2): some heads go
    Vertical-Slash and get kept columns, the others Pooled-Estimation with
    no columns; lists, columns and the attention of sampled query blocks
    against the oracle, head by head."""
    n = 8192
    x = synth.make_routing_family(seq_len=n, device="cuda")
    hq, hkv = x.q.shape[0], x.k.shape[0]
    cfg = B.make_cfg(tau=0.2)
    dims, bufs = _token_chain(x, cfg)
    N = B.num_blocks(n)
    route = bufs.route.cpu().numpy()
    assert 0 < int(route.sum()) < hq, "the family must mix both routes"
    cols = bufs.cols.cpu().numpy()
    ncols = bufs.ncols.cpu().numpy()
    below = bufs.col_below.cpu().numpy()
    count = bufs.blocks["count"].cpu().numpy()
    idx = bufs.blocks["idx"].cpu().numpy()
    out = bufs.out.cpu().numpy()
    qbs = [0, 1, 31, N - 1]
    for h in range(hq):
        g = h * hkv // hq
        q, k, v = to64(x.q[h]), to64(x.k[g]), to64(x.v[g])
        lists = gpu_lists(count, idx, h, N)
        if route[h] == B.ROUTE_PE:
            assert ncols[h] == 0 and not below[h].any()
            check_pe_lists(O.pe_pool(q), O.pe_pool(k), dims.scale, cfg.gamma_pe, lists, qbs)
            kept = []
        else:
            A, _ = O.proxy_map(q[n - BLK:], k, dims.scale)
            c, _ = O.token_scores(A)
            kept = cols[h, :ncols[h]].tolist()
            check_token_cols(c, cfg.alpha, 8 * BLK, 0, kept, float(bufs.blocks["floor_v"][h]))
        ref = O.attention_rows_mixed(q, k, v, lists, kept, dims.scale, qbs)
        for qb in qbs:
            check_attention(out[h, qb * BLK:(qb + 1) * BLK], ref[qb][0], f"head {h} qb {qb}")
