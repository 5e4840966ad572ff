"""GPU parity of the HIP path against the fp64 oracle (needs an MI355X).

Every call goes through the C ABI (libcrisp.so via the ctypes binding);
the oracle sees the same bf16 bits, generated on the GPU and copied back.
"""
import math

import numpy as np
import pytest
import torch

from dynamic_sparse_attention_proxy_amd import binding as B
from dynamic_sparse_attention_proxy_amd import synth
from oracle import crisp_oracle as O
from parity import (JSD_ABS, JSD_REL, REL_CSTRUCT, REL_JSD_EST, check_attention, check_gamma_set, check_lse,
                    check_noise_floor_mask, check_pe_lists,
                    check_route, gpu_lists, near, to64)

pytestmark = pytest.mark.gpu

BLK = 128


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    yield
    torch.cuda.synchronize()


def _cfg_oracle(cfg: B.crisp_cfg) -> O.OracleConfig:
    return O.OracleConfig(tau=cfg.tau, alpha=cfg.alpha, gamma_pe=cfg.gamma_pe, kmin_blocks=cfg.kmin_blocks,
                          sink_width=cfg.sink_width, recency_width=cfg.recency_width, nf_stat=cfg.nf_stat,
                          route_override=cfg.route_override)


_INPUTS = {}


def inputs(widx, seq_len=None):
    key = (widx, seq_len)
    if key not in _INPUTS:
        print(f"[gen] workload {widx} n={seq_len}", flush=True)
        _INPUTS[key] = synth.make_inputs(synth.workload(widx), device="cuda", seq_len=seq_len)
    return _INPUTS[key]


def run_chain(x, cfg, gamma=None, out_dtype=torch.float32, use_map=False):
    """The chain with the proxy map materialised beside the block masses;
    routing and selection read the masses unless use_map."""
    hq, hkv, n = x.q.shape[0], x.k.shape[0], x.q.shape[1]
    dims = B.make_dims(hq, hkv, n)
    bufs = B.CrispBuffers(dims, out_dtype=out_dtype, with_map=True)
    B.crisp_prefill(dims, cfg, x.q, x.k, x.v, bufs, gamma=gamma, use_map=use_map, dense_below=0)
    torch.cuda.synchronize()
    return dims, bufs


# ---------------------------------------------------------------------------
# attention kernels on given lists
# ---------------------------------------------------------------------------


def test_dense_attention_single_head_4k():
    x = inputs(0)
    dims = B.make_dims(1, 1, 4096)
    out = torch.empty((1, 4096, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((1, 4096), dtype=torch.float32, device="cuda")
    B.crisp_dense_attn(dims, x.q, x.k, x.v, out, lse)
    torch.cuda.synchronize()
    q, k, v = to64(x.q[0]), to64(x.k[0]), to64(x.v[0])
    ref = O.attention_rows(q, k, v, O.dense_lists(32), dims.scale, range(32))
    og, lg = out[0].cpu().numpy(), lse[0].cpu().numpy()
    for qb in range(32):
        check_attention(og[qb * BLK:(qb + 1) * BLK], ref[qb][0], f"qb {qb}")
        check_lse(lg[qb * BLK:(qb + 1) * BLK], ref[qb][1])
    # bf16 output is the fp32 result rounded once
    outb = torch.empty((1, 4096, 128), dtype=torch.bfloat16, device="cuda")
    B.crisp_dense_attn(dims, x.q, x.k, x.v, outb)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(outb.float().cpu().numpy(), out.to(torch.bfloat16).float().cpu().numpy())


def _random_lists(rng, N, kind):
    lists = []
    for qb in range(N):
        if kind == "diag":
            l = [qb]
        elif kind == "full":
            l = list(range(qb + 1))
        else:
            l = sorted(set(rng.choice(qb + 1, size=int(rng.integers(1, qb + 2)), replace=False).tolist()) | {qb})
        lists.append(l)
    return lists


def _pack_lists(all_lists, hq, N):
    count = np.zeros((hq, N), np.int32)
    idx = np.zeros(hq * N * (N + 1) // 2, np.int32)
    for h in range(hq):
        base = h * N * (N + 1) // 2
        for qb, l in enumerate(all_lists[h]):
            count[h, qb] = len(l)
            s = base + qb * (qb + 1) // 2
            idx[s:s + len(l)] = l
    return torch.from_numpy(count).cuda(), torch.from_numpy(idx).cuda()


@pytest.mark.parametrize("where", ["visible", "diagonal", "first"])
def test_attention_raises_running_max_mid_row(where):
    """Planted keys score about 23 (natural-log units) above everything the
    first step of a row sees, so the kernels' running max must be raised in
    the middle of a row: on a fully visible step ("visible", scores redone
    from K in global memory), on the masked diagonal steps ("diagonal", both
    halves of the block), or never after the first step ("first")."""
    n, N = 2048, 16
    w = synth.custom(2, 1, n, seed=77, needles=0)
    x = synth.make_inputs(w, device="cuda")
    g = torch.Generator().manual_seed(5)
    u = torch.randn(128, generator=g, dtype=torch.float64)
    u = (u / u.norm()).to("cuda")
    planted = {"visible": [5 * BLK + 17, 9 * BLK + 100], "diagonal": [12 * BLK + 3, 15 * BLK + 70],
               "first": [1]}[where]
    q = (x.q.double() + 5.0 * u).to(torch.bfloat16)
    k = x.k.double()
    for pos in planted:
        k[0, pos] += 60.0 * u
    k = k.to(torch.bfloat16)
    v = x.v
    print(f"[raise] where={where} planted={planted}", flush=True)
    dims = B.make_dims(2, 1, n)
    rng = np.random.default_rng(11)
    lists = [_random_lists(rng, N, "full"), _random_lists(rng, N, "random")]
    count, idx = _pack_lists(lists, 2, N)
    out = torch.empty((2, n, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((2, n), dtype=torch.float32, device="cuda")
    dense = torch.empty_like(out)
    dlse = torch.empty_like(lse)
    B.crisp_sparse_attn(dims, q, k, v, count, idx, out, lse)
    B.crisp_dense_attn(dims, q, k, v, dense, dlse)
    torch.cuda.synchronize()
    k64, v64 = to64(k[0]), to64(v[0])
    for h in range(2):
        q64 = to64(q[h])
        ref = O.attention_rows(q64, k64, v64, lists[h], dims.scale, range(N))
        dref = O.attention_rows(q64, k64, v64, O.dense_lists(N), dims.scale, range(N))
        og, lg = out[h].cpu().numpy(), lse[h].cpu().numpy()
        dg, dl = dense[h].cpu().numpy(), dlse[h].cpu().numpy()
        for qb in range(N):
            rows = slice(qb * BLK, (qb + 1) * BLK)
            check_attention(og[rows], ref[qb][0], f"{where} sparse h {h} qb {qb}")
            check_lse(lg[rows], ref[qb][1])
            check_attention(dg[rows], dref[qb][0], f"{where} dense h {h} qb {qb}")
            check_lse(dl[rows], dref[qb][1])
    # the planted keys dominate the rows that see them
    assert float(lse[0, planted[-1] + 1]) > 20.0


@pytest.mark.parametrize("hq,hkv,n,kind", [
    (1, 1, 256, "random"),     # smallest length (N = 2: heads of a block on adjacent ids)
    (3, 1, 640, "random"),     # N = 5, not a multiple of 8
    (4, 2, 1024, "diag"),      # local window only (N = 8: blocks dealt across XCDs)
    (7, 1, 384, "full"),       # 7:1 GQA, full lists = dense
    (8, 8, 1024, "random"),    # one KV head per query head
    (2, 1, 300, "random"),     # partial last block of 44 rows (N = 3)
    (4, 2, 1000, "full"),      # partial last block of 104 rows: full lists = dense
    (3, 1, 1601, "random"),    # partial last block of a single row (N = 13)
    (2, 2, 2110, "diag"),      # 62 rows: the last block's second 64-key step lies past n
])
def test_sparse_attention_matches_oracle_on_given_lists(hq, hkv, n, kind):
    rng = np.random.default_rng(hq * 1000 + n)
    w = synth.custom(hq, hkv, n, seed=hq + n, needles=2)
    x = synth.make_inputs(w, device="cuda")
    N = B.num_blocks(n)
    lists = [_random_lists(rng, N, kind) for _ in range(hq)]
    count, idx = _pack_lists(lists, hq, N)
    dims = B.make_dims(hq, hkv, n)
    out = torch.empty((hq, n, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((hq, n), dtype=torch.float32, device="cuda")
    print(f"[sparse] hq={hq} hkv={hkv} n={n} kind={kind}", flush=True)
    B.crisp_sparse_attn(dims, x.q, x.k, x.v, count, idx, out, lse)
    torch.cuda.synchronize()
    for h in range(hq):
        g = h * hkv // hq
        ref = O.attention_rows(to64(x.q[h]), to64(x.k[g]), to64(x.v[g]), lists[h], dims.scale, range(N))
        og, lg = out[h].cpu().numpy(), lse[h].cpu().numpy()
        for qb in range(N):
            check_attention(og[qb * BLK:(qb + 1) * BLK], ref[qb][0], f"h {h} qb {qb}")
            check_lse(lg[qb * BLK:(qb + 1) * BLK], ref[qb][1])
    if kind == "full":
        dense = torch.empty_like(out)
        B.crisp_dense_attn(dims, x.q, x.k, x.v, dense)
        torch.cuda.synchronize()
        assert torch.equal(dense, out)
    if n % BLK:
        # rows past n are not written: canary rows after the last head survive
        outc = torch.full((hq * n + BLK, 128), 7.0, dtype=torch.float32, device="cuda")
        lsec = torch.full((hq * n + BLK,), 7.0, dtype=torch.float32, device="cuda")
        B.crisp_sparse_attn(dims, x.q, x.k, x.v, count, idx, outc, lsec)
        torch.cuda.synchronize()
        assert torch.equal(outc[: hq * n].view(hq, n, 128), out)
        assert torch.equal(lsec[: hq * n].view(hq, n), lse)
        assert bool((outc[hq * n:] == 7.0).all()) and bool((lsec[hq * n:] == 7.0).all())


def test_attention_work_queue():
    """More (head, query block) items than the kernel's persistent
    workgroups, with list lengths spread from 1 to qb + 1 so that queues
    drain unevenly and workgroups take items from other XCDs' queues: every
    row is written exactly as by a call on a fresh workspace, whatever the
    workspace held before (the call clears its queue), on two calls in a
    row, and sampled blocks match the oracle."""
    hq, hkv, n = 8, 2, 16384
    rng = np.random.default_rng(7)
    x = synth.make_inputs(synth.custom(hq, hkv, n, seed=11, needles=2), device="cuda")
    N = B.num_blocks(n)
    lists = [_random_lists(rng, N, "random") for _ in range(hq)]
    count, idx = _pack_lists(lists, hq, N)
    dims = B.make_dims(hq, hkv, n)
    wsb = B.crisp_attn_workspace_bytes(dims)
    print(f"[work queue] hq={hq} n={n} items={hq * N} workspace={wsb}", flush=True)
    outs = []
    for fill in (0, 0x7F, 0xFF, 0x7F):
        ws = torch.full((wsb,), fill, dtype=torch.uint8, device="cuda")
        out = torch.full((hq, n, 128), float("nan"), dtype=torch.float32, device="cuda")
        lse = torch.full((hq, n), float("nan"), dtype=torch.float32, device="cuda")
        B.crisp_sparse_attn(dims, x.q, x.k, x.v, count, idx, out, lse, workspace=ws)
        B.crisp_sparse_attn(dims, x.q, x.k, x.v, count, idx, out, lse, workspace=ws)
        torch.cuda.synchronize()
        assert not bool(out.isnan().any()) and not bool(lse.isnan().any()), fill
        outs.append((out, lse))
    for out, lse in outs[1:]:
        assert torch.equal(out, outs[0][0]) and torch.equal(lse, outs[0][1])
    out, lse = outs[0]
    for h in (0, 5):
        g = h * hkv // hq
        qbs = [0, 1, N // 2, N - 2, N - 1]
        ref = O.attention_rows(to64(x.q[h]), to64(x.k[g]), to64(x.v[g]), lists[h], dims.scale, qbs)
        og, lg = out[h].cpu().numpy(), lse[h].cpu().numpy()
        for qb in qbs:
            check_attention(og[qb * BLK:(qb + 1) * BLK], ref[qb][0], f"h {h} qb {qb}")
            check_lse(lg[qb * BLK:(qb + 1) * BLK], ref[qb][1])
    dense = torch.full((hq, n, 128), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.full((wsb,), 0x55, dtype=torch.uint8, device="cuda")
    B.crisp_dense_attn(dims, x.q, x.k, x.v, dense, workspace=ws)
    torch.cuda.synchronize()
    assert not bool(dense.isnan().any())


def _long_short_lists(rng, N, kind):
    """"long": each causal block kept with probability 0.995 (the diagonal
    always), near-dense lists; "short": up to three
    random blocks below the diagonal, plus the diagonal."""
    out = []
    for qb in range(N):
        if kind == "long":
            m = rng.random(qb + 1) < 0.995
            m[qb] = True
            out.append(np.flatnonzero(m).tolist())
        else:
            below = rng.choice(qb, size=min(qb, int(rng.integers(0, 4))), replace=False).tolist() if qb else []
            out.append(sorted(below) + [qb])
    return out


def _schedule_sums(lists, N):
    """Sums the schedule pass forms over every (head, pair of blocks): the
    listed blocks cA + cB, and the bound min(cA + cB, 2p + 2) on the union."""
    own = bound = 0
    for hl in lists:
        for qa in range(0, N, 2):
            ca = len(hl[qa])
            if qa + 1 < N:
                cb = len(hl[qa + 1])
                own += ca + cb
                bound += min(ca + cb, qa + 2)
            else:
                own += ca
                bound += ca
    return own, bound


def _two_block(own, bound):
    """The launch rule: two blocks per workgroup when 2 bound <= 1.035 own."""
    return 2000 * bound <= 1035 * own


def _sums_left(ws):
    """The schedule sums the call left in its workspace (bytes 64..79)."""
    return tuple(int(t) for t in ws[64:80].view(torch.int64).cpu().tolist())


def _kernel_taken(ws):
    """Which attention kernel took the items, from the decision words the
    call left after the sums: "two", "one" or "runs"."""
    w = [int(t) for t in ws[80:128].view(torch.int64).cpu().tolist()]
    taken = [name for name, (a, b), runs_if_pays in (("two", w[0:2], True), ("one", w[2:4], False),
                                                      ("runs", w[4:6], False))
             if _two_block(a, b) == runs_if_pays]
    assert len(taken) == 1, w
    return taken[0]


@pytest.mark.parametrize("hq,hkv,n,kinds", [
    (4, 2, 16384, "LLLL"),     # N = 128
    (3, 1, 16512, "LLL"),      # N = 129: the last pair holds one block
    (2, 1, 16321, "LL"),       # partial last block of 65 rows, the second block of its pair
    (2, 2, 16257, "LL"),       # partial last block of one row
    (7, 1, 16384, "LLLSLLL"),  # 7:1 GQA; one head of short lists
])
def test_two_block_attention_matches_oracle(hq, hkv, n, kinds):
    """Near-dense lists go to the two-block kernel: the schedule sums the call
    leaves in its workspace equal the ones formed here from the lists, and
    they pick that kernel.  Rows of both blocks of sampled pairs (the first
    two, the middle one, the last) match the oracle on their own lists, for
    a short-list head too, whose blocks own few of the union's steps."""
    rng = np.random.default_rng(n + 7 * hq)
    x = synth.make_inputs(synth.custom(hq, hkv, n, seed=n + 1, needles=2), device="cuda")
    N = B.num_blocks(n)
    lists = [_long_short_lists(rng, N, "long" if c == "L" else "short") for c in kinds]
    count, idx = _pack_lists(lists, hq, N)
    dims = B.make_dims(hq, hkv, n)
    ws = torch.full((B.crisp_attn_workspace_bytes(dims),), 0x5A, dtype=torch.uint8, device="cuda")
    out = torch.full((hq, n, 128), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((hq, n), float("nan"), dtype=torch.float32, device="cuda")
    print(f"[two-block] hq={hq} hkv={hkv} n={n} kinds={kinds}", flush=True)
    B.crisp_sparse_attn(dims, x.q, x.k, x.v, count, idx, out, lse, workspace=ws)
    torch.cuda.synchronize()
    own, bound = _schedule_sums(lists, N)
    assert _sums_left(ws) == (own, bound)
    assert _two_block(own, bound) and _kernel_taken(ws) == "two"
    qbs = sorted({0, 1, 2, 3, N // 2, N // 2 + 1, N - 2, N - 1} | {(N - 1) & ~1})
    for h in range(hq):
        g = h * hkv // hq
        ref = O.attention_rows(to64(x.q[h]), to64(x.k[g]), to64(x.v[g]), lists[h], dims.scale, qbs)
        og, lg = out[h].cpu().numpy(), lse[h].cpu().numpy()
        for qb in qbs:
            check_attention(og[qb * BLK:(qb + 1) * BLK], ref[qb][0], f"two-block h {h} qb {qb}")
            check_lse(lg[qb * BLK:(qb + 1) * BLK], ref[qb][1])


@pytest.mark.parametrize("n,kernel", [(4096, "one"), (16384, "runs"), (16257, "runs"), (16512, "one")])
def test_one_block_kernel_takes_short_lists(n, kernel):
    """Short lists leave the two-block kernel unpaid: the sums pick the
    one-block kernel, dealt in runs of 16 query blocks per XCD when the block
    count is a multiple of 128 (16384, and 16257 with a last block of one
    row) and interleaved otherwise; every row matches the oracle."""
    hq, hkv = 4, 2
    rng = np.random.default_rng(3)
    x = synth.make_inputs(synth.custom(hq, hkv, n, seed=5, needles=2), device="cuda")
    N = B.num_blocks(n)
    lists = [_long_short_lists(rng, N, "short") for _ in range(hq)]
    count, idx = _pack_lists(lists, hq, N)
    dims = B.make_dims(hq, hkv, n)
    ws = torch.full((B.crisp_attn_workspace_bytes(dims),), 0xA5, dtype=torch.uint8, device="cuda")
    out = torch.full((hq, n, 128), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((hq, n), float("nan"), dtype=torch.float32, device="cuda")
    B.crisp_sparse_attn(dims, x.q, x.k, x.v, count, idx, out, lse, workspace=ws)
    torch.cuda.synchronize()
    own, bound = _schedule_sums(lists, N)
    assert _sums_left(ws) == (own, bound)
    assert not _two_block(own, bound) and _kernel_taken(ws) == kernel
    for h in range(hq):
        g = h * hkv // hq
        ref = O.attention_rows(to64(x.q[h]), to64(x.k[g]), to64(x.v[g]), lists[h], dims.scale, range(N))
        og, lg = out[h].cpu().numpy(), lse[h].cpu().numpy()
        for qb in range(N):
            check_attention(og[qb * BLK:(qb + 1) * BLK], ref[qb][0], f"one-block h {h} qb {qb}")
            check_lse(lg[qb * BLK:(qb + 1) * BLK], ref[qb][1])


def test_two_block_work_queue():
    """The two-block kernel's items, (head, pair of blocks), outnumber its
    workgroups: two calls in a row on workspaces of any contents write the
    same rows, and sampled pairs match the oracle."""
    hq, hkv, n = 8, 2, 16384
    rng = np.random.default_rng(17)
    x = synth.make_inputs(synth.custom(hq, hkv, n, seed=19, needles=2), device="cuda")
    N = B.num_blocks(n)
    lists = [_long_short_lists(rng, N, "long") for _ in range(hq)]
    count, idx = _pack_lists(lists, hq, N)
    dims = B.make_dims(hq, hkv, n)
    wsb = B.crisp_attn_workspace_bytes(dims)
    print(f"[two-block queue] hq={hq} n={n} pairs={hq * N // 2}", flush=True)
    outs = []
    for fill in (0, 0xFF, 0x7F):
        ws = torch.full((wsb,), fill, dtype=torch.uint8, device="cuda")
        out = torch.full((hq, n, 128), float("nan"), dtype=torch.float32, device="cuda")
        lse = torch.full((hq, n), float("nan"), dtype=torch.float32, device="cuda")
        B.crisp_sparse_attn(dims, x.q, x.k, x.v, count, idx, out, lse, workspace=ws)
        B.crisp_sparse_attn(dims, x.q, x.k, x.v, count, idx, out, lse, workspace=ws)
        torch.cuda.synchronize()
        assert _two_block(*_sums_left(ws)) and _kernel_taken(ws) == "two", fill
        assert not bool(out.isnan().any()) and not bool(lse.isnan().any()), fill
        outs.append((out, lse))
    for out, lse in outs[1:]:
        assert torch.equal(out, outs[0][0]) and torch.equal(lse, outs[0][1])
    out, lse = outs[0]
    for h in (1, 6):
        g = h * hkv // hq
        qbs = [0, 1, 2, 3, N // 2, N // 2 + 1, N - 2, N - 1]
        ref = O.attention_rows(to64(x.q[h]), to64(x.k[g]), to64(x.v[g]), lists[h], dims.scale, qbs)
        og, lg = out[h].cpu().numpy(), lse[h].cpu().numpy()
        for qb in qbs:
            check_attention(og[qb * BLK:(qb + 1) * BLK], ref[qb][0], f"h {h} qb {qb}")
            check_lse(lg[qb * BLK:(qb + 1) * BLK], ref[qb][1])


def test_two_block_malformed_lists():
    """The two-block kernel reads each list as the one-block kernel does
    (count clamped to [1, qb+1], last entry taken as qb, the others clamped
    to [0, qb-1]) and walks the distinct blocks so read once each, so a
    repeated entry counts once."""
    hq, hkv, n = 2, 1, 16384
    N = 128
    rng = np.random.default_rng(23)
    x = synth.make_inputs(synth.custom(hq, hkv, n, seed=29, needles=2), device="cuda")
    dims = B.make_dims(hq, hkv, n)
    lists = [_long_short_lists(rng, N, "long") for _ in range(hq)]
    # qb: (count, stored entries, blocks as read)
    bad = {5: (0, [], [5]),
           6: (2, [7, 1], [5, 6]),
           9: (4, [0, 2, 9, 3], [0, 2, 8, 9]),
           12: (99, list(range(13)), list(range(13))),
           13: (2, [-3, 6], [0, 13]),
           20: (3, [4, 4, 20], [4, 20])}
    count = np.zeros((hq, N), np.int32)
    idx = np.full(hq * N * (N + 1) // 2, 77, np.int32)
    read = []
    for h in range(hq):
        base = h * N * (N + 1) // 2
        rh = []
        for qb in range(N):
            c, stored, r = bad[qb] if qb in bad else (len(lists[h][qb]), lists[h][qb], lists[h][qb])
            count[h, qb] = c
            s = base + qb * (qb + 1) // 2
            idx[s:s + len(stored)] = stored
            rh.append(r)
        read.append(rh)
    ws = torch.zeros(B.crisp_attn_workspace_bytes(dims), dtype=torch.uint8, device="cuda")
    out = torch.empty((hq, n, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((hq, n), dtype=torch.float32, device="cuda")
    B.crisp_sparse_attn(dims, x.q, x.k, x.v, torch.from_numpy(count).cuda(), torch.from_numpy(idx).cuda(), out, lse,
                        workspace=ws)
    torch.cuda.synchronize()
    assert _two_block(*_sums_left(ws))
    qbs = sorted(set(q ^ b for q in bad for b in (0, 1)) | {0, 1, N - 2, N - 1})  # the bad blocks' pairs
    for h in range(hq):
        ref = O.attention_rows(to64(x.q[h]), to64(x.k[0]), to64(x.v[0]), read[h], dims.scale, qbs)
        og, lg = out[h].cpu().numpy(), lse[h].cpu().numpy()
        for qb in qbs:
            check_attention(og[qb * BLK:(qb + 1) * BLK], ref[qb][0], f"malformed two-block h {h} qb {qb}")
            check_lse(lg[qb * BLK:(qb + 1) * BLK], ref[qb][1])


# ---------------------------------------------------------------------------
# proxy, route, selection on the single-head 4k workload
# ---------------------------------------------------------------------------


def test_proxy_and_route_single_head_4k():
    x = inputs(0)
    cfg = B.make_cfg()
    dims, bufs = run_chain(x, cfg)
    q, k = to64(x.q[0]), to64(x.k[0])
    A_o, lse_o = O.proxy_map(q[-BLK:], k, dims.scale)
    A_g = bufs.attn_map[0].cpu().numpy().astype(np.float64)
    assert np.abs(A_g - A_o).max() <= 1e-6
    np.testing.assert_allclose(A_g.sum(axis=1), 1.0, atol=1e-4)
    for r in range(BLK):
        assert np.all(A_g[r, 4096 - BLK + r + 1:] == 0.0)
    np.testing.assert_allclose(bufs.row_lse[0].cpu().numpy(), lse_o, rtol=1e-5, atol=1e-5)
    planes_o = O.block_masses(A_o)
    bm = bufs.block_mass[:, 0].cpu().numpy().astype(np.float64)
    for c in range(4):
        np.testing.assert_allclose(bm[c], planes_o[c], rtol=1e-4, atol=1e-9, err_msg=f"plane {c}")
    assert bm[1, -1] == 0.0  # the masked half of the diagonal tile
    assert np.all(bm[2] == 0.0) and np.all(bm[3, :-1] == 0.0)
    c_o = O.c_struct(A_o)
    c_g = float(bufs.c_struct[0])
    assert abs(c_g - c_o) <= REL_CSTRUCT * c_o
    check_route(c_o, cfg.tau, int(bufs.route[0]), O.route(c_o, cfg.tau))


TAU_JSD = 0.1


@pytest.mark.parametrize("hq,hkv,n,family", [(1, 1, 4096, False), (8, 2, 4480, False), (14, 2, 2048, False),
                                             (32, 8, 8192, True), (4, 2, 3000, False)])
def test_jsd_routing_signal_matches_oracle(hq, hkv, n, family):
    """The comparison routing signal, and C_struct beside it, on the
    single-head 4k workload, a GQA layer whose 35 key blocks leave a partial
    workgroup, a 7:1 group (more heads per group than row groups per wave),
    and the graded-structure family, whose heads range from structureless to
    sink- or recency-dominated (C_struct from about 0.02 to 0.9)."""
    if family:
        x = synth.make_routing_family(seq_len=n, device="cuda")
    elif hq == 1:
        x = inputs(0)
    else:
        x = synth.make_inputs(synth.custom(hq, hkv, n, seed=hq * 31 + n, needles=4), device="cuda")
    dims = B.make_dims(hq, hkv, n)
    cfg = B.make_cfg(tau=0.2)
    N = B.num_blocks(n)
    mass = torch.empty((4, hq, N), dtype=torch.float32, device="cuda")
    partials = torch.empty(B.crisp_proxy_scratch_bytes(dims), dtype=torch.uint8, device="cuda")
    B.crisp_proxy(dims, x.q, x.k, None, partials=partials, block_mass=mass)
    cs = torch.empty(hq, dtype=torch.float32, device="cuda")
    rt = torch.empty(hq, dtype=torch.int32, device="cuda")
    B.crisp_route(dims, cfg, None, cs, rt, block_mass=mass)
    ws = torch.empty(B.crisp_route_jsd_workspace_bytes(dims), dtype=torch.uint8, device="cuda")
    dist = torch.empty(hq, dtype=torch.float32, device="cuda")
    route = torch.empty(hq, dtype=torch.int32, device="cuda")
    est = torch.empty((hq, N), dtype=torch.float32, device="cuda")
    B.crisp_route_jsd(dims, TAU_JSD, x.q, x.k, mass, dist, route, ws, estimate=est)
    torch.cuda.synchronize()
    est_g, dist_g, route_g = est.cpu().numpy(), dist.cpu().numpy(), route.cpu().numpy()
    cs_g, rt_g = cs.cpu().numpy(), rt.cpu().numpy()
    c_all = []
    for h in range(hq):
        g = h * hkv // hq
        q, k = to64(x.q[h]), to64(x.k[g])
        A, _ = O.proxy_map(q[n - BLK:], k, dims.scale)
        c_o = O.c_struct(A)
        c_all.append(c_o)
        assert abs(float(cs_g[h]) - c_o) <= REL_CSTRUCT * c_o, (h, cs_g[h], c_o)
        check_route(c_o, cfg.tau, int(rt_g[h]), O.route(c_o, cfg.tau))
        a_bar = O.jsd_actual(A)
        p_est = O.jsd_estimate(q[n - BLK:], k, dims.scale)
        np.testing.assert_allclose(est_g[h], p_est, rtol=REL_JSD_EST, atol=1e-9, err_msg=f"head {h}")
        d_o, r_o = O.jsd_route(p_est, a_bar, TAU_JSD)
        d_g = float(dist_g[h])
        assert abs(d_g * d_g - d_o * d_o) <= JSD_ABS + JSD_REL * d_o * d_o, f"head {h}: {d_g} vs {d_o}"
        check_route(d_o, TAU_JSD, int(route_g[h]), r_o)
        # the kernel's decision, taken on its own distance
        assert int(route_g[h]) == (B.ROUTE_VS if d_g >= TAU_JSD else B.ROUTE_PE)
    if family:
        # both routes occur, so the agreement measurement is not degenerate
        assert min(c_all) < 0.05 and max(c_all) > 0.8
        assert 0 < int(rt_g.sum()) < hq and 0 < int(route_g.sum()) < hq


@pytest.mark.parametrize("hq,hkv,n", [(1, 1, 4096), (8, 2, 4480), (4, 2, 256), (4, 2, 1000), (2, 1, 1090),
                                     (3, 1, 2100), (2, 2, 4097)])
def test_one_pass_block_masses(hq, hkv, n):
    """Block masses alone come from the stats pass (each row's part per key
    block against its running max, then weighed by 2^(max - lse2)); with the
    map they come from the second pass.  Both against the oracle's
    definition and against each other, on a layer whose last 1024-key chunk
    holds three key blocks, on the shortest layer, and on lengths with a
    partial last block: 104 positions in one chunk; a last chunk of 66 keys
    that starts past the first 62 proxy rows; 52 positions (its second
    64-key step lies past n); a single position."""
    x = inputs(0) if hq == 1 else synth.make_inputs(synth.custom(hq, hkv, n, seed=n + 7, needles=4), device="cuda")
    dims = B.make_dims(hq, hkv, n)
    N = B.num_blocks(n)
    part = torch.empty(B.crisp_proxy_scratch_bytes(dims), dtype=torch.uint8, device="cuda")
    m1 = torch.empty((4, hq, N), dtype=torch.float32, device="cuda")
    m2 = torch.empty_like(m1)
    amap = torch.empty((hq, BLK, n), dtype=torch.float32, device="cuda")
    lse1 = torch.empty((hq, BLK), dtype=torch.float32, device="cuda")
    lse2 = torch.empty_like(lse1)
    B.crisp_proxy(dims, x.q, x.k, None, lse1, part, block_mass=m1)
    B.crisp_proxy(dims, x.q, x.k, amap, lse2, part, block_mass=m2)
    torch.cuda.synchronize()
    # the diagonal sub-tiles are summed in another order when the parts are kept
    np.testing.assert_allclose(lse1.cpu().numpy(), lse2.cpu().numpy(), rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(m1.cpu().numpy(), m2.cpu().numpy(), rtol=1e-5, atol=1e-10)
    g1 = m1.cpu().numpy().astype(np.float64)
    g2 = m2.cpu().numpy().astype(np.float64)
    amap_g = amap.cpu().numpy().astype(np.float64)
    cfg = B.make_cfg()
    cs = torch.empty(hq, dtype=torch.float32, device="cuda")
    rt = torch.empty(hq, dtype=torch.int32, device="cuda")
    cs_map = torch.empty_like(cs)
    B.crisp_route(dims, cfg, None, cs, rt, block_mass=m1)
    B.crisp_route(dims, cfg, amap, cs_map, rt)
    torch.cuda.synchronize()
    for h in range(hq):
        A, _ = O.proxy_map(to64(x.q[h, n - BLK:]), to64(x.k[h * hkv // hq]), dims.scale)
        assert np.abs(amap_g[h] - A).max() <= 1e-6, f"head {h} map"
        planes = O.block_masses(A)
        for c, name in enumerate(("band N-1-kb", "band N-2-kb", "band N-3-kb", "recency")):
            np.testing.assert_allclose(g1[c, h], planes[c], rtol=1e-4, atol=1e-9, err_msg=f"head {h} {name}")
            np.testing.assert_allclose(g2[c, h], planes[c], rtol=1e-4, atol=1e-9, err_msg=f"head {h} {name} 2p")
        assert g1[1, h, -1] == 0.0 and g1[2, h, -1] == 0.0  # nothing of the last block lies past its band
        if n % BLK == 0:
            assert np.all(g1[2, h] == 0.0)
        c_o = O.c_struct(A)
        assert abs(float(cs[h]) - c_o) <= REL_CSTRUCT * c_o, (h, float(cs[h]), c_o)
        assert abs(float(cs_map[h]) - c_o) <= REL_CSTRUCT * c_o, (h, float(cs_map[h]), c_o)


@pytest.mark.parametrize("alpha,stat", [(1.25, B.NF_MEDIAN), (1.0, B.NF_MEDIAN), (1.25, B.NF_MEAN)])
def test_noise_floor_selection_single_head_4k(alpha, stat):
    x = inputs(0)
    cfg = B.make_cfg(route_override=B.ROUTE_FORCE_VS, alpha=alpha, nf_stat=stat)
    dims, bufs = run_chain(x, cfg)
    hr = O.select_head(to64(x.q[0]), to64(x.k[0]), _cfg_oracle(cfg), dims.scale)
    N = 32
    vg = bufs.blocks["v_score"][0].cpu().numpy()
    sg = bufs.blocks["s_score"][0].cpu().numpy()
    np.testing.assert_allclose(vg, hr.v, rtol=1e-4, atol=1e-9)
    np.testing.assert_allclose(sg, hr.sl, rtol=1e-4, atol=1e-9)
    vm = bufs.blocks["v_mask"][0].cpu().numpy()
    sm = bufs.blocks["s_mask"][0].cpu().numpy()
    check_noise_floor_mask(hr.v, alpha, 8, stat, vm, float(bufs.blocks["floor_v"][0]))
    check_noise_floor_mask(hr.sl, alpha, 8, stat, sm, float(bufs.blocks["floor_s"][0]))
    assert int(bufs.blocks["n_v"][0]) == int(vm.sum())
    assert int(bufs.blocks["n_s"][0]) == int(sm.sum())
    lists_g = gpu_lists(bufs.blocks["count"].cpu().numpy(), bufs.blocks["idx"].cpu().numpy(), 0, N)
    assert lists_g == O.vs_lists(vm.astype(bool), sm.astype(bool))
    ref = O.attention_rows(to64(x.q[0]), to64(x.k[0]), to64(x.v[0]), lists_g, dims.scale, range(N))
    og = bufs.out[0].cpu().numpy()
    for qb in range(N):
        check_attention(og[qb * BLK:(qb + 1) * BLK], ref[qb][0], f"qb {qb}")


def test_pe_selection_single_head_4k():
    x = inputs(0)
    cfg = B.make_cfg(route_override=B.ROUTE_FORCE_PE)
    dims, bufs = run_chain(x, cfg)
    q, k = to64(x.q[0]), to64(x.k[0])
    lists_g = gpu_lists(bufs.blocks["count"].cpu().numpy(), bufs.blocks["idx"].cpu().numpy(), 0, 32)
    check_pe_lists(O.pe_pool(q), O.pe_pool(k), dims.scale, cfg.gamma_pe, lists_g)
    assert bufs.blocks["v_mask"].sum().item() == 0
    ref = O.attention_rows(q, k, to64(x.v[0]), lists_g, dims.scale, range(32))
    og = bufs.out[0].cpu().numpy()
    for qb in range(32):
        check_attention(og[qb * BLK:(qb + 1) * BLK], ref[qb][0], f"qb {qb}")


@pytest.mark.parametrize("gamma", [0.95, 0.97])
def test_gamma_comparison_chain_single_head_4k(gamma):
    x = inputs(0)
    cfg = B.make_cfg(route_override=B.ROUTE_FORCE_VS)
    dims, bufs = run_chain(x, cfg, gamma=gamma)
    hr = O.select_head(to64(x.q[0]), to64(x.k[0]), _cfg_oracle(cfg), dims.scale, gamma=gamma)
    for key, xs in (("v_mask", hr.v), ("s_mask", hr.sl)):
        got = set(np.nonzero(bufs.blocks[key][0].cpu().numpy())[0].tolist())
        check_gamma_set(xs, range(32), gamma, got, {0}, extra_fill=8)


# ---------------------------------------------------------------------------
# Llama-3.1-8B-shaped 32k layer: every head through proxy/route/select,
# attention on sampled query blocks
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("override", [B.ROUTE_AUTO, B.ROUTE_FORCE_VS])
def test_llama_32k_layer(override):
    x = inputs(1)
    cfg = B.make_cfg(route_override=override)
    print(f"[chain] llama 32k override={override}", flush=True)
    dims, bufs = run_chain(x, cfg)
    hq, N = 32, 256
    ocfg = _cfg_oracle(cfg)
    count = bufs.blocks["count"].cpu().numpy()
    idx = bufs.blocks["idx"].cpu().numpy()
    cs = bufs.c_struct.cpu().numpy()
    rt = bufs.route.cpu().numpy()
    rng = np.random.default_rng(5)
    heads = sorted({0, 21, 22, 31} | set(rng.choice(hq, 2, replace=False).tolist()))
    for h in range(hq):
        g = h // 4
        q, k = to64(x.q[h]), to64(x.k[g])
        A, _ = O.proxy_map(q[-BLK:], k, dims.scale)
        c_o = O.c_struct(A)
        assert abs(cs[h] - c_o) <= REL_CSTRUCT * c_o, (h, cs[h], c_o)
        r_o = O.route(c_o, cfg.tau, override)
        check_route(c_o, cfg.tau, int(rt[h]), r_o)
        lists_g = gpu_lists(count, idx, h, N)
        if rt[h] == O.ROUTE_VS:
            ct, dg = O.token_scores(A)
            v, sl = O.pooled_scores(ct, dg)
            vm = bufs.blocks["v_mask"][h].cpu().numpy()
            sm = bufs.blocks["s_mask"][h].cpu().numpy()
            check_noise_floor_mask(v, cfg.alpha, 8, 0, vm, float(bufs.blocks["floor_v"][h]))
            check_noise_floor_mask(sl, cfg.alpha, 8, 0, sm, float(bufs.blocks["floor_s"][h]))
            assert lists_g == O.vs_lists(vm.astype(bool), sm.astype(bool))
        elif h in heads:
            check_pe_lists(O.pe_pool(q), O.pe_pool(k), dims.scale, cfg.gamma_pe, lists_g,
                           qbs=[0, 1, 2, 100, 254, 255])
        if h in heads:
            qbs = [0, 1, 128, 254, 255]
            ref = O.attention_rows(q, k, to64(x.v[g]), lists_g, dims.scale, qbs)
            og = bufs.out[h].cpu().numpy()
            for qb in qbs:
                check_attention(og[qb * BLK:(qb + 1) * BLK], ref[qb][0], f"h {h} qb {qb}")


# ---------------------------------------------------------------------------
# lengths that 128 does not divide: every step of the chain on a partial
# last block
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("n,mode,use_map", [
    (5000, "auto", False),      # graded family: both routes; 8 positions in the last block
    (5000, "auto", True),       # the same from the materialised map
    (3333, "vs", False),        # forced VS; 5 positions, a last 1024-key chunk of 261 keys
    (4160, "pe", False),        # forced PE; 64 positions
    (3001, "gamma", False),     # gamma 0.95 comparison chain; a single position
])
def test_ragged_length_chain(n, mode, use_map):
    """Route, selection and attention at lengths with a partial last block,
    head by head against the oracle: C_struct and the route, the VS floors,
    masks and lists, the PE lists (the last query block pooled over its own
    rows), and the attention of query blocks that include the partial one."""
    hq, hkv = 8, 2
    if mode == "auto":
        x = synth.make_routing_family(seq_len=n, num_q_heads=hq, num_kv_heads=hkv, device="cuda")
    else:
        x = synth.make_inputs(synth.custom(hq, hkv, n, seed=n, needles=4), device="cuda")
    override = {"auto": B.ROUTE_AUTO, "vs": B.ROUTE_FORCE_VS, "pe": B.ROUTE_FORCE_PE, "gamma": B.ROUTE_FORCE_VS}[mode]
    cfg = B.make_cfg(tau=0.2 if mode == "auto" else 0.5, route_override=override)
    gamma = 0.95 if mode == "gamma" else None
    print(f"[ragged] n={n} mode={mode} map={use_map}", flush=True)
    dims, bufs = run_chain(x, cfg, gamma=gamma, use_map=use_map)
    N = B.num_blocks(n)
    assert n % BLK and N == n // BLK + 1
    count = bufs.blocks["count"].cpu().numpy()
    idx = bufs.blocks["idx"].cpu().numpy()
    cs = bufs.c_struct.cpu().numpy()
    rt = bufs.route.cpu().numpy()
    out = bufs.out.cpu().numpy()
    lse = bufs.lse.cpu().numpy()
    qbs = [0, 1, N // 2, N - 2, N - 1]
    for h in range(hq):
        g = h * hkv // hq
        q, k, v = to64(x.q[h]), to64(x.k[g]), to64(x.v[g])
        A, _ = O.proxy_map(q[n - BLK:], k, dims.scale)
        c_o = O.c_struct(A)
        assert abs(cs[h] - c_o) <= REL_CSTRUCT * c_o, (h, cs[h], c_o)
        check_route(c_o, cfg.tau, int(rt[h]), O.route(c_o, cfg.tau, override))
        lists_g = gpu_lists(count, idx, h, N)
        assert all(l[-1] == qb for qb, l in enumerate(lists_g))
        if rt[h] == O.ROUTE_VS:
            ct, dg = O.token_scores(A)
            vs, sl = O.pooled_scores(ct, dg)
            np.testing.assert_allclose(bufs.blocks["v_score"][h].cpu().numpy(), vs, rtol=1e-4, atol=1e-9)
            np.testing.assert_allclose(bufs.blocks["s_score"][h].cpu().numpy(), sl, rtol=1e-4, atol=1e-9)
            vm = bufs.blocks["v_mask"][h].cpu().numpy()
            sm = bufs.blocks["s_mask"][h].cpu().numpy()
            if gamma is None:
                check_noise_floor_mask(vs, cfg.alpha, 8, 0, vm, float(bufs.blocks["floor_v"][h]))
                check_noise_floor_mask(sl, cfg.alpha, 8, 0, sm, float(bufs.blocks["floor_s"][h]))
            else:
                for xs, m in ((vs, vm), (sl, sm)):
                    check_gamma_set(xs, range(N), gamma, set(np.nonzero(m)[0].tolist()), {0}, extra_fill=8)
            assert lists_g == O.vs_lists(vm.astype(bool), sm.astype(bool))
        else:
            check_pe_lists(O.pe_pool(q), O.pe_pool(k), dims.scale, gamma or cfg.gamma_pe, lists_g, qbs=qbs)
        ref = O.attention_rows(q, k, v, lists_g, dims.scale, qbs)
        for qb in qbs:
            rows = slice(qb * BLK, min((qb + 1) * BLK, n))
            check_attention(out[h, rows], ref[qb][0], f"n {n} h {h} qb {qb}")
            check_lse(lse[h, rows], ref[qb][1])
    if mode == "auto":
        assert 0 < int(rt.sum()) < hq  # both routes occur


@pytest.mark.parametrize("override", [B.ROUTE_AUTO, B.ROUTE_FORCE_VS])
def test_map_and_block_mass_paths_agree(override):
    """Routing and selection from the block masses (the default chain) and
    from a pass over the materialised map: the same C_struct up to fp32
    summation order, and the same kept blocks except within the parity
    tolerance of a threshold."""
    x = inputs(1)
    cfg = B.make_cfg(route_override=override)
    _, bm = run_chain(x, cfg)
    _, bp = run_chain(x, cfg, use_map=True)
    c1, c2 = bm.c_struct.cpu().numpy(), bp.c_struct.cpu().numpy()
    np.testing.assert_allclose(c1, c2, rtol=1e-5)
    assert torch.equal(bm.route, bp.route)
    for key in ("v_score", "s_score"):
        np.testing.assert_allclose(bm.blocks[key].cpu().numpy(), bp.blocks[key].cpu().numpy(), rtol=1e-5,
                                   atol=1e-9)
    if override == B.ROUTE_FORCE_VS:
        for key, skey, fkey in (("v_mask", "v_score", "floor_v"), ("s_mask", "s_score", "floor_s")):
            m1, m2 = bm.blocks[key].cpu().numpy(), bp.blocks[key].cpu().numpy()
            xs = bp.blocks[skey].cpu().numpy()
            fl = bp.blocks[fkey].cpu().numpy()
            for h, b in zip(*np.nonzero(m1 != m2)):
                assert abs(xs[h, b] - fl[h]) <= 1e-3 * fl[h], (key, h, b)
    else:
        assert torch.equal(bm.blocks["count"], bp.blocks["count"])


def test_gated_short_layer_is_the_dense_kernel():
    """Below the context-length gate crisp_prefill runs the dense kernel."""
    n = B.DENSE_BELOW // 2
    w = synth.custom(4, 2, n, seed=21, needles=2)
    x = synth.make_inputs(w, device="cuda")
    dims = B.make_dims(4, 2, n)
    bufs = B.CrispBuffers(dims, out_dtype=torch.float32)
    B.crisp_prefill(dims, B.make_cfg(), x.q, x.k, x.v, bufs)
    dense = torch.empty_like(bufs.out)
    B.crisp_dense_attn(dims, x.q, x.k, x.v, dense)
    torch.cuda.synchronize()
    assert torch.equal(bufs.out, dense)


def test_chain_is_deterministic():
    x = inputs(1)
    cfg = B.make_cfg(route_override=B.ROUTE_FORCE_VS)
    _, b1 = run_chain(x, cfg)
    _, b2 = run_chain(x, cfg)
    assert torch.equal(b1.attn_map, b2.attn_map)
    assert torch.equal(b1.block_mass, b2.block_mass)
    for key in ("count", "v_score", "s_score", "v_mask", "s_mask", "floor_v", "floor_s"):
        assert torch.equal(b1.blocks[key], b2.blocks[key]), key
    c, i1, i2 = b1.blocks["count"].cpu().numpy(), b1.blocks["idx"].cpu().numpy(), b2.blocks["idx"].cpu().numpy()
    for h in (0, 13, 31):
        assert gpu_lists(c, i1, h, 256) == gpu_lists(c, i2, h, 256)
    assert torch.equal(b1.out, b2.out)
    assert torch.equal(b1.lse, b2.lse)


@pytest.mark.parametrize("n", [2048, 2000])
def test_full_coverage_is_the_dense_kernel(n):
    """gamma_PE = 1 keeps every block (no shorter prefix reaches the whole
    mass), so every pooled-estimation list is 0..qb and the sparse kernel's
    output and log-sum-exp equal the dense kernel's bit for bit; the same
    for the gamma comparison chain at gamma = 1 on Vertical-Slash heads."""
    hq, hkv = 4, 2
    x = synth.make_inputs(synth.custom(hq, hkv, n, seed=n + 3, needles=3), device="cuda")
    dims = B.make_dims(hq, hkv, n)
    N = B.num_blocks(n)
    dense = torch.empty((hq, n, 128), dtype=torch.float32, device="cuda")
    dlse = torch.empty((hq, n), dtype=torch.float32, device="cuda")
    B.crisp_dense_attn(dims, x.q, x.k, x.v, dense, dlse)
    for override, gamma in ((B.ROUTE_FORCE_PE, None), (B.ROUTE_FORCE_VS, 1.0)):
        cfg = B.make_cfg(gamma_pe=1.0, route_override=override)
        print(f"[full coverage] n={n} override={override} gamma={gamma}", flush=True)
        bufs = B.CrispBuffers(dims, out_dtype=torch.float32)
        B.crisp_prefill(dims, cfg, x.q, x.k, x.v, bufs, gamma=gamma, dense_below=0)
        torch.cuda.synchronize()
        count = bufs.blocks["count"].cpu().numpy()
        idx = bufs.blocks["idx"].cpu().numpy()
        for h in range(hq):
            assert gpu_lists(count, idx, h, N) == [list(range(qb + 1)) for qb in range(N)], (override, h)
        assert torch.equal(bufs.out, dense)
        assert torch.equal(bufs.lse, dlse)


@pytest.mark.parametrize("tau,expect", [(0.0, 1), (1.0, 0)])
def test_route_threshold_extremes(tau, expect):
    """C_struct lies in [0, 1] and is below 1 whenever any key outside the
    sink and recency columns is visible: tau = 0 routes every head to
    Vertical-Slash, tau = 1 every head to pooled estimation."""
    hq, hkv, n = 8, 2, 3000
    x = synth.make_routing_family(seq_len=n, num_q_heads=hq, num_kv_heads=hkv, device="cuda")
    cfg = B.make_cfg(tau=tau)
    dims, bufs = run_chain(x, cfg)
    cs = bufs.c_struct.cpu().numpy()
    assert np.all((cs >= 0.0) & (cs < 1.0))
    assert np.all(bufs.route.cpu().numpy() == expect)


def test_malformed_lists_never_weight_future_keys():
    """Lists that break the contract are read defensively: the count is
    clamped to [1, qb+1], the last entry taken as the diagonal block and
    every other entry clamped to [0, qb-1].  The output must equal the
    oracle's attention on the list so read, so no key past a query is ever
    weighted (a diagonal entry anywhere but last would otherwise be computed
    without the causal mask)."""
    hq, hkv, n = 2, 1, 1024
    N = 8
    x = synth.make_inputs(synth.custom(hq, hkv, n, seed=404, needles=2), device="cuda")
    dims = B.make_dims(hq, hkv, n)
    # (count, stored entries, list as read)
    rows = [(0, [], [0]),
            (2, [1, 0], [0, 1]),
            (2, [2, 2], [1, 2]),
            (2, [7, 1], [2, 3]),
            (4, [0, 2, 4, 3], [0, 2, 3, 4]),
            (9, [0, 1, 2, 3, 4, 5], [0, 1, 2, 3, 4, 5]),
            (2, [-3, 6], [0, 6]),
            (2, [3, 5], [3, 7])]
    count = np.zeros((hq, N), np.int32)
    idx = np.full(hq * N * (N + 1) // 2, 99, np.int32)
    for h in range(hq):
        base = h * N * (N + 1) // 2
        for qb, (c, stored, _) in enumerate(rows):
            count[h, qb] = c
            s = base + qb * (qb + 1) // 2
            idx[s:s + len(stored)] = stored
    out = torch.empty((hq, n, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((hq, n), dtype=torch.float32, device="cuda")
    B.crisp_sparse_attn(dims, x.q, x.k, x.v, torch.from_numpy(count).cuda(), torch.from_numpy(idx).cuda(), out, lse)
    torch.cuda.synchronize()
    read = [r[2] for r in rows]
    for h in range(hq):
        ref = O.attention_rows(to64(x.q[h]), to64(x.k[0]), to64(x.v[0]), read, dims.scale, range(N))
        og, lg = out[h].cpu().numpy(), lse[h].cpu().numpy()
        for qb in range(N):
            check_attention(og[qb * BLK:(qb + 1) * BLK], ref[qb][0], f"malformed h {h} qb {qb}")
            check_lse(lg[qb * BLK:(qb + 1) * BLK], ref[qb][1])


@pytest.mark.parametrize("gate", ["gated", "ungated"])
def test_one_call_layer_through_the_c_abi(gate):
    """crisp_prefill of the C ABI on a 4k layer: below its context-length
    gate it runs the dense kernel alone (selection outputs untouched, output
    equal to the oracle's dense causal attention); with the gate at the
    layer's length it runs the whole chain (routes, C_struct, selection and
    attention against the oracle's whole-layer driver)."""
    hq, hkv, n = 4, 2, 4096
    N = n // BLK
    x = synth.make_inputs(synth.custom(hq, hkv, n, seed=515, needles=3), device="cuda")
    dims = B.make_dims(hq, hkv, n)
    cfg = B.make_cfg()
    bufs = B.CrispBuffers(dims, out_dtype=torch.float32)
    bufs.blocks["count"].fill_(-7)
    bufs.route.fill_(-7)
    print(f"[prefill] {gate}", flush=True)
    B.crisp_prefill(dims, cfg, x.q, x.k, x.v, bufs, dense_below=None if gate == "gated" else n)
    torch.cuda.synchronize()
    q, k, v = to64(x.q), to64(x.k), to64(x.v)
    if gate == "gated":
        assert n < B.DENSE_BELOW
        assert bool((bufs.blocks["count"] == -7).all()) and bool((bufs.route == -7).all())
        for h in range(hq):
            g = h * hkv // hq
            ref = O.attention_rows(q[h], k[g], v[g], O.dense_lists(N), dims.scale, range(N))
            og, lg = bufs.out[h].cpu().numpy(), bufs.lse[h].cpu().numpy()
            for qb in range(N):
                check_attention(og[qb * BLK:(qb + 1) * BLK], ref[qb][0], f"gated h {h} qb {qb}")
                check_lse(lg[qb * BLK:(qb + 1) * BLK], ref[qb][1])
        return
    res = O.run_layer(q, k, v, _cfg_oracle(cfg), scale=dims.scale)
    count = bufs.blocks["count"].cpu().numpy()
    idx = bufs.blocks["idx"].cpu().numpy()
    for h in range(hq):
        hr = res[h]
        g = h * hkv // hq
        c_g = float(bufs.c_struct[h])
        assert abs(c_g - hr.c_struct) <= REL_CSTRUCT * hr.c_struct
        check_route(hr.c_struct, cfg.tau, int(bufs.route[h]), hr.route)
        lists = gpu_lists(count, idx, h, N)
        if int(bufs.route[h]) == O.ROUTE_PE:
            check_pe_lists(O.pe_pool(q[h]), O.pe_pool(k[g]), dims.scale, cfg.gamma_pe, lists)
        ref = O.attention_rows(q[h], k[g], v[g], lists, dims.scale, range(N))
        og, lg = bufs.out[h].cpu().numpy(), bufs.lse[h].cpu().numpy()
        for qb in range(N):
            check_attention(og[qb * BLK:(qb + 1) * BLK], ref[qb][0], f"chain h {h} qb {qb}")
            check_lse(lg[qb * BLK:(qb + 1) * BLK], ref[qb][1])
            if lists[qb] == hr.lists[qb]:
                check_attention(og[qb * BLK:(qb + 1) * BLK], hr.attn[qb][0], f"chain oracle h {h} qb {qb}")
