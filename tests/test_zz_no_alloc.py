"""crisp_select_noalloc (selection with the library's static per-device
scratch, for callers that cannot allocate) against crisp_select with a
caller workspace: identical counts, lists and diagnostics, on consecutive
calls whose second is the smaller layer, so the scratch holds the previous
call's contents."""
import numpy as np
import pytest
import torch

from dynamic_sparse_attention_proxy_amd import binding as B
from dynamic_sparse_attention_proxy_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    yield
    torch.cuda.synchronize()


def _blocks(dims, dev):
    hq, N = dims.num_q_heads, B.num_blocks(dims.seq_len)
    f32, i32 = torch.float32, torch.int32
    out = {"count": torch.full((hq, N), -5, dtype=i32, device=dev),
           "idx": torch.full((B.crisp_list_capacity(dims),), -5, dtype=i32, device=dev)}
    for name in ("v_score", "s_score", "v_mask", "s_mask"):
        out[name] = torch.full((hq, N), -5, dtype=f32 if "score" in name else i32, device=dev)
    for name in ("floor_v", "floor_s", "n_v", "n_s"):
        out[name] = torch.full((hq,), -5, dtype=f32 if "floor" in name else i32, device=dev)
    return out


def _lists(out, hq, N):
    count = out["count"].cpu().numpy()
    idx = out["idx"].cpu().numpy()
    T = N * (N + 1) // 2
    return [[idx[h * T + qb * (qb + 1) // 2: h * T + qb * (qb + 1) // 2 + count[h, qb]].tolist() for qb in range(N)]
            for h in range(hq)]


def _compare(w, routes, cfg, gamma_note):
    x = synth.make_inputs(w, device="cuda")
    hq, hkv, n = w.num_q_heads, w.num_kv_heads, w.seq_len
    N = B.num_blocks(n)
    dims = B.make_dims(hq, hkv, n)
    assert B.crisp_select_workspace_bytes(dims) <= B.NOALLOC_SCRATCH_BYTES
    mass = torch.empty((4, hq, N), dtype=torch.float32, device="cuda")
    partials = torch.empty(B.crisp_proxy_scratch_bytes(dims), dtype=torch.uint8, device="cuda")
    B.crisp_proxy(dims, x.q, x.k, None, partials=partials, block_mass=mass)
    route = torch.tensor(routes, dtype=torch.int32, device="cuda")
    ws = torch.empty(B.crisp_select_workspace_bytes(dims), dtype=torch.uint8, device="cuda")
    ref = _blocks(dims, "cuda")
    got = _blocks(dims, "cuda")
    print(f"[noalloc] {w.name} n={n} routes={routes} {gamma_note}", flush=True)
    B.crisp_select(dims, cfg, x.q, x.k, None, route, ref, ws, block_mass=mass)
    B.crisp_select_noalloc(dims, cfg, x.q, x.k, None, route, got, block_mass=mass)
    torch.cuda.synchronize()
    assert torch.equal(ref["count"], got["count"])
    assert _lists(ref, hq, N) == _lists(got, hq, N)
    for name in ("v_score", "s_score", "v_mask", "s_mask", "floor_v", "floor_s", "n_v", "n_s"):
        assert torch.equal(ref[name], got[name]), name
    # both routes took part
    assert 0 < sum(routes) < hq
    return int(ref["count"].sum())


def test_noalloc_select_matches_workspace_select_on_consecutive_calls():
    cfg = B.make_cfg()
    big = synth.workload("qwen2.5-7b-128k")
    t1 = _compare(big, [h % 2 for h in range(big.num_q_heads)], cfg, "first call")
    small = synth.custom(4, 1, 3000, seed=61, needles=2)
    t2 = _compare(small, [1, 0, 0, 1], B.make_cfg(alpha=1.0), "second, smaller call")
    assert t1 > t2 > 0


def test_noalloc_select_rejects_layers_beyond_its_scratch():
    dims = B.make_dims(32, 32, 524288)  # 68 MiB of selection workspace
    assert B.crisp_select_workspace_bytes(dims) > B.NOALLOC_SCRATCH_BYTES
    t = torch.empty(16, dtype=torch.int32, device="cuda")
    out = {"count": t, "idx": t}
    with pytest.raises(B.CrispError) as e:
        B.crisp_select_noalloc(dims, B.make_cfg(), t, t, None, t, out, block_mass=t)
    assert e.value.status == 5
