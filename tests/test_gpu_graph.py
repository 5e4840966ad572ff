"""A whole layer captured in a HIP graph (torch.cuda.CUDAGraph).

Every entry point only enqueues kernels on the caller's stream: no
allocation, no memset, no synchronisation.  So the chain can be captured
once and replayed, and each replay must reproduce the eager result bit for
bit (the chain is deterministic).  Between replays the outputs are
overwritten by eager work, and the program synchronises, so that a replay
that skipped a node or read stale memory would show."""
import pytest
import torch

from dynamic_sparse_attention_proxy_amd import binding as B
from dynamic_sparse_attention_proxy_amd import synth

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    yield
    torch.cuda.synchronize()


def _capture(fn):
    """Warm up on a side stream, then capture one call of fn."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    torch.cuda.synchronize()
    return graph


def _replay_and_check(graph, outputs, refs, label):
    for r in range(REPLAYS):
        for t in outputs:  # eager work between replays: clobber every output
            if t.dtype.is_floating_point:
                t.fill_(float("nan"))
            else:
                t.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (t, ref) in enumerate(zip(outputs, refs)):
            assert torch.equal(t, ref), f"{label}: replay {r}, output {i}"


@pytest.mark.parametrize("override", [B.ROUTE_AUTO, B.ROUTE_FORCE_VS, B.ROUTE_FORCE_PE])
def test_block_chain_replays_from_a_graph(override):
    hq, hkv, n = 8, 2, 4096 + 77  # a partial last block as well
    x = synth.make_routing_family(seq_len=n, num_q_heads=hq, num_kv_heads=hkv, device="cuda")
    dims = B.make_dims(hq, hkv, n)
    cfg = B.make_cfg(tau=0.2, route_override=override)
    bufs = B.CrispBuffers(dims, out_dtype=torch.float32)

    def layer():
        B.crisp_prefill(dims, cfg, x.q, x.k, x.v, bufs, dense_below=0)

    print(f"[graph] block chain override={override}", flush=True)
    layer()
    torch.cuda.synchronize()
    outputs = [bufs.out, bufs.lse, bufs.c_struct, bufs.route, bufs.blocks["count"]]
    refs = [t.clone() for t in outputs]
    # the listed entries of idx (entries past a row's count are not written)
    N = B.num_blocks(n)
    count = refs[4].cpu()
    idx_ref = bufs.blocks["idx"].clone()
    graph = _capture(layer)
    _replay_and_check(graph, outputs, refs, f"block chain {override}")
    idx = bufs.blocks["idx"].cpu()
    ir = idx_ref.cpu()
    for h in range(hq):
        base = h * (N * (N + 1) // 2)
        for qb in range(N):
            s = base + qb * (qb + 1) // 2
            c = int(count[h, qb])
            assert torch.equal(idx[s:s + c], ir[s:s + c]), (h, qb)
    if override == B.ROUTE_AUTO:
        assert 0 < int(refs[3].sum()) < hq  # both routes inside the graph


def test_token_chain_replays_from_a_graph():
    hq, hkv, n = 4, 2, 3100
    x = synth.make_inputs(synth.custom(hq, hkv, n, seed=31, needles=4), device="cuda")
    dims = B.make_dims(hq, hkv, n)
    cfg = B.make_cfg(route_override=B.ROUTE_FORCE_VS)
    bufs = B.CrispBuffers(dims, tokens=True)

    def layer():
        B.crisp_prefill_tokens(dims, cfg, x.q, x.k, x.v, bufs)

    print("[graph] token chain", flush=True)
    layer()
    torch.cuda.synchronize()
    outputs = [bufs.out, bufs.lse, bufs.ncols, bufs.col_below, bufs.blocks["count"]]
    refs = [t.clone() for t in outputs]
    graph = _capture(layer)
    _replay_and_check(graph, outputs, refs, "token chain")
