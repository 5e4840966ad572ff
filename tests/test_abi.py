"""Host-side tests of the C ABI (no GPU): the library loads, exports every
declared entry point, sizes its buffers as documented and rejects invalid
arguments before touching the device."""
import ctypes
import os
import re
import shutil
import subprocess

import pytest

from dynamic_sparse_attention_proxy_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "crisp.h")

# Fake device addresses: never dereferenced, every case fails validation first.
P16 = 0x10000
P8 = 0x10008


def _declared():
    text = open(HEADER).read()
    return re.findall(r"CRISP_API\s+[\w\s\*]+?\b(crisp_\w+)\s*\(", text)


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert len(names) == 21
    lib = B.lib()
    for n in names:
        assert hasattr(lib, n), n
    if shutil.which("nm"):
        out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True).stdout
        exported = set(re.findall(r"\bT (crisp_\w+)", out))
        assert set(names) == exported


def test_abi_version_and_status_strings():
    assert B.crisp_abi_version() >> 16 == 5  # every attention call takes a work-queue workspace
    lib = B.lib()
    for s in range(8):
        assert lib.crisp_status_string(s)
    assert lib.crisp_status_string(99) == b"unknown status"


def test_sizes():
    d = B.make_dims(32, 8, 524288)
    N = 524288 // 128
    assert B.crisp_list_capacity(d) == 32 * N * (N + 1) // 2
    ws = B.crisp_select_workspace_bytes(d)
    # pooled keys of every KV group and the four block-mass planes; the pooled
    # queries never reach memory (each logit workgroup pools its own)
    assert ws >= 8 * N * 128 * 4 + 4 * 32 * N * 4
    assert ws < 24 << 20
    assert B.crisp_proxy_scratch_bytes(d) >= 32 * 128 * 4
    bad = B.make_dims(32, 8, 255)
    assert B.crisp_list_capacity(bad) == 0
    assert B.crisp_select_workspace_bytes(bad) == 0
    # a partial last block counts as a block
    r = B.make_dims(4, 2, 1000)
    assert B.crisp_list_capacity(r) == 4 * 8 * 9 // 2
    assert B.crisp_proxy_scratch_bytes(r) >= 4 * 8 * 128 * 16


def _dense(dims, q=P16, k=P16, v=P16, out=P16, fp32=0, lse=None, ws=P16, ws_bytes=1 << 20):
    return B.lib().crisp_dense_attn(ctypes.byref(dims), q, k, v, out, fp32, lse, ws, ws_bytes, None)


@pytest.mark.parametrize("hq,hkv,n,d,blk,status", [
    (32, 8, 255, 128, 128, 2),     # n below two blocks
    (32, 8, 128, 128, 128, 2),
    (32, 8, 4096, 64, 128, 2),     # head_dim
    (32, 8, 4096, 128, 64, 2),     # block
    (30, 8, 4096, 128, 128, 2),    # Hq % Hkv
    (32, 0, 4096, 128, 128, 2),
    (32, 8, 1 << 21, 128, 128, 2), # beyond the supported length
    (32, 8, 524289, 128, 128, 2),  # one position past the longest layer
])
def test_shape_errors(hq, hkv, n, d, blk, status):
    dims = B.crisp_dims(hq, hkv, n, d, blk, 0.088)
    assert _dense(dims) == status


def test_pointer_and_param_errors():
    dims = B.make_dims(4, 2, 1024)
    assert _dense(dims, q=None) == 1
    assert _dense(dims, out=P8) == 4
    assert _dense(dims, lse=P8) == 4
    assert _dense(dims, fp32=2) == 3
    bad_scale = B.crisp_dims(4, 2, 1024, 128, 128, -1.0)
    assert _dense(bad_scale) == 3
    lib = B.lib()
    assert lib.crisp_sparse_attn(ctypes.byref(dims), P16, P16, P16, None, P16, P16, 0, None, P16, 1 << 20,
                                 None) == 1
    # the attention work queue: required, and at least crisp_attn_workspace_bytes
    need = B.crisp_attn_workspace_bytes(dims)
    assert 32 <= need <= 4096
    assert _dense(dims, ws=None) == 1
    assert _dense(dims, ws_bytes=need - 1) == 5
    assert lib.crisp_sparse_attn(ctypes.byref(dims), P16, P16, P16, P16, P16, P16, 0, None, P16, need - 1,
                                 None) == 5
    assert lib.crisp_sparse_attn_cols(ctypes.byref(dims), P16, P16, P16, P16, P16, P16, P16, P16, P16, None, 1 << 20,
                                      None) == 1
    assert lib.crisp_sparse_attn_cols(ctypes.byref(dims), P16, P16, P16, P16, P16, P16, P16, P16, P16, P16, need - 1,
                                      None) == 5
    assert B.crisp_attn_workspace_bytes(B.make_dims(32, 8, 255)) == 0
    # proxy scratch too small
    assert lib.crisp_proxy(ctypes.byref(dims), P16, P16, P16, None, None, P16, 16, None) == 5
    assert lib.crisp_proxy(None, P16, P16, P16, None, None, P16, 1 << 30, None) == 1


NAN, INF = float("nan"), float("inf")


@pytest.mark.parametrize("field,value", [
    ("tau", 1.5), ("tau", -0.1), ("alpha", 0.0), ("gamma_pe", 0.0), ("gamma_pe", 1.01), ("kmin_blocks", 0),
    ("sink_width", 0), ("recency_width", 600), ("nf_stat", 2), ("route_override", 3),
    ("tau", NAN), ("alpha", NAN), ("alpha", INF), ("gamma_pe", NAN), ("tau", -INF),
])
def test_cfg_errors(field, value):
    dims = B.make_dims(4, 2, 1024)
    cfg = B.make_cfg()
    setattr(cfg, field, value)
    lib = B.lib()
    assert lib.crisp_route(ctypes.byref(dims), ctypes.byref(cfg), P16, None, P16, P16, None) == 3
    blocks = B.crisp_blocks()
    blocks.count = P16
    blocks.idx = P16
    assert lib.crisp_select(ctypes.byref(dims), ctypes.byref(cfg), P16, P16, P16, None, P16, ctypes.byref(blocks), P16,
                            1 << 40, None) == 3


@pytest.mark.parametrize("value", [NAN, INF, -INF, 0.0, -0.5])
def test_non_finite_scale_and_thresholds_are_param_errors(value):
    """NaN and infinite method parameters are rejected before any launch
    (CRISP_ERR_PARAM), never passed on to the kernels."""
    lib = B.lib()
    dims = B.crisp_dims(4, 2, 1024, 128, 128, value)
    assert _dense(dims) == 3
    good = B.make_dims(4, 2, 1024)
    cfg = B.make_cfg()
    blocks = B.crisp_blocks()
    blocks.count = P16
    blocks.idx = P16
    assert lib.crisp_select_gamma(ctypes.byref(good), ctypes.byref(cfg), value, P16, P16, P16, None, P16,
                                  ctypes.byref(blocks), P16, 1 << 40, None) == 3
    if value != 0.0:  # a JSD threshold of 0 is allowed
        assert lib.crisp_route_jsd(ctypes.byref(good), ctypes.c_float(value), P16, P16, P16, P16, P16, None, P16,
                                   1 << 40, None) == 3


def test_route_cols_validation():
    """crisp_route_cols checks its pointers and the configuration like
    crisp_route, takes any widths in 1..n/2, and reaches the device check
    with valid arguments (no GPU here: 6)."""
    lib = B.lib()
    dims = B.make_dims(4, 2, 1024)

    def call(cfg, colm=P16, c=P16, r=P16, d=dims):
        return lib.crisp_route_cols(ctypes.byref(d), ctypes.byref(cfg), colm, c, r, None)

    assert call(B.make_cfg(), colm=None) == 1
    assert call(B.make_cfg(), c=None) == 1
    assert call(B.make_cfg(), r=None) == 1
    assert call(B.make_cfg(), colm=P8) == 4
    assert call(B.make_cfg(tau=float("nan"))) == 3
    bad = B.make_cfg()
    bad.sink_width = 0
    assert call(bad) == 3
    bad = B.make_cfg()
    bad.recency_width = 513
    assert call(bad) == 3
    for ws, wr in ((1, 1), (64, 200), (512, 512)):
        cfg = B.make_cfg()
        cfg.sink_width, cfg.recency_width = ws, wr
        assert call(cfg) == 6
    assert call(B.make_cfg(), d=B.make_dims(4, 3, 1024)) == 2


def test_select_noalloc_validation():
    """The allocation-free selection validates like crisp_select; a layer
    whose selection workspace exceeds the static scratch is
    CRISP_ERR_WORKSPACE before any device call, a fitting one reaches the
    device check (no GPU here: 6)."""
    lib = B.lib()
    cfg = B.make_cfg()
    blocks = B.crisp_blocks()
    blocks.count = P16
    blocks.idx = P16

    def call(dims, q=P16, route=P16, mass=P16, blk=blocks, c=cfg):
        return lib.crisp_select_noalloc(ctypes.byref(dims), ctypes.byref(c), q, P16, None, mass, route,
                                        None if blk is None else ctypes.byref(blk), None)

    text = open(HEADER).read()
    m = re.search(r"#define\s+CRISP_NOALLOC_SCRATCH_BYTES\s+\((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == B.NOALLOC_SCRATCH_BYTES
    for hq, hkv, n in ((32, 8, 524288), (64, 8, 524288), (28, 4, 131072), (4, 2, 1024)):
        d = B.make_dims(hq, hkv, n)
        assert B.crisp_select_workspace_bytes(d) <= B.NOALLOC_SCRATCH_BYTES
        assert call(d) == 6
    for hq, hkv, n in ((32, 32, 524288), (64, 16, 524288)):
        d = B.make_dims(hq, hkv, n)
        assert B.crisp_select_workspace_bytes(d) > B.NOALLOC_SCRATCH_BYTES
        assert call(d) == 5
    d = B.make_dims(4, 2, 1024)
    assert call(d, q=None) == 1
    assert call(d, route=P8) == 4
    assert call(d, mass=None) == 1
    assert call(d, blk=None) == 1
    assert call(d, c=B.make_cfg(alpha=float("nan"))) == 3


def test_select_errors():
    dims = B.make_dims(4, 2, 1024)
    cfg = B.make_cfg()
    lib = B.lib()
    blocks = B.crisp_blocks()
    blocks.count = P16
    blocks.idx = None
    assert lib.crisp_select(ctypes.byref(dims), ctypes.byref(cfg), P16, P16, P16, None, P16, ctypes.byref(blocks), P16,
                            1 << 40, None) == 1
    blocks.idx = P16
    blocks.v_score = P8
    assert lib.crisp_select(ctypes.byref(dims), ctypes.byref(cfg), P16, P16, P16, None, P16, ctypes.byref(blocks), P16,
                            1 << 40, None) == 4
    blocks.v_score = None
    assert lib.crisp_select(ctypes.byref(dims), ctypes.byref(cfg), P16, P16, P16, None, P16, ctypes.byref(blocks), P16,
                            64, None) == 5
    assert lib.crisp_select_gamma(ctypes.byref(dims), ctypes.byref(cfg), 0.0, P16, P16, P16, None, P16,
                                  ctypes.byref(blocks), P16, 1 << 40, None) == 3
    assert lib.crisp_select_gamma(ctypes.byref(dims), ctypes.byref(cfg), 1.2, P16, P16, P16, None, P16,
                                  ctypes.byref(blocks), P16, 1 << 40, None) == 3


def test_map_or_block_mass_rules():
    """The proxy output is the map, the block masses or both: at least one,
    each aligned; routing from block masses needs one-block widths.  A call
    that passes validation reaches the device check (no GPU here: 6)."""
    dims = B.make_dims(4, 2, 1024)
    lib = B.lib()
    sb = 1 << 30
    assert lib.crisp_proxy(ctypes.byref(dims), P16, P16, None, None, None, P16, sb, None) == 1
    assert lib.crisp_proxy(ctypes.byref(dims), P16, P16, None, P8, None, P16, sb, None) == 4
    assert lib.crisp_proxy(ctypes.byref(dims), P16, P16, P8, P16, None, P16, sb, None) == 4
    assert lib.crisp_proxy(ctypes.byref(dims), P16, P16, None, P16, None, P16, sb, None) == 6
    assert lib.crisp_proxy(ctypes.byref(dims), P16, P16, P16, P16, P16, P16, sb, None) == 6
    cfg = B.make_cfg()
    assert lib.crisp_route(ctypes.byref(dims), ctypes.byref(cfg), None, None, P16, P16, None) == 1
    assert lib.crisp_route(ctypes.byref(dims), ctypes.byref(cfg), None, P16, P16, P16, None) == 6
    for field in ("sink_width", "recency_width"):
        c2 = B.make_cfg()
        setattr(c2, field, 64)
        assert lib.crisp_route(ctypes.byref(dims), ctypes.byref(c2), None, P16, P16, P16, None) == 3
        assert lib.crisp_route(ctypes.byref(dims), ctypes.byref(c2), P16, None, P16, P16, None) == 6
    blocks = B.crisp_blocks()
    blocks.count = P16
    blocks.idx = P16
    assert lib.crisp_select(ctypes.byref(dims), ctypes.byref(cfg), P16, P16, None, None, P16, ctypes.byref(blocks),
                            P16, 1 << 40, None) == 1
    assert lib.crisp_select(ctypes.byref(dims), ctypes.byref(cfg), P16, P16, None, P16, P16, ctypes.byref(blocks),
                            P16, 1 << 40, None) == 6
    assert lib.crisp_select_gamma(ctypes.byref(dims), ctypes.byref(cfg), 0.95, P16, P16, None, P8, P16,
                                  ctypes.byref(blocks), P16, 1 << 40, None) == 4


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="libcrisp.so not found"):
        B.lib()


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="needs hipcc for a host build")
@pytest.mark.parametrize("sanitized", [False, True])
@pytest.mark.parametrize("hq,hkv,nblk,runs", [(32, 8, 4096, False), (28, 4, 1024, False), (1, 1, 32, False),
                                              (3, 1, 5, False), (16, 16, 64, False), (4, 2, 3, False),
                                              (32, 8, 4096, True), (28, 4, 1024, True), (2, 1, 128, True)])
def test_row_map_is_a_bijection(tmp_path_factory, hq, hkv, nblk, runs, sanitized):
    """The workgroup map (and its deal in runs of 16 blocks), also built
    with host AddressSanitizer and UndefinedBehaviorSanitizer (host code
    only; any report aborts)."""
    exe = tmp_path_factory.getbasetemp() / ("row_map_check_san" if sanitized else "row_map_check")
    if not exe.exists():
        hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
        flags = ["-O2"]
        if sanitized:
            flags = ["-O1", "-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                     "-Xarch_host", "-fno-sanitize-recover=all"]
        subprocess.run([hipcc, *flags, "-std=c++17", os.path.join(ROOT, "tests", "cpp", "row_map_check.cpp"),
                        "-o", str(exe)], check=True, capture_output=True)
    r = subprocess.run([str(exe), str(hq), str(hkv), str(nblk)] + (["runs"] if runs else []), capture_output=True,
                       text=True)
    assert r.returncode == 0, r.stdout + r.stderr


def test_prefill_marshalling_and_composed_chains(monkeypatch):
    """The binding's crisp_prefill hands the default layer to the library's
    one-call crisp_prefill (dense_below None -> -1, the library default);
    with a gamma, or a map in the buffers, it calls the steps one by one and
    never gates."""
    import types

    seen = []

    class FakeLib:
        def crisp_prefill(self, dims, cfg, dense_below, *rest):
            seen.append(dense_below)
            return 0

    monkeypatch.setattr(B, "_lib", FakeLib())
    calls = []
    for name in ("crisp_proxy", "crisp_route", "crisp_select", "crisp_select_gamma", "crisp_sparse_attn",
                 "crisp_dense_attn"):
        monkeypatch.setattr(B, name, lambda *a, _n=name, **kw: calls.append(_n))
    import torch

    bufs = types.SimpleNamespace(out=torch.empty(1), lse=None, attn_map=None, block_mass=None, row_lse=None,
                                 partials=None, c_struct=None, route=None, blocks={"count": None, "idx": None},
                                 workspace=None, prefill_workspace=torch.empty(16, dtype=torch.uint8),
                                 attn_workspace=None)
    monkeypatch.setattr(B, "_stream", lambda s: None)
    cfg = B.make_cfg()
    for n in (1024, B.DENSE_BELOW, 4 * B.DENSE_BELOW):
        B.crisp_prefill(B.make_dims(32, 8, n), cfg, None, None, None, bufs)
    B.crisp_prefill(B.make_dims(32, 8, 1024), cfg, None, None, None, bufs, dense_below=0)
    B.crisp_prefill(B.make_dims(32, 8, 1024), cfg, None, None, None, bufs, dense_below=4096)
    assert seen == [-1, -1, -1, 0, 4096] and calls == []
    B.crisp_prefill(B.make_dims(32, 8, 1024), cfg, None, None, None, bufs, gamma=0.95)
    assert calls == ["crisp_proxy", "crisp_route", "crisp_select_gamma", "crisp_sparse_attn"]
    calls.clear()
    bufs.attn_map = torch.empty(1)
    B.crisp_prefill(B.make_dims(32, 8, 1024), cfg, None, None, None, bufs, use_map=True)
    assert calls == ["crisp_proxy", "crisp_route", "crisp_select", "crisp_sparse_attn"]
    assert len(seen) == 5


def test_prefill_gate_default_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define\s+CRISP_DENSE_BELOW_DEFAULT\s+(\d+)", text)
    assert m and int(m.group(1)) == B.DENSE_BELOW


def test_prefill_validation():
    """The one-call layer validates every argument before any launch,
    whichever way the gate goes; a valid call reaches the device check (6)."""
    lib = B.lib()
    dims = B.make_dims(4, 2, 1024)
    ws = B.crisp_prefill_workspace_bytes(dims)
    ps, ss = B.crisp_proxy_scratch_bytes(dims), B.crisp_select_workspace_bytes(dims)
    assert ws >= -(-ps // 256) * 256 + ss + B.crisp_attn_workspace_bytes(dims)
    assert B.crisp_prefill_workspace_bytes(B.make_dims(4, 2, 255)) == 0
    blocks = B.crisp_blocks()
    blocks.count = P16
    blocks.idx = P16

    def call(dims=dims, cfg=None, gate=-1, q=P16, k=P16, v=P16, blk=blocks, mass=None, cs=None, rt=None, out=P16,
             fp32=0, lse=None, w=P16, wb=ws):
        cfg = cfg or B.make_cfg()
        return lib.crisp_prefill(ctypes.byref(dims), ctypes.byref(cfg), gate, q, k, v,
                                 None if blk is None else ctypes.byref(blk), mass, cs, rt, out, fp32, lse, w, wb,
                                 None)

    assert call() == 6
    assert call(gate=0) == 6
    assert call(gate=1 << 30) == 6
    assert call(mass=P16, cs=P16, rt=P16, lse=P16, fp32=1) == 6
    assert call(v=None) == 1
    assert call(blk=None) == 1
    assert call(out=None) == 1
    assert call(w=None) == 1
    assert call(mass=P8) == 4
    assert call(rt=P8) == 4
    assert call(lse=P8) == 4
    assert call(wb=ws - 1) == 5
    assert call(fp32=2) == 3
    assert call(cfg=B.make_cfg(sink_width=64)) == 3
    assert call(cfg=B.make_cfg(tau=float("nan"))) == 3
    assert call(dims=B.crisp_dims(4, 2, 1024, 128, 128, float("nan"))) == 3
    # the gate does not skip validation: a short layer with a bad list pointer fails too
    b2 = B.crisp_blocks()
    b2.count = P16
    assert call(blk=b2, gate=1 << 30) == 1


def test_route_jsd_errors():
    """The JSD routing signal validates like the other calls: a finite,
    non-negative threshold, every required pointer, an aligned optional
    estimate and a large enough workspace; then the device check (6)."""
    dims = B.make_dims(4, 2, 1024)
    lib = B.lib()
    ws = B.crisp_route_jsd_workspace_bytes(dims)
    assert ws >= 4 * 128 * 4 + 4 * 8 * 4
    assert B.crisp_route_jsd_workspace_bytes(B.make_dims(4, 2, 255)) == 0

    def call(tau=0.1, q=P16, k=P16, mass=P16, dist=P16, route=P16, est=None, w=P16, wb=ws):
        return lib.crisp_route_jsd(ctypes.byref(dims), tau, q, k, mass, dist, route, est, w, wb, None)

    assert call() == 6
    assert call(est=P16) == 6
    assert call(tau=-0.01) == 3
    assert call(tau=float("nan")) == 3
    assert call(tau=float("inf")) == 3
    assert call(mass=None) == 1
    assert call(k=None) == 1
    assert call(route=None) == 1
    assert call(dist=P8) == 4
    assert call(est=P8) == 4
    assert call(wb=ws - 4) == 5
    bad = B.crisp_dims(4, 2, 255, 128, 128, 0.088)
    assert lib.crisp_route_jsd(ctypes.byref(bad), 0.1, P16, P16, P16, P16, P16, None, P16, ws, None) == 2
