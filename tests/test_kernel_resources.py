"""Resource usage of every kernel, from the compiler's own report (host-side
cross-compile for gfx950; no GPU).

No kernel may use scratch memory.  Scratch accesses count in the same
vector-memory counter as the LDS-DMA prefetches, so a wait the compiler
places for a scratch load also waits for the tiles in flight.  A branch
choosing which of several accumulators to update was once compiled into a
pointer select over a stack array, which put a pipeline-wide wait in every
step of the proxy pass while every result stayed correct.  The attention
kernels must also keep two waves per SIMD (two workgroups per CU)."""
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from dynamic_sparse_attention_proxy_amd import build as bld

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="needs hipcc for a gfx950 cross-compile")


def _report(src, out_dir):
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + bld.flags_for(src) + ["-Rpass-analysis=kernel-resource-usage", "-c", os.path.join(bld.CSRC, src),
                                 "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    kernels, name = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            kernels[name] = {}
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[[^\]]*\])?: (\d+)", line)
        if m and name is not None:
            kernels[name][m.group(1).strip()] = int(m.group(2))
    return src, kernels


@pytest.fixture(scope="module")
def reports(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("resources"))
    with ThreadPoolExecutor(max_workers=4) as ex:
        return dict(ex.map(lambda s: _report(s, out), bld.SOURCES))


def test_every_kernel_source_reports_its_kernels(reports):
    for src in ("proxy.hip", "select.hip", "attn.hip", "jsd.hip", "cols.hip"):
        assert reports[src], f"no kernel resource report for {src}"
    assert not reports["api.hip"]  # the C ABI layer holds no kernels


def test_no_kernel_uses_scratch(reports):
    bad = {name: k.get("ScratchSize") for ks in reports.values() for name, k in ks.items()
           if k.get("ScratchSize", 0) != 0}
    assert not bad, bad


def test_attention_keeps_two_waves_per_simd(reports):
    attn = {name: k for name, k in reports["attn.hip"].items() if "fa_fwd_kernel" in name}
    assert len(attn) == 4
    for name, k in attn.items():
        assert k.get("Occupancy") == 2, (name, k)
