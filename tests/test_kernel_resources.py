"""Register, scratch and occupancy budget of the device kernels, read from the
compiler's resource report (hipcc -Rpass-analysis=kernel-resource-usage; no
GPU needed).

- No kernel of the library spills vector registers or uses scratch memory
  (scalar registers may spill, into vector-register lanes: no memory traffic;
  the large-row selections do).
- Every instantiation of the single-kernel decode fits six waves per SIMD
  (80 VGPRs or fewer), so three eight-wave workgroups share a compute unit;
  the 13B-shape decode runs 2.5 rows per CU and loses its third workgroup
  otherwise.  The grouped-ranking instantiations (four query heads' products
  per token) fit four waves per SIMD (128 VGPRs), two workgroups per CU."""

import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_attention_decode_loki_amd", "csrc")
SOURCES = ["fused_kernels.hip", "decode_kernels.hip", "append_kernels.hip", "probe_kernels.hip"]


def _hipcc():
    for c in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return None


def _report(src, tmp):
    from sparse_attention_decode_loki_amd import build_lib
    cmd = [_hipcc(), *build_lib.HIPCC_FLAGS, "-Rpass-analysis=kernel-resource-usage", "-c",
           os.path.join(CSRC, src), "-o", os.path.join(tmp, src + ".o")]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    kernels, cur = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = kernels.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+(VGPRs|VGPRs Spill|SGPRs Spill|ScratchSize \[bytes/lane\]|"
                      r"Occupancy \[waves/SIMD\]): (\d+)", line)
        if m and cur is not None:
            cur[m.group(1)] = int(m.group(2))
    return kernels


@pytest.fixture(scope="module")
def resources(tmp_path_factory):
    if _hipcc() is None:
        pytest.skip("needs hipcc")
    tmp = str(tmp_path_factory.mktemp("res"))
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        reports = list(ex.map(lambda s: _report(s, tmp), SOURCES))
    return {k: v for rep in reports for k, v in rep.items()}


def test_no_kernel_spills(resources):
    kernels = {k: v for k, v in resources.items() if "VGPRs" in v}
    assert len(kernels) > 50
    bad = {k: v for k, v in kernels.items()
           if v.get("VGPRs Spill", 0) or v.get("ScratchSize [bytes/lane]", 0)}
    assert not bad, bad


def _group_size(name):
    """The last template argument of a fused_kernel instantiation (its
    grouped-ranking head count; mangled as ...Lb?ELi<n>EE)."""
    m = re.search(r"Lb[01]ELi(\d+)EE", name)
    assert m, name
    return int(m.group(1))


def test_fused_kernel_fits_three_workgroups_per_cu(resources):
    fused = {k: v for k, v in resources.items() if "fused_kernel" in k and "VGPRs" in v}
    # {f32, bf16} x D {64, 128} x slab lane counts x {SMALL or not} x {decode, step}
    single = {k: v for k, v in fused.items() if _group_size(k) == 1}
    assert len(single) >= 40
    bad = {k: v for k, v in single.items()
           if v["VGPRs"] > 80 or v.get("Occupancy [waves/SIMD]", 0) < 6}
    assert not bad, bad
    grouped = {k: v for k, v in fused.items() if _group_size(k) > 1}
    assert len(grouped) >= 8  # bf16, D = 128: slab lane counts x {SMALL or not}
    bad = {k: v for k, v in grouped.items()
           if v["VGPRs"] > 128 or v.get("Occupancy [waves/SIMD]", 0) < 4}
    assert not bad, bad
