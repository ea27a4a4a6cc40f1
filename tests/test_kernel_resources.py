"""Resource guard for the gfx950 kernels (no GPU needed): every kernel of the
library compiles with no scratch memory and no vector-register spills.  A
spill in the decode loop puts a wait for all outstanding memory operations
into every tile, so a regression must fail here rather than show up only as a
slower benchmark.  (Scalar-register spills are allowed: they go to lanes of
vector registers, not to memory.)  The compiler's own resource-usage report
is parsed; the 128-head FP8 decode kernels must also keep occupancy 1 with
the whole register file (they are written for it)."""
import os
import re
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from sparse_mla_attention_decode_amd import build as B


def _report(src):
    cmd = [B.hipcc(), *B.compile_flags(), "--cuda-device-only", "-c", "-o", os.devnull,
           "-Rpass-analysis=kernel-resource-usage", src]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    kernels, cur = {}, None
    for line in res.stderr.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = kernels.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[[^\]]*\])?: (\w+) \[-Rpass-analysis", line)
        if m and cur is not None:
            cur[m.group(1).strip()] = m.group(2)
    return kernels


@pytest.fixture(scope="module")
def reports():
    try:
        B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    with ThreadPoolExecutor(max_workers=3) as ex:
        return dict(zip(B.sources(), ex.map(_report, B.sources())))


# The generic decode over the bf16 cache (sparse prefill) keeps Q (144 VGPRs)
# and O (256 AGPRs) like the FP8 kernel but stages rows through registers
# with less care, and spills; these are its current counts, an upper bound
# until that kernel is restructured.  Every other kernel must not spill.
KNOWN_SPILLS = {"_ZN3mla13decode_kernelILi1ELi4EEEvNS_12DecodeParamsE": 57,
                "_ZN3mla13decode_kernelILi1ELi2EEEvNS_12DecodeParamsE": 126}


def test_no_kernel_uses_scratch_or_spills(reports):
    seen = 0
    for src, kernels in reports.items():
        for name, r in kernels.items():
            if "kernel" not in name:
                continue
            seen += 1
            if name in KNOWN_SPILLS:
                assert int(r.get("VGPRs Spill")) <= KNOWN_SPILLS[name], (name, r)
                continue
            assert r.get("ScratchSize") == "0", (os.path.basename(src), name, r)
            assert r.get("VGPRs Spill") == "0", (os.path.basename(src), name, r)
            assert r.get("Dynamic Stack") == "False", (os.path.basename(src), name, r)
    assert seen >= 10


def test_h128_decode_keeps_the_whole_register_file(reports):
    names = {n: r for k in reports.values() for n, r in k.items()}
    dec = {n: r for n, r in names.items() if "decode_fp8_h128_kernel" in n}
    # 656-byte rows: flat / paged address x sparse / dense x 128 / 64 heads;
    # V4 and V4.1: paged sparse x 128 / 64 heads
    assert len(dec) == 12
    for n, r in dec.items():
        h64 = re.search(r"ILb[01]ELb[01]ELb([01])E", n).group(1) == "1"
        # O^T for 128 dims x 128 heads fills the 256 AGPRs; with 64 heads half of it
        assert r["Occupancy"] == "1" and int(r["AGPRs"]) >= (128 if h64 else 256), (n, r)
    for needle in ("combine_packed_kernel", "combine_kernel", "decode_kernel", "indexer_score_kernel",
                   "indexer_topk_kernel", "sched_parallel_kernel"):
        assert any(needle in n for n in names), needle
