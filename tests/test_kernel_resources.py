"""Register and scratch budgets of the decode-step kernels (CPU: compiles only).

hipcc reports each gfx950 kernel's resources (``-Rpass-analysis=
kernel-resource-usage``).  Two properties the step's speed rests on are
checked from that report, since neither shows up as a wrong result:

* no kernel of the decode step or of any selection plan (the chunk-exact
  kernels, whose 16-32 keys per thread sit at the 128-register limit,
  included) keeps anything in scratch (private) memory:
  a register array demoted to scratch turns every access into a memory round
  trip, and the dirty scratch lines are written back during the next launch
  (measured: +15 us on each of the two large launches of a 128K step);
* the filter kernel fits four 512-thread workgroups per CU (at most 64
  VGPRs), so every chunk of a 128K step is resident at once.
"""

import os
import re
import shutil
import subprocess

import pytest

from sparse_attention_long_kv_amd import build_lib as bl

pytestmark = pytest.mark.skipif(not os.path.exists(bl.HIPCC) and shutil.which("hipcc") is None,
                                reason="hipcc not available")

# kernels of every selection plan, the decode step and the extensions
# (mangled-name fragments; "merge_kernel" also matches the other merges)
HOT = ("chunk_select_kernel", "merge_regs_kernel", "merge_kernel", "append_bound_kernel",
       "sample_kernel", "filter_kernel", "filter_merge_kernel", "unit_kernel",
       "score_all_kernel", "scores_merge_kernel", "scores_select_attend_kernel",
       "select_attend_kernel", "decode_kernel", "combine_kernel", "append_kv_kernel",
       "linear_gate_kernel", "index_score_kernel")


def _resources(source, tmp_path):
    cmd = [bl.HIPCC] + list(bl.HIP_FLAGS) + [
        "-Rpass-analysis=kernel-resource-usage", "--offload-device-only", "-c",
        os.path.join(bl.CSRC, source), "-o", str(tmp_path / (source + ".o"))]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    out, name = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            out[name] = {}
            continue
        m = re.search(r"remark: +(VGPRs|ScratchSize \[bytes/lane\]): (\d+)", line)
        if m and name:
            out[name]["vgpr" if m.group(1) == "VGPRs" else "scratch"] = int(m.group(2))
    return out


@pytest.fixture(scope="module")
def resources(tmp_path_factory):
    import concurrent.futures as cf
    tmp = tmp_path_factory.mktemp("res")
    res = {}
    srcs = ("indexer.hip", "decode.hip", "append.hip", "linear_gate.hip")
    with cf.ThreadPoolExecutor(len(srcs)) as ex:
        for part in ex.map(lambda s: _resources(s, tmp), srcs):
            res.update(part)
    return res


def test_decode_step_kernels_use_no_scratch(resources):
    hot = {n: r for n, r in resources.items() if any(h in n for h in HOT)}
    assert len(hot) > 40, sorted(resources)
    bad = {n: r["scratch"] for n, r in hot.items() if r.get("scratch", 0) > 0}
    assert not bad, bad


def test_filter_kernel_fits_four_workgroups_per_cu(resources):
    filt = {n: r for n, r in resources.items() if "filter_kernel" in n}
    assert filt
    for n, r in filt.items():
        assert r["vgpr"] <= 64, (n, r)
