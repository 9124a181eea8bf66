"""Every kernel of the library, compiled for gfx950 with the build's own flags, keeps
its values in registers: the compiler's resource report shows no vector-register
spills and no scratch memory for any of them.  (A spill reload inside a tile loop
waits on the same memory counter as the tile's LDS-DMA, so one spilled register
can serialise a kernel's loads behind its products.)  Runs on the CPU: hipcc
cross-compiles the device code without a GPU."""
import concurrent.futures as cf
import glob
import os
import re
import subprocess

import pytest

from context_cp_attn_amd import build as b


def _resource_report(src: str, out_dir: str) -> list[dict]:
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    cmd = [b.HIPCC, *b.FLAGS, "--cuda-device-only", "-c", src, "-o", obj, "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"hipcc failed on {src}:\n{r.stderr[-3000:]}"
    kernels, cur = [], None
    for line in r.stderr.splitlines():
        m = re.search(r"remark: +(.*?) \[-Rpass-analysis", line)
        if not m:
            continue
        text = m.group(1).strip()
        if text.startswith("Function Name:"):
            cur = {"name": text.split(":", 1)[1].strip()}
            kernels.append(cur)
        elif cur is not None and ":" in text:
            key, val = text.split(":", 1)
            cur[key.strip()] = val.strip()
    return kernels


@pytest.mark.skipif(not os.path.exists(b.HIPCC), reason="hipcc is not installed")
def test_no_kernel_spills_vector_registers_or_uses_scratch(tmp_path):
    srcs = sorted(glob.glob(os.path.join(b.CSRC, "*.hip")))
    assert srcs
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        reports = dict(zip(srcs, ex.map(lambda s: _resource_report(s, str(tmp_path)), srcs)))
    checked, bad = 0, []
    for src, kernels in reports.items():
        for k in kernels:
            checked += 1
            spill, scratch = k.get("VGPRs Spill"), k.get("ScratchSize [bytes/lane]")
            if spill != "0" or scratch != "0":
                bad.append((os.path.basename(src), k["name"], f"VGPR spill {spill}", f"scratch {scratch} B/lane"))
    # the attention sources alone instantiate dozens of kernels; an empty report
    # would mean the remarks were not parsed
    assert checked >= 40, f"only {checked} kernel reports parsed"
    assert not bad, "kernels that spill or use scratch:\n" + "\n".join(map(str, bad))
