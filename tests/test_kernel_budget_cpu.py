"""Register budgets of the timed step kernels, read from the compiler (no GPU needed).

The step kernels' speed rests on their register budgets: a kernel that spills its
state to scratch on every step, or that fits fewer workgroups per CU than it was cut
for, still passes every parity test but loses 10-80 % of its bandwidth.  This test
compiles the kernel translation units for gfx950 exactly as the library build does,
with the compiler's resource remarks, and holds each workload's kernel to its scratch
and occupancy budget.  Template arguments are read from the mangled names in order:
Mamba-2 <NB, IO, TMAX, MFMA fold, copy, checkpoint, heads per workgroup>, GDN <NB,
IO, TMAX, copy, checkpoint, strips per wave>; io 1 = bf16; copy 0/1/2 = none/FP8/MXFP4;
checkpoint 0/1/2 = fp32/fp16/FP8.
"""
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from hybrid_decode_replay_amd import build as hb

CSRC = os.path.join(os.path.dirname(hb.__file__), "csrc")

# (kernel, template arguments): (bytes of scratch per lane allowed, minimum waves per SIMD, workload)
BUDGET = {
    ("mamba2", (8, 1, 1, 1, 0, 0, 1)): (0, 6, "Mamba-2 batch 256, fp32 checkpoint (the headline layer)"),
    ("mamba2", (8, 1, 1, 1, 0, 1, 1)): (0, 6, "Mamba-2, fp16 checkpoint"),
    ("mamba2", (8, 1, 1, 1, 0, 2, 4)): (0, 4, "Mamba-2, FP8 checkpoint (four heads per workgroup)"),
    ("mamba2", (8, 1, 1, 1, 2, 2, 4)): (0, 3, "Mamba-2, FP8 checkpoint + MXFP4 copy"),
    ("mamba2", (8, 1, 1, 1, 1, 0, 4)): (0, 4, "Mamba-2, fp32 checkpoint + FP8 copy"),
    ("mamba2", (8, 1, 1, 1, 2, 0, 4)): (0, 4, "Mamba-2, fp32 checkpoint + MXFP4 copy"),
    ("mamba2", (8, 1, 4, 1, 0, 0, 1)): (0, 6, "Mamba-2 spec rounds, 4 drafts"),
    ("gdn", (8, 1, 1, 0, 0, 1)): (0, 6, "GDN batch 256, fp32 checkpoint"),
    ("gdn", (8, 1, 1, 0, 1, 2)): (0, 5, "GDN, fp16 checkpoint"),
    ("gdn", (8, 1, 1, 0, 2, 2)): (0, 5, "GDN, FP8 checkpoint"),
    # the fold of this one keeps a value in scratch (fold steps only)
    ("gdn", (8, 1, 1, 2, 2, 2)): (8, 5, "GDN, FP8 checkpoint + MXFP4 copy"),
    ("gdn", (8, 1, 1, 1, 0, 2)): (0, 5, "GDN batch 128, fp32 checkpoint + FP8 copy"),
    ("gdn", (8, 1, 1, 2, 0, 2)): (0, 5, "GDN batch 128, fp32 checkpoint + MXFP4 copy"),
    ("gdn", (8, 1, 4, 0, 0, 1)): (0, 6, "GDN spec rounds, 4 drafts"),
}
UNITS = ["mamba2.hip", "mamba2_f16.hip", "mamba2_fp8.hip", "gdn.hip", "gdn_f16.hip", "gdn_fp8.hip"]


def _remarks(src, out_dir):
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    cmd = [hb.HIPCC] + hb.FLAGS + ["--offload-device-only", "-c", os.path.join(CSRC, src), "-o", obj,
                                   "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=CSRC)
    assert r.returncode == 0, r.stderr[-2000:]
    return r.stderr


def _parse(text):
    """{(kind, args): (vgprs, scratch bytes per lane, waves per SIMD)} from the remarks."""
    out, name, vg, sc = {}, None, None, None
    for line in text.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"VGPRs: (\d+)", line)
        if m:
            vg = int(m.group(1))
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m:
            sc = int(m.group(1))
        m = re.search(r"Occupancy \[waves/SIMD\]: (\d+)", line)
        if m and name:
            kind = "mamba2" if "mamba2_step_kernel" in name else "gdn" if "gdn_step_kernel" in name else None
            if kind:
                args = tuple(int(x) for x in re.findall(r"L[ib](\d+)E", name))
                out[(kind, args)] = (vg, sc, int(m.group(1)))
    return out


@pytest.mark.skipif(not (os.path.exists(hb.HIPCC) or shutil.which(hb.HIPCC)), reason="hipcc not available")
def test_timed_step_kernels_keep_their_register_budgets(tmp_path):
    with ThreadPoolExecutor(max_workers=len(UNITS)) as ex:
        texts = list(ex.map(lambda u: _remarks(u, str(tmp_path)), UNITS))
    seen = {}
    for t in texts:
        seen.update(_parse(t))
    bad = []
    for key, (scratch, waves, what) in BUDGET.items():
        assert key in seen, f"{what}: kernel {key} not instantiated"
        vg, sc, occ = seen[key]
        if sc > scratch or occ < waves:
            bad.append(f"{what} {key}: {vg} VGPRs, {sc} B/lane scratch (allowed {scratch}), "
                       f"{occ} waves/SIMD (needs {waves})")
    assert not bad, "\n".join(bad)
