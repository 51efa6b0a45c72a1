"""The block scale's division by 6 as the GPU kernels form it, pinned over every input.

The NVFP4 block scale is E4M3(min(fp32(fp32(amax * q) / 6), 448)) (the library's reading of
the group-16 quantization of "Cake SiTU backend"; the pages give no formula).  The kernels
form the quotient as RN(x * RN(1/6)) with one fused multiply-add correction of the
residual instead of an IEEE division.  A plain C program (tests/c/scale_division.c, built
with gcc, operations rounded one at a time, the C library's fmaf) runs both over every
non-negative finite float x and lists the inputs where they differ; here the oracle's
E4M3 encoder must give the same scale byte for both quotients of every listed input.
"""

import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _has_fma():
    try:
        with open("/proc/cpuinfo") as fh:
            return any(ln.startswith("flags") and " fma " in ln + " " for ln in fh)
    except OSError:
        return False


def test_fma_quotient_gives_the_ieee_quotients_scale_byte_for_every_float(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    exe = tmp_path / "scale_division"
    flags = ["-O2", "-std=c99", "-ffp-contract=off", "-fopenmp", "-Wall", "-Werror"]
    if _has_fma():
        flags.append("-mfma")                 # hardware fused multiply-add (same result)
    subprocess.run([gcc, *flags, os.path.join(ROOT, "tests", "c", "scale_division.c"), "-lm",
                    "-o", str(exe)], check=True)
    out = tmp_path / "differ.bin"
    r = subprocess.run([str(exe), str(out)], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr
    checked, differ = (int(v) for v in r.stdout.split()[1::2])
    assert checked == 0x7F800000                   # every non-negative finite float
    rec = np.fromfile(out, dtype=np.uint32).reshape(-1, 3)
    assert rec.shape[0] == differ
    vals = rec.view(np.float32).astype(np.float64)
    x, fma_q, ieee_q = vals[:, 0], vals[:, 1], vals[:, 2]
    # where the two quotients differ they are one float apart ...
    assert np.all(np.abs(rec[:, 1].astype(np.int64) - rec[:, 2].astype(np.int64)) == 1)
    # ... and the scale byte is the same (min(., 448) then round to nearest even)
    b_fma = oracle.e4m3_encode(np.minimum(fma_q, 448.0))
    b_ieee = oracle.e4m3_encode(np.minimum(ieee_q, 448.0))
    assert np.array_equal(b_fma, b_ieee)
    # the differences sit far below the smallest E4M3 scale: every such block scales to 0
    assert differ == 0 or (x.max() < 2.0 ** -100 and np.all(b_ieee == 0))
