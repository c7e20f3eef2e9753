"""The bf16 quantization kernels replace the per-element division x / s by a
reciprocal multiply with one fused correction step (Markstein's method) on
rows whose scale is at least 2^-96.  This test proves, on the CPU and over
every pair of bf16 values |x| <= absmax, that the replacement gives the same
int8 code as the IEEE division (scale absmax / 127), and the same e4m3 code
for the FP8 kernels (scale absmax / 448), and that the kernels' rounding trick (adding
1.5 * 2^23) is round-half-to-even with the code in the low byte.

Host logic only: no GPU and no oracle involved."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def test_reciprocal_quotient_matches_division_exhaustively(tmp_path):
    exe = str(tmp_path / "quotient_check")
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-o", exe,
                    os.path.join(HERE, "csrc", "quotient_check.c"), "-lm"], check=True)
    env = dict(os.environ, OMP_NUM_THREADS=str(min(8, os.cpu_count() or 1)))
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    pairs = int(r.stdout.split()[1])
    assert pairs > 5 * 10 ** 8       # every (absmax, x) pair above the threshold
    # the FP8 kernels' divisor 448: the same quotient gives the same e4m3 codes
    r8 = subprocess.run([exe, "448"], capture_output=True, text=True, env=env, timeout=600)
    assert r8.returncode == 0, r8.stdout + r8.stderr
    assert int(r8.stdout.split()[1]) > 5 * 10 ** 8
