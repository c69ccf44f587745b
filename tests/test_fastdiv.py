"""Host check of the quantize kernel's division scheme: for every finite bf16
amax > 0 and every bf16 x with |x| <= amax, the reciprocal + one-fma-correction
quotient gives the same int8 code as the correctly rounded fp32 quotient
(see tests/fastdiv_check.c); and, for the fp8 variant's divisor 448, the same
e4m3 value.  CPU only; about 40 CPU-seconds."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def test_fastdiv_codes_match_ieee_division_exhaustively(tmp_path):
    exe = tmp_path / "fastdiv_check"
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-fopenmp", "-ffp-contract=off",
                           "-o", str(exe), os.path.join(HERE, "fastdiv_check.c"), "-lm"])
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "mismatches=0" in r.stdout
    assert "pairs=532701119" in r.stdout   # every finite bf16 pair with 0 <= x <= amax, amax > 0
    r = subprocess.run([str(exe), "fp8"], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "mismatches=0" in r.stdout
