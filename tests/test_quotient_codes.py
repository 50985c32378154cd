"""The token quantizer's division (one IEEE reciprocal per group, then a product corrected by
its exact remainder) gives the same codes as the IEEE quotient x / s that the oracle encodes,
for every bf16 group maximum and every bf16 value below it, both code types and both scale
formats: an exhaustive CPU check (tests/native/quotient_codes.c) against the oracle's
encoders. On the GPU the quantizer is then compared with the oracle bit for bit."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def test_corrected_reciprocal_quotient_codes_exhaustive(orc, tmp_path):
    exe = tmp_path / "quotient_codes"
    src = os.path.join(HERE, "native", "quotient_codes.c")
    libdir = os.path.dirname(orc.LIB_PATH)
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-std=c11", "-o", str(exe), src,
                    "-L" + libdir, "-loracle", "-Wl,-rpath," + libdir, "-lm"], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=900)
    assert r.returncode == 0 and r.stdout.strip() == "0", (r.stdout, r.stderr[-2000:])
