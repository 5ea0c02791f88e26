"""The column scale c_j = m_j / Qb of the codec (reading R3: one IEEE fp32
operation, round to nearest even) is computed on the device by a
three-operation sequence instead of a division: q0 = m r, then one fma for
the exact residual m - q0 Qb and one to correct q0 (r = 1/Qb rounded).
This pins that the sequence equals the correctly rounded quotient for every
positive finite fp32 m, for Qb = 127, 31 and 7 (8-, 6- and 4-bit codes), by
exhaustion (tests/division_check.c, OpenMP over the host cores)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def test_column_scale_quotient_is_correctly_rounded(tmp_path):
    exe = tmp_path / "division_check"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", os.path.join(HERE, "division_check.c"), "-lm",
                    "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True, timeout=600).stdout.split()
    got = {float(out[i]): int(out[i + 1]) for i in range(0, len(out), 2)}
    assert got == {127.0: 0, 31.0: 0, 7.0: 0}, got
