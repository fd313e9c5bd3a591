"""The activation quantisation's fast quotient (quant_div in the device code)
against the correctly rounded division, on the host: every bf16 x up to the
token's amax, for a stride of bf16 amax values (QUANT_DIV_STRIDE, default 9;
1 checks every amax, about 30 s).  The property is about codes: both values
must round to the same E4M3 code."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def test_quant_div_matches_division(tmp_path):
    exe = tmp_path / "quant_div_check"
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-o", str(exe),
                    os.path.join(HERE, "quant_div_check.c"), "-lm"], check=True)
    stride = os.environ.get("QUANT_DIV_STRIDE", "9")
    r = subprocess.run([str(exe), stride], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout
    assert "mismatches 0" in r.stdout and int(r.stdout.split()[1]) > 10_000_000, r.stdout
