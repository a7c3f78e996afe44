"""The fp8 key store divides each key's values by its scale with one
reciprocal per key and an fma correction per value (see the store kernel).
This host test checks that arithmetic against float32 division on random bf16
keys: every quotient whose e4m3fn code can be nonzero must match bit for bit.
The library's own output is compared with the oracle by the GPU store tests."""
from __future__ import annotations

import subprocess
from pathlib import Path

HERE = Path(__file__).resolve().parent


def test_division_free_quotient_matches_division(tmp_path):
    exe = tmp_path / "store_quotient_check"
    subprocess.run(["gcc", "-O2", "-mfma", "-ffp-contract=off", str(HERE / "store_quotient_check.c"),
                    "-o", str(exe), "-lm"], check=True)
    for seed in ("88172645463325252", "1234567"):
        r = subprocess.run([str(exe), "15000000", seed], capture_output=True, text=True, timeout=300)
        assert r.returncode == 0, r.stdout + r.stderr
        assert " 0 differ" in r.stdout
