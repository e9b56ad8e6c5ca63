"""Exhaustive CPU proof that the quantize kernel's fast division returns the IEEE
quotient RN(x/a) for every bf16 and every fp16 pair inside the region where the
kernel uses it (see tests/native/div_check.c): the per-block reciprocal (the
hardware's approximate reciprocal refined by one fused-multiply-add step) is
RN(1/a) for every approximation within 2 ulp, and Markstein's correction then
gives the quotient.  The kernel divides every other element with the full IEEE
sequence."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    out = str(tmp_path_factory.mktemp("divcheck") / "div_check")
    subprocess.run([cc, "-O2", "-ffp-contract=off", "-o", out,
                    os.path.join(HERE, "native", "div_check.c"), "-lm"], check=True)
    return out


@pytest.mark.parametrize("fmt", ["bf16", "fp16"])
def test_fast_division_is_exact(checker, fmt):
    res = subprocess.run([checker, fmt], capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stdout + res.stderr
    lines = res.stdout.strip().splitlines()
    rec = lines[-2].split()
    assert rec[0] == "recips" and rec[-1] == "0"
    assert int(rec[1]) > (20_000 if fmt == "bf16" else 50_000)   # every absmax of the fast region, 2-3 each
    last = lines[-1].split()
    assert last[0] == "pairs" and last[-1] == "0"
    assert int(last[3]) > 200_000_000          # the fast region is the bulk of the pairs
