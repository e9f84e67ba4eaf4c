"""Host check (no GPU): the divide-free quotient of the INT4-FP8 activation
quantiser (one divide per row for the reciprocal, then per value one multiply
and Markstein's FMA correction, on values scaled by 2^64 for bf16 rows with
s < 2^-60) gives the same E4M3 code as the correctly rounded quotient for
every scale the quantiser can produce and every fp16 or bf16 x it can meet
(bf16 scales of at least 2^-126; smaller ones divide)
(fp8_quotient_check.c states the argument)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CLANG = shutil.which("clang") or "/opt/rocm/llvm/bin/clang"
SLICES = 8


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    if not os.path.exists(CLANG):
        pytest.skip("no clang to build the host checker")
    exe = str(tmp_path_factory.mktemp("fp8q") / "fp8_quotient_check")
    subprocess.run([CLANG, "-O2", "-ffp-contract=off", "-o", exe, os.path.join(HERE, "fp8_quotient_check.c"), "-lm"],
                   check=True)
    return exe


@pytest.mark.parametrize("mode", ["0", "1"], ids=["fp16", "bf16"])
def test_divide_free_quotient_exhaustive(checker, mode):
    procs = [subprocess.Popen([checker, str(i), str(SLICES), mode], stdout=subprocess.PIPE, text=True)
             for i in range(SLICES)]
    outs = [(p.communicate()[0], p.returncode) for p in procs]
    for out, rc in outs:
        assert rc == 0, out
    total = sum(int(o.split(":")[1].split()[0]) for o, _ in outs)
    assert total > 400_000_000  # every reachable (s, x) pair
