"""Host check (no GPU): the divide-free rounding of the W4A8 activation
quantiser (the form the kernels compute: one FMA snapping x * r to a
multiple of 2^-13, a clamp, and the integer read from the low byte after adding
1.5 * 2^23) equals clamp(rint(x / s)) for every scale the quantiser can produce
and every fp16 or bf16 x it can meet (bf16 scales of at least 2^-126; smaller
ones divide), with the reciprocal off by up to one ulp
(quant_rounding_check.c states the argument)."""
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
    exe = str(tmp_path_factory.mktemp("qround") / "quant_rounding_check")
    subprocess.run([CLANG, "-O2", "-o", exe, os.path.join(HERE, "quant_rounding_check.c"), "-lm"], check=True)
    return exe


@pytest.mark.parametrize("mode", ["2", "3"], ids=["fp16", "bf16"])
def test_divide_free_rounding_exhaustive(checker, mode):
    procs = [subprocess.Popen([checker, str(i), str(SLICES), "1", mode], stdout=subprocess.PIPE, text=True)
             for i in range(SLICES)]
    outs = [(p.communicate()[0], p.returncode) for p in procs]
    for out, rc in outs:
        assert rc == 0, out
    total = sum(int(o.split(":")[1].split()[0]) for o, _ in outs)
    assert total > 2_000_000_000  # every reachable (s, x) pair, three reciprocals each
