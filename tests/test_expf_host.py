"""The gated activation's exp (int8_hadamard_rotated_amd/csrc/expf_cr.h), built
for the host from the same source as the kernels, against exp rounded once
from x87 extended precision on every binary32 argument in [-104, 89] (about
2.2e9 of them), and its double-double path alone on a strided sample.  No GPU
is involved; the GPU tests check the device build on a large sample."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER_DIR = os.path.join(ROOT, "int8_hadamard_rotated_amd", "csrc")

PROGRAM = r'''
#include <cmath>
#include <cstdio>
#include <cstring>
#include "expf_cr.h"
static unsigned bits(float f) { unsigned u; std::memcpy(&u, &f, 4); return u; }
int main(int argc, char **argv)
{
    const long long stride = argc > 1 ? atoll(argv[1]) : 1;
    const bool slow = argc > 2;
    long long bad = 0, checked = 0;
    #pragma omp parallel for reduction(+:bad,checked) schedule(dynamic, 1 << 16)
    for (long long i = 0; i < (1LL << 32); i += stride) {
        const unsigned u = (unsigned)i;
        float x;
        std::memcpy(&x, &u, 4);
        if (!(x >= -104.0f && x <= 89.0f))
            continue;
        const float want = (float)expl((long double)x);
        const float got = slow ? convrot_expf::expf_slow(x) : convrot_expf::expf_cr(x);
        ++checked;
        if (bits(want) != bits(got)) {
            if (bad < 10)
                std::printf("x=%a got %a want %a\n", x, got, want);
            ++bad;
        }
    }
    std::printf("checked %lld mismatches %lld\n", checked, bad);
    return bad != 0;
}
'''


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    d = tmp_path_factory.mktemp("expf")
    src = d / "check.cpp"
    src.write_text(PROGRAM)
    exe = d / "check"
    subprocess.run(["g++", "-O2", "-std=c++17", "-fopenmp", "-mfma", "-ffp-contract=off",
                    "-DCONVROT_HD=", "-DCONVROT_NOINLINE=__attribute__((noinline))",
                    "-I", HEADER_DIR, str(src), "-o", str(exe)], check=True, capture_output=True)
    return str(exe)


def run(exe, *args):
    r = subprocess.run([exe, *args], capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stdout + r.stderr
    return r.stdout


def test_expf_every_argument(checker):
    out = run(checker)
    assert "mismatches 0" in out and "checked 2239889410" in out, out


def test_expf_double_double_path(checker):
    out = run(checker, "97", "slow")
    assert "mismatches 0" in out, out
