"""The library's fp64 -> binary16 rounding helper (used by the uint4 quantizer
for the group scale and by the dequantizer) agrees with NumPy's direct
double -> half conversion, including ties, subnormals, overflow and signed
zeros.  The helper is plain C++, so it is compiled here for the host."""
import os
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR_DIR = os.path.join(ROOT, "sparse_kv_cache_gqa_amd", "csrc", "kernels")

PROG = r"""
#include "f16_round.h"
#include <stdio.h>
int main(int argc, char **argv) {
    FILE *in = fopen(argv[1], "rb"), *out = fopen(argv[2], "wb");
    double x;
    while (fread(&x, sizeof x, 1, in) == 1) {
        uint16_t h = da::f64_to_f16_rne(x);
        fwrite(&h, sizeof h, 1, out);
    }
    fclose(in); fclose(out);
    return 0;
}
"""


def _values():
    rng = np.random.default_rng(0)
    vals = [0.0, -0.0, 1.0, -1.0, 65504.0, 65519.99, 65520.0, 70000.0, -1e9, 2.0 ** -24,
            2.0 ** -25, 2.0 ** -25 * 1.0000001, 2.0 ** -26, 3 * 2.0 ** -25, 2.0 ** -14,
            2.0 ** -14 - 2.0 ** -25, 1e-300, 5e-324, np.inf, -np.inf]
    # exact ties between neighbouring halves, and values just off them
    h = np.arange(0, 0x7C00, 7, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = (h[:-1] + h[1:]) / 2
    vals += list(mids) + list(np.nextafter(mids, np.inf)) + list(np.nextafter(mids, -np.inf))
    vals += list(rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 6, 20000))
    vals += list(rng.uniform(0, 1, 5000) / 15.0)
    return np.array(vals, dtype=np.float64)


def test_f64_to_f16_matches_numpy(tmp_path):
    cxx = shutil.which("g++") or shutil.which("c++")
    if not cxx:
        pytest.skip("no host C++ compiler")
    src = tmp_path / "t.cpp"
    src.write_text(PROG)
    exe = tmp_path / "t"
    subprocess.run([cxx, "-O2", "-std=c++17", f"-I{HDR_DIR}", str(src), "-o", str(exe)], check=True)
    x = _values()
    fin = tmp_path / "in.bin"
    fout = tmp_path / "out.bin"
    x.tofile(fin)
    subprocess.run([str(exe), str(fin), str(fout)], check=True)
    got = np.fromfile(fout, dtype=np.uint16)
    want = x.astype(np.float16).view(np.uint16)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(x[i], hex(got[i]), hex(want[i])) for i in bad[:10]]
