"""The oracle's pins must be able to fail: plant plausible mistakes in a copy of
the oracle source (a wrong offset, a swapped nibble order, a dropped scale
bit, a wrong sign, a wrong index, a transposed operand, ...), rebuild it with
gcc in a scratch directory, and check that the pin tests reject every mutant.
CPU only; the repository's own oracle is never modified."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PIN_FILES = ["tests/test_oracle_decode.py", "tests/test_oracle_dot.py", "tests/test_oracle_embed.py",
             "tests/test_oracle_quant.py"]

MUTANTS = {
    "q4_0 offset": ("return d * (double)(q - 8);", "return d * (double)(q - 7);"),
    "q4_0 nibble order": ("int q = (e < 16) ? (qs[e] & 15) : (qs[e - 16] >> 4);",
                          "int q = (e < 16) ? (qs[e] >> 4) : (qs[e - 16] & 15);"),
    "q8_0 unsigned code": ("int q = (int)(int8_t)blk[2 + e];", "int q = (int)blk[2 + e];"),
    "q4_k min bit dropped": ("*m = s[j + 4] & 63;", "*m = s[j + 4] & 31;"),
    "q4_k scale high bits from wrong byte": ("*sc = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);",
                                             "*sc = (s[j + 4] & 15) | ((s[j] >> 6) << 4);"),
    "q4_k min sign": ("return d * (double)sc * (double)q - dmin * (double)m;",
                      "return d * (double)sc * (double)q + dmin * (double)m;"),
    "q4_k code group": ("uint8_t byte = qs[32 * (j / 2) + l];", "uint8_t byte = qs[32 * (j % 4) + l];"),
    "q4_k dmin/d swapped": ("double dmin = oracle_half_to_double(rd16(blk + 2));",
                            "double dmin = oracle_half_to_double(rd16(blk));"),
    "q6_k high-bit shift": ("int hi = (qh[32 * h + l] >> (2 * g)) & 3;", "int hi = (qh[32 * h + l] >> g) & 3;"),
    "q6_k scale index": ("return d * (double)sc[e / 16] * (double)(q - 32);",
                         "return d * (double)sc[e / 32] * (double)(q - 32);"),
    "q6_k d position": ("double d = oracle_half_to_double(rd16(blk + 208));",
                        "double d = oracle_half_to_double(rd16(blk + 192));"),
    "q5_0 offset": ("return d * (double)(q - 16);", "return d * (double)(q - 15);"),
    "q5_0 high bit of the wrong element": ("int q = lo | (int)(((qh >> e) & 1u) << 4);",
                                           "int q = lo | (int)(((qh >> (e % 16)) & 1u) << 4);"),
    "q5_k high-bit plane": ("int q = lo | (((qh[l] >> j) & 1) << 4);", "int q = lo | (((qh[l] >> (j / 2)) & 1) << 4);"),
    "q5_k qh offset": ("const uint8_t *qh = blk + 16;", "const uint8_t *qh = blk + 17;"),
    "fp16 exponent bias": ("v = ldexp((double)(1024 + f), e - 25);", "v = ldexp((double)(1024 + f), e - 24);"),
    "gemv batch index": ("double p = (double)wrow[i] * (double)x[b * k + i];",
                         "double p = (double)wrow[i] * (double)x[i];"),
    "gemv abs as sum": ("acc += p;", "acc += fabs(p);"),
    "fp16 ties away from zero": ("double m = rint(ldexp(a, 10 - E));", "double m = floor(ldexp(a, 10 - E) + 0.5);"),
    "fp16 subnormal binade": ("if (E < -14)", "if (E < -15)"),
    "fp16 overflow threshold": ("if (bits >= 0x7c00)", "if (bits >= 0x7bff)"),
    "embed invalid id reads row 0": ("memset(dst, 0, (size_t)k * sizeof(float));", "dequant_row(t, table, k, dst);"),
    "embed id order": ("int64_t id = ids[i];", "int64_t id = ids[seq - 1 - i];"),
    "q8_0 encode ties to even": ("blk[2 + i] = (uint8_t)(int8_t)(int)roundf(v);",
                                 "blk[2 + i] = (uint8_t)(int8_t)(int)rintf(v);"),
    "q8_0 encode scale 1/128": ("float d = amax / 127.0f;", "float d = amax / 128.0f;"),
    "q4_0 encode offset 8": ("float u = v + 8.5f;", "float u = v + 8.0f;"),
    "q4_0 encode last max wins": ("if (fabsf(x[i]) > amax) {", "if (fabsf(x[i]) >= amax) {"),
    "q4_0 encode no clamp": ("q[i] = c < 15 ? c : 15;", "q[i] = c;"),
    "q4_0 encode nibble pairing": ("blk[2 + i] = (uint8_t)(q[i] | (q[i + 16] << 4));",
                                   "blk[2 + i] = (uint8_t)(q[2 * i] | (q[2 * i + 1] << 4));"),
    "gemm row index": ("double p = oracle_half_to_double(x[mm * k + i]) * (double)wrow[i];",
                       "double p = oracle_half_to_double(x[ii * k + i]) * (double)wrow[i];"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(name, tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    old, new = MUTANTS[name]
    src = open(os.path.join(ROOT, "oracle", "qmm_oracle.c")).read()
    assert src.count(old) >= 1, "mutation site vanished: " + name
    root = tmp_path / "mut"
    (root / "oracle").mkdir(parents=True)
    shutil.copy(os.path.join(ROOT, "oracle", "__init__.py"), root / "oracle" / "__init__.py")
    (root / "oracle" / "qmm_oracle.c").write_text(src.replace(old, new))
    os.symlink(os.path.join(ROOT, "tests"), root / "tests")
    os.symlink(os.path.join(ROOT, "qmm_inputs"), root / "qmm_inputs")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "--rootdir", str(root), *PIN_FILES],
                       cwd=root, capture_output=True, text=True, timeout=600)
    assert r.returncode == 1 and "failed" in r.stdout, (name, r.stdout[-2000:], r.stderr[-2000:])
