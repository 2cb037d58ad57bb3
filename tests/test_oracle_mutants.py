"""Planted mistakes in a copy of the oracle must be caught by its pins.

Each mutant is one plausible slip (a tie broken the wrong way, a swapped
bit field, a dropped term, a wrong exponent bias ...) applied to a temporary
copy of oracle.c.  The copy is built with gcc and the pin suite is run
against it in a subprocess; the suite must fail.  CPU only."""
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")
HDR = os.path.join(ROOT, "oracle", "oracle.h")
PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")

MUTANTS = [
    ("ties to the higher position",
     "if (mag[q] > mag[p] || (mag[q] == mag[p] && q < p)) ++rank;\n        }\n        keep[p] = rank < 2;",
     "if (mag[q] > mag[p] || (mag[q] == mag[p] && q > p)) ++rank;\n        }\n        keep[p] = rank < 2;"),
    ("keeps the two smallest", "keep[p] = rank < 2;", "keep[p] = rank > 1;"),
    ("signed magnitude", 'mag[p] = fabs(x);                          /* int8: |-128| = 128 */', 'mag[p] = x;                          /* int8: |-128| = 128 */'),
    ("N:M signed magnitude", "mag[p] = fabs(x);\n            }\n            orc_select_nm", "mag[p] = x;\n            }\n            orc_select_nm"),
    ("index fields swapped", "(uint8_t)(pos[0] | (pos[1] << 2))", "(uint8_t)(pos[1] | (pos[0] << 2))"),
    ("group nibbles swapped", "meta[m * ldm + g / 2] |= (uint8_t)(nib << (4 * (g % 2)));",
     "meta[m * ldm + g / 2] |= (uint8_t)(nib << (4 * ((g + 1) % 2)));"),
    ("decode reads the wrong nibble", "int nib = (meta[m * ldm + g / 2] >> (4 * (g % 2))) & 0xF;",
     "int nib = (meta[m * ldm + g / 2] >> (4 * ((g + 1) % 2))) & 0xF;"),
    ("last k term dropped", "for (int64_t k = 0; k < K; ++k) {\n                        double t = rowf[k] * bt[n * K + k];",
     "for (int64_t k = 0; k + 1 < K; ++k) {\n                        double t = rowf[k] * bt[n * K + k];"),
    ("int8 product reads the wrong B column",
     "for (int64_t k = 0; k < K; ++k) acc += rowi[k] * bti[n * K + k];",
     "for (int64_t k = 0; k < K; ++k) acc += rowi[k] * bti[(N - 1 - n) * K + k];"),
    ("fp16 subnormal scale", "v = ldexp((double)f, -24);", "v = ldexp((double)f, -25);"),
    ("bf16 exponent bias", "v = ldexp((double)(128 + f), e - 134);", "v = ldexp((double)(128 + f), e - 133);"),
    ("-0 counted as a residual non-zero", "if (keep[p] || elem_f64(dt, A, m * lda + k) == 0.0) continue;",
     "if (keep[p] || (dt == ORC_I8 ? elem_f64(dt, A, m * lda + k) == 0.0 : ((const uint16_t*)A)[m * lda + k] == 0)) continue;"),
    ("last residual entry of a row dropped",
     "first entry */\n        for (int64_t j = row_ptr[m]; j < row_ptr[m + 1]; ++j) {",
     "first entry */\n        for (int64_t j = row_ptr[m]; j + 1 < row_ptr[m + 1]; ++j) {"),
    ("a gap of exactly 255 gets a filler", "static int64_t fillers_for_gap(int64_t gap) { return (gap - 1) / 255; }",
     "static int64_t fillers_for_gap(int64_t gap) { return gap / 255; }"),
    ("delta fill bridges gaps of 255", "for (; gap > 255; gap -= 255) {", "for (; gap >= 255; gap -= 255) {"),
    ("delta gaps counted from column 0", "int64_t pos = drow_ptr[m], prev = -1;", "int64_t pos = drow_ptr[m], prev = 0;"),
    ("filler carries the entry's value", "elem_zero(dt, dvals, pos);", "elem_copy(dt, dvals, pos, rvals, j);"),
    ("delta decode starts at column 0", "int64_t k = -1;                            /* delta-coded",
     "int64_t k = 0;                            /* delta-coded"),
    ("csr product skips the row's first entry", "for (int64_t j = row_ptr[m]; j < row_ptr[m + 1]; ++j) {\n                int64_t k = col[j];",
     "for (int64_t j = row_ptr[m] + 1; j < row_ptr[m + 1]; ++j) {\n                int64_t k = col[j];"),
    ("e4m3 exponent bias", "v = ldexp((double)(8 + f), e - 10);", "v = ldexp((double)(8 + f), e - 9);"),
    ("e5m2 subnormal scale", "v = ldexp((double)f, -16);", "v = ldexp((double)f, -15);"),
    ("N:M ties to the higher position",
     "if (mag[q] > mag[p] || (mag[q] == mag[p] && q < p)) ++rank;\n        }\n        keep[p] = rank < nm_n;",
     "if (mag[q] > mag[p] || (mag[q] == mag[p] && q > p)) ++rank;\n        }\n        keep[p] = rank < nm_n;"),
    ("N:M keeps one more per group", "keep[p] = rank < nm_n;", "keep[p] = rank <= nm_n;"),
    ("N:M mask bits in reversed order", "mask[m * ldmask + k / 8] |= (uint8_t)(1u << (k % 8));",
     "mask[m * ldmask + k / 8] |= (uint8_t)(1u << (7 - k % 8));"),
    ("N:M values of a group stored at the 2:4 stride", "elem_copy(dt, vals, m * ldv + g * nm_n + t++, A, m * lda + k);",
     "elem_copy(dt, vals, m * ldv + g * (nm_m / 2) + t++, A, m * lda + k);"),
    ("N:M expansion takes a group's values in reverse", "int64_t v = m * ldv + g * nm_n + t++;",
     "int64_t v = m * ldv + g * nm_n + (nm_n - 1 - t++);"),
    ("N:M accepts groups with fewer bits", "if (cnt != nm_n) { ++bad; continue; }", "if (cnt > nm_n) { ++bad; continue; }"),
    ("N:M expansion drops the sign", "rowf[k] = elem_f64(dt, vals, v);", "rowf[k] = fabs(elem_f64(dt, vals, v));"),
    ("i4 nibbles in the other order", "int nib = (((const uint8_t*)base)[i / 2] >> (4 * (i % 2))) & 0xF;",
     "int nib = (((const uint8_t*)base)[i / 2] >> (4 * (1 - i % 2))) & 0xF;"),
    ("i4 sign extended from the wrong bit", "return nib >= 8 ? nib - 16 : nib;", "return nib >= 8 ? nib - 8 : nib;"),
    ("i4 store keeps the old nibble", "*b = (uint8_t)((*b & ~(0xF << sh)) | ((v & 0xF) << sh));",
     "*b = (uint8_t)(*b | ((v & 0xF) << sh));"),
    ("complement-bitmap lanes in row-major order", "const int q = l / 16, r = l % 16;   /* lane l = 16q + r */",
     "const int q = l % 4, r = l / 4;   /* lane l = 16q + r */"),
    ("complement-bitmap slots swapped", "word |= 1u << (2 * gi + j);", "word |= 1u << (2 * gi + 1 - j);"),
    ("complement taken from one kept position only", "if (p != i0 && p != i1) c[n++] = p;",
     "if (p != i0 && n < 2) c[n++] = p;"),
    ("complement-bitmap total one short", "roff[T * S] = (int32_t)out;", "roff[T * S] = (int32_t)out - 1;"),
    ("bound accumulates signed terms",
     "bt[n * K + k];\n                        acc += t;\n                        s += fabs(t);\n                    }\n                    Cf[m * ldc + n] = acc;",
     "bt[n * K + k];\n                        acc += t;\n                        s += t;\n                    }\n                    Cf[m * ldc + n] = acc;"),
]


def _run_mutant(tmp, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation anchor not unique: %s" % name
    d = os.path.join(tmp, "m%d" % abs(hash(name)))
    os.makedirs(d)
    with open(os.path.join(d, "oracle.c"), "w") as f:
        f.write(src.replace(old, new))
    shutil.copy(HDR, d)
    lib = os.path.join(d, "liboracle.so")
    subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-fPIC", "-shared", os.path.join(d, "oracle.c"),
                    "-o", lib, "-lm"], check=True)
    env = dict(os.environ, SSG_ORACLE_LIB=lib, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", PINS],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return name, r.returncode


def test_pins_catch_every_planted_mistake(tmp_path):
    with cf.ThreadPoolExecutor(max_workers=4) as ex:
        results = list(ex.map(lambda m: _run_mutant(str(tmp_path), *m), MUTANTS))
    survivors = [name for name, rc in results if rc == 0]
    assert not survivors, "pins did not catch: %s" % survivors


def test_unmutated_copy_passes(tmp_path):
    # the harness itself must not fail a correct oracle
    name, rc = _run_mutant(str(tmp_path), "identity", "int orc_num_threads(void) {", "int orc_num_threads(void) {")
    assert rc == 0
