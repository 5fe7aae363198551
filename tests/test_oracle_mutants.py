"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that
at least one pin catches each: evidence that the pins constrain every step
(representative vector, mean query, score, top-K, causal key set, page-table
indirection, GQA mapping, softmax and each backward term)."""
import os
import shutil
import subprocess

import pytest

import oracle
from oracle_pins import PINS

# (name, original text, planted mistake); each original must occur exactly once
MUTANTS = [
    ("rep divides by ps-1", "out[x] /= (double)s->ps;", "out[x] /= (double)(s->ps - 1);"),
    ("qmean interleaved groups", "for (int32_t g = h * G; g < (h + 1) * G; ++g) {",
     "for (int32_t g = h; g < s->hq; g += s->hkv) {"),
    ("qmean divides by C only", "out[x] /= (double)s->c * (double)G;", "out[x] /= (double)s->c;"),
    ("score reads head 0", "const double* b = rep + ((int64_t)n * s->hkv + h) * D;",
     "const double* b = rep + ((int64_t)n * s->hkv + 0) * D;"),
    ("ties to higher page", "return (a->page > b->page) - (a->page < b->page);",
     "return (a->page < b->page) - (a->page > b->page);"),
    ("selection not ascending", "qsort(out, (size_t)keff, sizeof(int32_t), by_int);", "(void)by_int;"),
    ("selection picks lowest", "if (a->score > b->score) return -1;\n  if (a->score < b->score) return 1;",
     "if (a->score < b->score) return -1;\n  if (a->score > b->score) return 1;"),
    ("diagonal dropped", "return (int64_t)ora_keff(s) * s->ps + t + 1;",
     "return (int64_t)ora_keff(s) * s->ps + t + (t == 0);"),
    ("page table ignored", "return pool_offset(s, page_table[page], h, row);",
     "return pool_offset(s, page, h, row);"),
    ("local chunk off by a page", "page = s->n + u / s->ps;", "page = s->n - 1 + u / s->ps;"),
    ("GQA modulo mapping", "if (g / G != h) continue;                        /* reading (e) */",
     "if (g % s->hkv != h) continue;"),
    ("LSE without max", "const double L = m + log(denom);", "const double L = log(denom) + 0.0 * m;"),
    ("no softmax scale", "sbuf[j] = sc * dot(qrow, ks->k + j * D, D);", "sbuf[j] = dot(qrow, ks->k + j * D, D);"),
    ("scale 1/D", "return s->scale > 0.0 ? s->scale : 1.0 / sqrt((double)s->d);",
     "return s->scale > 0.0 ? s->scale : 1.0 / (double)s->d;"),
    ("ds sign in dq", "const double ds = p * (dot(drow, ks.v + j * D, D) - dt[i]);",
     "const double ds = p * (dot(drow, ks.v + j * D, D) + dt[i]);"),
    ("dq uses V", "out[x] += sc * ds * ks.k[j * D + x];", "out[x] += sc * ds * ks.v[j * D + x];"),
    ("dq no scale", "out[x] += sc * ds * ks.k[j * D + x];", "out[x] += ds * ks.k[j * D + x];"),
    ("dk without Dt", "const double ds = p * (dot(drow, vj, D) - dt[i]);", "const double ds = p * dot(drow, vj, D);"),
    ("dk no scale", "if (dkj) dkj[x] += sc * ds * qrow[x];", "if (dkj) dkj[x] += ds * qrow[x];"),
    ("dv transposed operand", "if (dvj) dvj[x] += p * drow[x];", "if (dvj) dvj[x] += p * qrow[x];"),
    ("dk causal ignored", "if (jj >= visible_keys(s, t)) continue;         /* causal: u > t */", ""),
    ("Dt from dO.dO", "dt[i] = dot(drow, orow, D);", "dt[i] = dot(drow, drow, D);"),
    ("bf16 widening shift", "uint32_t bits = (uint32_t)((const uint16_t*)base)[i] << 16;",
     "uint32_t bits = (uint32_t)((const uint16_t*)base)[i] << 15;"),
]


@pytest.fixture(scope="module")
def workdir(tmp_path_factory):
    d = tmp_path_factory.mktemp("mutants")
    shutil.copy(os.path.join(oracle.HERE, "oomb_oracle.h"), d)
    return d


@pytest.mark.parametrize("name,orig,bad", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(workdir, name, orig, bad):
    src = open(oracle.SRC).read()
    assert src.count(orig) == 1, f"mutation site for '{name}' not unique/absent"
    tag = "".join(ch if ch.isalnum() else "_" for ch in name)
    csrc = workdir / f"m_{tag}.c"
    csrc.write_text(src.replace(orig, bad))
    lib = workdir / f"libm_{tag}.so"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off", "-std=c11",
                           "-I", str(workdir), str(csrc), "-o", str(lib), "-lm"])
    mutant = oracle.Oracle(str(lib))
    caught = []
    for pin_name, pin in sorted(PINS.items()):
        try:
            pin(mutant)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            caught.append(pin_name)
    assert caught, f"no pin catches planted mistake '{name}'"
