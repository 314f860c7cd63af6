"""The pins bite: plausible mistakes planted in a copy of the oracle (on the CPU) must each fail them.

Every mutation below is one exact textual change to oracle/oracle.c (a dropped term, a wrong sign, index,
rounding or constant).  The copy is built with the oracle's own flags, the oracle's pin suites run against it
in a separate process (ZERO_ORACLE_LIB), and each must fail.  An unmutated copy built the same way must pass,
so a failure is the mutation's doing.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")
PINS = ["tests/test_oracle_layout.py", "tests/test_oracle_numerics.py", "tests/test_oracle_adamw.py"]

MUTATIONS = {
    "first moment sign": ("    m_new = m_old + m_new;", "    m_new = m_old - m_new;"),
    "second bias correction dropped": ("    d = d / s.bc2_sqrt;", "    d = d;"),
    "first bias correction dropped": ("  s->step_size = (float)(hp->lr / bc1);", "  s->step_size = (float)(hp->lr);"),
    "decoupled decay dropped": ("    float p = master[i] * s.decay;", "    float p = master[i];"),
    "eps dropped": ("    d = d + s.eps;", "    d = d;"),
    "1 - beta2 swapped": ("  s->omb2 = (float)(1.0 - hp->beta2);", "  s->omb2 = (float)(hp->beta2);"),
    "unscale dropped": ("    g = g * s.gscale;", "    g = g;"),
    "square dropped": ("    double sq = g * g;", "    double sq = g;"),
    "flag ignored": ("    if ((x[i] & expmask) == expmask) flag = 1;", "    (void)expmask;"),
    "floor partition": ("  int64_t shard = psi / world + (psi % world != 0 ? 1 : 0);", "  int64_t shard = psi / world;"),
    "padding not zeroed": ("      shard[j] = 0;", "      shard[j] = 1;"),
    "ZeRO-2 ledger": ("  out->bytes_zero2 = 2 * out->padded_numel + (2 + 12) * shard;",
                      "  out->bytes_zero2 = 2 * out->padded_numel + 12 * shard;"),
    "ZeRO-3 communication": ("  out->comm_zero3 = one_collective + one_collective + one_collective;",
                             "  out->comm_zero3 = one_collective + one_collective;"),
    "clip not clamped": ("  return coef < 1.0 ? coef : 1.0;", "  return coef;"),
    "scale not halved on overflow": ("    *scale = *scale * 0.5;", "    *scale = *scale;"),
    "cosine phase": ("(1.0 + cos(M_PI * frac))", "(1.0 + cos(M_PI * frac * 0.5))"),
    "bf16 ties away from zero": ("    round_up = (int)(kept & 1u);", "    round_up = 1;"),
    "binary16 ties away from zero": ("  if (rest > 0.5 || (rest == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;",
                                     "  if (rest >= 0.5) r += 1.0;"),
    "binary16 subnormal exponent": ("  if (E < -14) E = -14;", "  if (E < -15) E = -15;"),
}


def _build(tmp, name, text):
    src = os.path.join(tmp, f"{name}.c")
    lib = os.path.join(tmp, f"lib{name}.so")
    with open(src, "w", encoding="utf-8") as f:
        f.write(text)
    subprocess.run(["sh", os.path.join(ROOT, "oracle", "build.sh"), src, lib], check=True, capture_output=True)
    return lib


def _pins_pass(lib) -> bool:
    env = dict(os.environ, ZERO_ORACLE_LIB=lib)
    res = subprocess.run([sys.executable, "-m", "pytest", *PINS, "-x", "-q", "-p", "no:cacheprovider"], cwd=ROOT,
                         env=env, capture_output=True, text=True, timeout=600)
    return res.returncode == 0


@pytest.mark.slow
def test_planted_mistakes_fail_the_pins(tmp_path):
    text = open(SRC, encoding="utf-8").read()
    libs = {"control": _build(str(tmp_path), "control", text)}
    for k, (name, (old, new)) in enumerate(MUTATIONS.items()):
        assert text.count(old) == 1, f"mutation {name!r} no longer matches the oracle source"
        libs[name] = _build(str(tmp_path), f"m{k}", text.replace(old, new))
    with ThreadPoolExecutor(max_workers=4) as ex:
        passed = dict(zip(libs, ex.map(_pins_pass, libs.values())))
    assert passed.pop("control"), "the unmutated copy must pass the pins"
    survivors = [name for name, ok in passed.items() if ok]
    assert not survivors, f"mistakes the pins do not catch: {survivors}"
