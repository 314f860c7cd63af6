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
    "second bias correction from beta1": ("  s->bc2_sqrt = (float)sqrt(bc2);", "  s->bc2_sqrt = (float)sqrt(bc1);"),
    "eps added before the bias correction": ("    d = d / s.bc2_sqrt;\n    d = d + s.eps;",
                                             "    d = d + s.eps;\n    d = d / s.bc2_sqrt;"),
    "decay applied after the Adam term": ("    float p = master[i] * s.decay;\n    p = p - u;",
                                          "    float p = master[i] - u;\n    p = p * s.decay;"),
    "first moment decays with beta2": ("    float m_old = s.b1 * m[i];", "    float m_old = s.b2 * m[i];"),
    "second moment decays with beta1": ("    float v_old = s.b2 * v[i];", "    float v_old = s.b1 * v[i];"),
    "second moment of g, not g squared": ("    float gg = g * g;", "    float gg = g;"),
    "clip epsilon dropped": ("  double coef = max_norm / (norm + 1e-6);", "  double coef = max_norm / norm;"),
    "clip on the squared norm": ("  double norm = sqrt(global_sqnorm);", "  double norm = global_sqnorm;"),
    "scale grows one step late": ("    if (*good_steps >= growth_interval) {", "    if (*good_steps > growth_interval) {"),
    "overflow keeps the good-step count": ("    *scale = *scale * 0.5;\n    *good_steps = 0;",
                                           "    *scale = *scale * 0.5;"),
    "norm unscaled by the scale, not its square": ("    double unscaled = total / (scale * scale);",
                                                   "    double unscaled = total / scale;"),
    "update factor ignores the loss scale": ("    *grad_scale = coef / scale;", "    *grad_scale = coef;"),
    "square-norm accumulated in fp32": ("    acc = acc + sq;", "    acc = (float)(acc + sq);"),
    "binary16 decode subnormal scale": ("    mag = ldexp((double)frac, -24);", "    mag = ldexp((double)frac, -25);"),
    "binary16 decode exponent bias": ("    mag = ldexp((double)(frac + 1024), e - 25);",
                                      "    mag = ldexp((double)(frac + 1024), e - 24);"),
    "bf16 NaN not kept quiet": ("    return (uint16_t)((u >> 16) | 0x0040u);", "    return (uint16_t)(u >> 16);"),
    "ZeRO-1 ledger without the full gradients": (
        "  out->bytes_zero1 = 2 * out->padded_numel + 2 * out->padded_numel + 12 * shard;",
        "  out->bytes_zero1 = 2 * out->padded_numel + 12 * shard;"),
    "valid count not clamped to the shard": ("  if (valid > shard) valid = shard;", "  (void)0;"),
    "underflowed loss scale accepted": ("  if (!flag && !isfinite(total / (scale * scale))) return ORC_ERR_INVALID;",
                                        "  (void)0;"),
    "infinite loss scale accepted": ("  if (!isfinite(scale)) return ORC_ERR_INVALID;", "  (void)0;"),
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
