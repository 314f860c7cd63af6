"""Code-generation invariants of the HIP library (CPU only: compiles the source
to gfx950 assembly with the library's own flags and reads it).

* Every vector load and store of the streaming update kernels (every
  gradient and parameter format) carries the non-temporal hint: the compiler
  has been seen to drop it silently for some kernel shapes, which costs the
  update 13% of its bandwidth on MI355X.
* No scalar-cache writes of any kind, and no packed-fp32 arithmetic.
"""
import os
import re
import subprocess
import tempfile

import pytest

from mixed_precision_adam_amd import build as B

HIPCC = B.HIPCC


@pytest.fixture(scope="module")
def asm():
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "zs.s")
        flags = [f for f in B.FLAGS if f != "-fPIC"]
        subprocess.run([HIPCC, *flags, "-I", os.path.join(B.ROOT, "include"), "--cuda-device-only", "-S", "-o", out,
                        B.SRC], check=True, capture_output=True)
        return open(out).read()


def kernels(text):
    """name -> body (instruction lines) for every kernel in the assembly.  A kernel can have several exits
    (s_endpgm), so its body runs to its .Lfunc_end label."""
    out = {}
    for m in re.finditer(r"^(_Z\S*):\s*;\s*@", text, re.M):
        name = m.group(1)
        end = text.index(".Lfunc_end", m.end())
        out[name] = [l.strip() for l in text[m.end():end].splitlines() if re.match(r"\s+[a-z_]+\d*", l)]
    return out


def test_streaming_update_accesses_are_nontemporal(asm):
    ks = kernels(asm)
    update = {n: b for n, b in ks.items() if "adamw_tiled_kernel" in n or "adamw_vec_kernel" in n}
    assert len(update) == 8  # {bf16, fp16} gradients x {bf16, fp16} parameters, both state layouts
    for name, body in update.items():
        wide = [l for l in body if re.match(r"global_(load|store)_dwordx[24]\b", l)]
        assert len(wide) >= 8, name
        plain = [l for l in wide if not re.search(r"\bnt\b", l)]
        assert not plain, f"{name}: {len(plain)} wide accesses without the non-temporal hint, e.g. {plain[:2]}"


def test_flatten_uses_global_streaming_reads(asm):
    """Source reads of the vector body stream (non-temporal) when source and destination share their 16-byte
    phase: its four unrolled vectors and its remainder loop, at least five wide non-temporal loads.  The
    phase-shifted bodies read every aligned source block twice (two adjacent threads), so those loads keep the
    ordinary cache policy on purpose.  The shard is written with ordinary stores (the update reads it back
    next, which measured faster for the whole step).  No flat (generic) memory instructions."""
    ks = kernels(asm)
    flat = {n: b for n, b in ks.items() if "flatten_kernel" in n}
    assert len(flat) == 3
    for name, body in flat.items():
        assert not [l for l in body if l.startswith("flat_")], f"{name}: flat (not global) memory instructions"
        loads = [l for l in body if re.match(r"global_load_dwordx4\b", l)]
        assert sum(1 for l in loads if re.search(r"\bnt\b", l)) >= 5, name


def test_no_scalar_memory_writes_and_no_packed_fp32(asm):
    bad = re.findall(r"^\s*(s_store\w*|s_buffer_store\w*|s_atomic\w*|s_buffer_atomic\w*|s_dcache_wb\w*|"
                     r"s_scratch_store\w*|v_pk_(?:add|mul|fma)_f32)\b", asm, re.M)
    assert not bad, sorted(set(bad))
