"""The ctypes structures of the three bindings against their C headers (CPU only).

For each structure passed across a boundary -- the library's (include/zero_shard.h), the oracle's
(oracle/oracle.h) and the input generator's (synth/synth_core.h) -- a C program compiled against that header
alone prints its size and field offsets, which must equal the binding's, so no argument is silently misread.
"""
import ctypes
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def c_layout(tmp_path, header_dir, header, structs):
    lines = ["#include <stddef.h>", "#include <stdio.h>", f'#include "{header}"', "int main(void) {"]
    for cname, cls in structs.items():
        lines.append(f'  printf("{cname} %zu\\n", sizeof({cname}));')
        for field, _ in cls._fields_:
            lines.append(f'  printf("{cname}.{field} %zu\\n", offsetof({cname}, {field}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / f"layout_{header.split('.')[0]}.c"
    src.write_text("\n".join(lines) + "\n")
    exe = str(src)[:-2]
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Werror", "-I", header_dir, "-o", exe, str(src)], check=True)
    out = subprocess.run([exe], capture_output=True, text=True, check=True).stdout
    return dict(line.split() for line in out.splitlines())


def check(got, structs):
    for cname, cls in structs.items():
        assert int(got[cname]) == ctypes.sizeof(cls), cname
        for field, _ in cls._fields_:
            assert int(got[f"{cname}.{field}"]) == getattr(cls, field).offset, f"{cname}.{field}"


@pytest.fixture(autouse=True)
def _gcc():
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")


def test_library_structures(tmp_path):
    import mixed_precision_adam_amd as Z

    structs = {"zero_layout": Z.zero_layout, "zero_segment": Z.zero_segment, "zero_flat_seg": Z.zero_flat_seg,
               "zero_adamw_hparams": Z.zero_adamw_hparams, "zero_step_state": Z.zero_step_state}
    got = c_layout(tmp_path, os.path.join(ROOT, "include"), "zero_shard.h", structs)
    check(got, structs)
    assert int(got["zero_step_state"]) <= 128  # the drivers allocate 128 bytes for it


def test_oracle_structures(tmp_path):
    import oracle

    structs = {"orc_layout": oracle._Layout, "orc_segment": oracle._Segment, "orc_hparams": oracle._HParams,
               "orc_scalars": oracle._Scalars}
    check(c_layout(tmp_path, os.path.join(ROOT, "oracle"), "oracle.h", structs), structs)


def test_generator_structures(tmp_path):
    import synth

    structs = {"syn_field": synth.Field, "syn_piece": synth.Piece}
    check(c_layout(tmp_path, os.path.join(ROOT, "synth"), "synth_core.h", structs), structs)
