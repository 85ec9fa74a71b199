"""CPU-side checks of the C ABI: the library loads, exports every entry point the
header declares, and rejects bad arguments before touching the GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "clha.h")


def _declared():
    txt = open(HEADER).read()
    return re.findall(r"CLHA_API\s+[\w\s\*]*?\b(clha_\w+)\s*\(", txt)


def test_header_declares_the_three_phases():
    names = _declared()
    for n in ("clha_collect_hessians", "clha_aggregate", "clha_gptq_quantize", "clha_sync"):
        assert n in names


def test_library_exports_every_declared_symbol():
    import gptq_calibration_moe_amd as g
    lib = ctypes.CDLL(g.LIB_PATH)
    names = _declared()
    assert len(names) >= 15
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(g.EXPORTS)


def test_create_rejects_bad_shapes_without_a_device():
    import gptq_calibration_moe_amd as g
    h = ctypes.c_void_p()
    for desc in [(100, 8, 2, 0, 10), (256, 0, 1, 0, 10), (256, 8, 9, 0, 10), (256, 8, 0, 0, 10),
                 (256, 300, 2, 0, 10), (256, 8, 2, -1, 10), (256, 8, 2, 0, 0), (16384, 8, 2, 0, 10)]:
        st = g.lib.clha_create(ctypes.byref(g.MoeDesc(*desc)), ctypes.byref(h))
        assert st == g.ERR_SHAPE, desc
    assert g.lib.clha_create(None, ctypes.byref(h)) == g.ERR_INVALID_ARG
    assert g.lib.clha_destroy(None) == g.OK
    assert g.lib.clha_sync(None, None) == g.ERR_INVALID_ARG


def test_build_entry_compiles_for_gfx950():
    src = open(os.path.join(ROOT, "gptq_calibration_moe_amd", "build.py")).read()
    assert "gfx950" in src and "-packed-fp32-ops" in src


def test_job_struct_layout_matches_the_header(tmp_path):
    """The binding's ctypes clha_gptq_job has the C struct's size and field offsets
    (a host C program built against include/clha.h prints them)."""
    import subprocess
    import gptq_calibration_moe_amd as g
    fields = [f for f, _ in g.GptqJob._fields_]
    src = tmp_path / "layout.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "clha.h"\nint main(void) {\n'
                   '  printf("%zu\\n", sizeof(clha_gptq_job));\n'
                   + "".join(f'  printf("%zu\\n", offsetof(clha_gptq_job, {f}));\n' for f in fields)
                   + "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    out = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    assert out[0] == ctypes.sizeof(g.GptqJob)
    assert out[1:] == [getattr(g.GptqJob, f).offset for f in fields]
