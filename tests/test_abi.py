"""The C-ABI library loads and exports every entry point include/gdn.h declares (CPU only)."""
import os
import re
import subprocess

import pytest

from chunked_gated_delta_gdn_amd import binding as b

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for required in ["gdn_chunk_prepare", "gdn_scan", "gdn_segment_compose", "gdn_decode_step"]:
        assert required in names


def test_library_exports_every_declared_symbol():
    lib = b.library()
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    out = subprocess.run(["nm", "-D", "--defined-only", b.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    assert set(declared_functions()) <= exported


def test_binding_mirrors_the_abi_names():
    for name in declared_functions():
        if name in ("gdn_status_string", "gdn_last_error"):
            continue
        assert hasattr(b, name), name


def test_status_strings_and_version():
    lib = b.library()
    for code in range(5):
        assert lib.gdn_status_string(code).decode().startswith("GDN_")
    assert b.gdn_version() >= 100


def test_problem_struct_layout_matches_c(tmp_path):
    """The ctypes mirror of gdn_problem has the C compiler's size and offsets."""
    import ctypes
    fields = [f[0] for f in b.GdnProblem._fields_]
    src = tmp_path / "layout.c"
    src.write_text("#include <stdio.h>\n#include <stddef.h>\n#include \"gdn.h\"\nint main(void) {\n"
                   + '  printf("%zu\\n", sizeof(gdn_problem));\n'
                   + "".join(f'  printf("%zu\\n", offsetof(gdn_problem, {f}));\n' for f in fields)
                   + "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True,
                                          check=True).stdout.split()]
    assert got[0] == ctypes.sizeof(b.GdnProblem)
    assert got[1:] == [getattr(b.GdnProblem, f).offset for f in fields]


def test_probe_library_exports_its_declared_symbol():
    """The benchmark's matrix-core rate probe (include/gdn_probe.h, libgdn_probe.so)."""
    import re
    from chunked_gated_delta_gdn_amd import _build
    text = open(os.path.join(ROOT, "include", "gdn_probe.h")).read()
    declared = set(re.findall(r"\b(gdn_probe_\w+)\s*\(", text))
    assert declared == {"gdn_probe_mfma_bf16", "gdn_probe_mfma_f32"}
    if not os.path.exists(_build.PROBE_LIB):
        pytest.skip("libgdn_probe.so not built")
    out = subprocess.run(["nm", "-D", "--defined-only", _build.PROBE_LIB], capture_output=True,
                         text=True, check=True).stdout
    for name in declared:
        assert re.search(rf"\b{name}\b", out), name
