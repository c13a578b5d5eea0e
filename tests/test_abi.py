"""CPU-side checks of the C ABI: the library loads, exports every function
include/cad.h declares, and rejects bad arguments on the host before any
device work (these calls never reach the HIP runtime)."""
import ctypes
import os
import re

import pytest

cad = pytest.importorskip("verify_forward_amd")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared():
    text = open(os.path.join(ROOT, "include", "cad.h")).read()
    return sorted(set(re.findall(r"^\s*(?:cad_status|void|const char\*)\s+(cad_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    names = declared()
    assert set(names) == set(cad.EXPORTS), names


def test_library_exports_every_declared_symbol():
    L = cad.lib()
    for name in declared():
        assert hasattr(L, name), name


def good_config(**kw):
    c = cad.cad_config(2, 128, 4, 2, 64, 256, 512, 1, 10000.0, 1e-5, cad.CAD_BF16, 16)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


@pytest.mark.parametrize("field,value,status", [
    ("n_layers", 0, cad.CAD_E_ARG),
    ("vocab", -1, cad.CAD_E_ARG),
    ("dtype", 7, cad.CAD_E_ARG),
    ("n_kv_heads", 3, cad.CAD_E_ARG),
    ("head_dim", 96, cad.CAD_E_UNSUPPORTED),
    ("d_model", 100, cad.CAD_E_UNSUPPORTED),
    ("loop_depth", 0, cad.CAD_E_ARG),
    ("rope_theta", -1.0, cad.CAD_E_ARG),
])
def test_create_rejects_bad_config(field, value, status):
    c = good_config(**{field: value})
    h = ctypes.c_void_p()
    w = cad.cad_weights()
    st = cad.lib().cad_model_create(ctypes.byref(c), ctypes.byref(w), ctypes.byref(h))
    assert st == status
    assert h.value is None
    assert cad.cad_last_error() != ""


def test_create_rejects_shape_beyond_the_rotary_stage():
    """64 query and 64 KV heads of 128 (d_model 8192): the rotary kernel
    could not stage a whole row of q, k and v heads, so create refuses the
    shape up front instead of failing a later call mid-way."""
    c = good_config(d_model=8192, n_q_heads=64, n_kv_heads=64, head_dim=128)
    h = ctypes.c_void_p()
    w = cad.cad_weights()
    assert cad.lib().cad_model_create(ctypes.byref(c), ctypes.byref(w), ctypes.byref(h)) == cad.CAD_E_UNSUPPORTED
    assert h.value is None
    assert "16384" in cad.cad_last_error()


def test_create_rejects_missing_weights():
    c = good_config()
    h = ctypes.c_void_p()
    w = cad.cad_weights()
    assert cad.lib().cad_model_create(ctypes.byref(c), ctypes.byref(w), ctypes.byref(h)) == cad.CAD_E_ARG
    assert "weights" in cad.cad_last_error()


def test_looped_config_needs_single_layer():
    c = good_config(loop_depth=4)
    h = ctypes.c_void_p()
    w = cad.cad_weights()
    assert cad.lib().cad_model_create(ctypes.byref(c), ctypes.byref(w), ctypes.byref(h)) == cad.CAD_E_ARG


def test_calls_reject_null_model_and_bad_sizes():
    L = cad.lib()
    kv = cad.cad_kv()
    assert L.cad_splice_forward(None, ctypes.byref(kv), 0, None, 1, None, 0, None, None, None, None, None) == cad.CAD_E_ARG
    assert L.cad_decode_step(None, ctypes.byref(kv), 0, None, None, None, None, None, None) == cad.CAD_E_ARG
    buf = (ctypes.c_int32 * 4)()
    p = ctypes.cast(buf, ctypes.c_void_p)
    # bad n-gram bounds, K and T are caught before any launch
    assert L.cad_propose_suffix_match(p, 4, 0, 1, 4, p, p, p, None) == cad.CAD_E_ARG
    assert L.cad_propose_suffix_match(p, 4, 4, 5, 4, p, p, p, None) == cad.CAD_E_ARG
    assert L.cad_propose_suffix_match(p, 4, 65, 1, 4, p, p, p, None) == cad.CAD_E_ARG
    assert L.cad_propose_suffix_match(p, 4, 4, 1, 0, p, p, p, None) == cad.CAD_E_ARG
    assert L.cad_propose_suffix_match(p, -1, 4, 1, 4, p, p, p, None) == cad.CAD_E_ARG
    assert L.cad_propose_suffix_match(None, 4, 4, 1, 4, p, p, p, None) == cad.CAD_E_ARG
    assert L.cad_propose_suffix_match(p, 4, 4, 1, 4, None, p, p, None) == cad.CAD_E_ARG


STRUCTS = ("cad_config", "cad_weights", "cad_kv", "cad_loop_group", "cad_loop_params", "cad_loop_stats",
           "cad_program_table", "cad_program_params", "cad_program_stats")


def test_binding_structs_match_the_header(tmp_path):
    """The binding's ctypes structures have the header's size and field
    offsets (a C program built with the host compiler prints them)."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("no host C compiler")
    lines = ["#include <stddef.h>", "#include <stdio.h>", '#include "cad.h"', "int main(void) {"]
    for name in STRUCTS:
        lines.append(f'  printf("{name} size %zu\\n", sizeof({name}));')
        for f, _ in getattr(cad, name)._fields_:
            lines.append(f'  printf("{name} {f} %zu\\n", offsetof({name}, {f}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = {}
    for ln in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.splitlines():
        s, f, v = ln.split()
        got[(s, f)] = int(v)
    for name in STRUCTS:
        T = getattr(cad, name)
        assert got[(name, "size")] == ctypes.sizeof(T), name
        for f, _ in T._fields_:
            assert got[(name, f)] == getattr(T, f).offset, (name, f)


def test_binding_constants_match_the_header():
    """Every ``#define CAD_*`` number and every ``cad_status`` / ``cad_mode``
    enumerator of include/cad.h has the same value in the binding."""
    text = open(os.path.join(ROOT, "include", "cad.h")).read()
    defines = {}
    for name, expr in re.findall(r"^#define\s+(CAD_[A-Z0-9_]+)\s+(\(?-?[0-9][0-9xu <()-]*)", text, re.M):
        defines[name] = eval(expr.replace("u", ""))
    enums = {name: int(v) for name, v in re.findall(r"\b(CAD_[A-Z0-9_]+)\s*=\s*(-?\d+)", text)}
    both = {**defines, **enums}
    assert {"CAD_DEV_F16_RANGE", "CAD_KV_BLOCK", "CAD_OK", "CAD_COMMIT"} <= set(both)
    for name, value in both.items():
        assert getattr(cad, name) == value, name
