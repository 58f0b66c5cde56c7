"""The binding's ctypes structures lay out every field where the C header
puts it: a small C program built with gcc against include/csa2.h prints each
struct's size and each field's offset, which must equal the ctypes ones."""
import ctypes
import os
import shutil
import subprocess
import tempfile

import pytest

from kv_cache_compression_csa2_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

STRUCTS = {
    "csa2_dims": B.Dims,
    "csa2_kv_cache": B.KVCache,
    "csa2_layer": B.Layer,
    "csa2_compress_args": B.CompressArgs,
    "csa2_plan_layer": B.PlanLayer,
    "csa2_trace_record": B.TraceRecord,
}


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_ctypes_structs_match_the_header():
    lines = ['#include <stddef.h>', '#include <stdio.h>', '#include "csa2.h"', "int main(void) {"]
    for cname, py in STRUCTS.items():
        lines.append(f'  printf("{cname} size %zu\\n", sizeof({cname}));')
        for field, _ in py._fields_:
            lines.append(f'  printf("{cname} {field} %zu\\n", offsetof({cname}, {field}));')
    lines += ["  return 0;", "}"]
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "layout.c"), os.path.join(d, "layout")
        with open(src, "w") as f:
            f.write("\n".join(lines) + "\n")
        subprocess.run(["gcc", "-std=c11", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), src, "-o", exe],
                       check=True, capture_output=True, text=True)
        out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout
    c = {}
    for line in out.splitlines():
        name, key, val = line.split()
        c[(name, key)] = int(val)
    for cname, py in STRUCTS.items():
        assert c[(cname, "size")] == ctypes.sizeof(py), cname
        for field, _ in py._fields_:
            assert c[(cname, field)] == getattr(py, field).offset, f"{cname}.{field}"


def _c_kind(t: str):
    t = t.replace("const", "").strip()
    if "*" in t:
        return "ptr"
    base = t.split()[0]
    return {"int": ("int", 4), "int32_t": ("int", 4), "uint32_t": ("int", 4), "int64_t": ("int", 8),
            "size_t": ("int", 8), "float": ("float", 4), "double": ("float", 8)}[base]


def _py_kind(ct):
    if ct in (ctypes.c_void_p, ctypes.c_char_p) or (isinstance(ct, type) and issubclass(ct, ctypes._Pointer)):
        return "ptr"
    if ct in (ctypes.c_float, ctypes.c_double):
        return ("float", ctypes.sizeof(ct))
    return ("int", ctypes.sizeof(ct))


def test_binding_argtypes_match_the_prototypes():
    """Every function the binding declares has the header prototype's
    parameter count, and each parameter (and the result) the same kind and
    width: pointer, integer of 4 or 8 bytes, or float."""
    import re

    with open(os.path.join(ROOT, "include", "csa2.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = "\n".join(l for l in text.splitlines() if not l.lstrip().startswith("#"))
    protos = {}
    for ret, name, params in re.findall(r"([A-Za-z_][\w\s\*]*?)\b(csa2_\w+)\s*\(([^;{}]*?)\)\s*;", text):
        plist = [] if params.strip() in ("", "void") else [p.strip() for p in params.split(",")]
        # a parameter's type is what precedes its name
        protos[name] = (ret.strip().splitlines()[-1], [re.sub(r"\b\w+\s*$", "", p).strip() or p for p in plist])
    checked = 0
    for name in B.EXPORTED:
        fn = getattr(B._lib, name)
        assert name in protos, name
        ret, ptypes = protos[name]
        if fn.argtypes is not None:
            assert len(fn.argtypes) == len(ptypes), name
            for i, (ct, t) in enumerate(zip(fn.argtypes, ptypes)):
                assert _py_kind(ct) == _c_kind(t), f"{name} parameter {i}: {t}"
        if fn.restype is not None:
            assert _py_kind(fn.restype) == _c_kind(ret), f"{name} result: {ret}"
        checked += 1
    assert checked == len(B.EXPORTED)
