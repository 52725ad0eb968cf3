"""The ctypes binding against the public header, with no GPU: every C entry
point's parameter list and return type, the enum values, LA_MAX_HEADS and the
la_norm struct layout.  A mismatch here would pass wrong arguments silently
(ctypes converts whatever it is told to)."""

import ctypes
import os
import re

import pytest

from linear_attention_la_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header():
    src = open(os.path.join(ROOT, "include", "la.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return re.sub(r"//[^\n]*", "", src)


def _prototypes():
    protos = {}
    for m in re.finditer(r"\b(la_status|const\s+char\s*\*)\s*(la_\w+)\s*\(([^)]*)\)\s*;",
                         _header()):
        params = [p.strip() for p in m.group(3).split(",")]
        if params == ["void"]:
            params = []
        protos[m.group(2)] = (m.group(1), params)
    return protos


def _c_type(param):
    """The C type of one declared parameter, without its name and const."""
    t = re.sub(r"\bconst\b", "", param)
    t = re.sub(r"\b\w+\s*$", "", t) if not t.strip().endswith("*") else t
    return re.sub(r"\s+", "", t)


# What each C type of the header must be bound as.
_SCALARS = {
    "int32_t": ctypes.c_int32,
    "int64_t": ctypes.c_int64,
    "size_t": ctypes.c_size_t,
    "float": ctypes.c_float,
    # la_status and la_dtype have int32_t as their base type
    "la_dtype": ctypes.c_int32,
    "la_status": ctypes.c_int32,
}


def _compatible(c_type, ct):
    if c_type.endswith("*"):
        pointee = c_type[:-1]
        if ct is ctypes.c_void_p:
            return True
        if pointee in ("la_norm",):
            return ct is ctypes.POINTER(B.LaNorm)
        if pointee in _SCALARS:
            return ct is ctypes.POINTER(_SCALARS[pointee])
        return False
    want = _SCALARS.get(c_type)
    if want is None or ct is None:
        return False
    if want is ctypes.c_float or ct in (ctypes.c_float, ctypes.c_double):
        return ct is want
    # integers: same width and signedness (c_int and c_int32 are one type here)
    return ctypes.sizeof(ct) == ctypes.sizeof(want) and (ct(-1).value < 0) == (want(-1).value < 0)


def test_header_has_every_bound_function():
    protos = _prototypes()
    assert len(protos) >= 17
    lib = B.lib()
    for name in protos:
        assert getattr(lib, name).argtypes is not None or name == "la_last_error", name


@pytest.mark.parametrize("name", sorted(_prototypes()))
def test_argtypes_match_header(name):
    ret, params = _prototypes()[name]
    fn = getattr(B.lib(), name)
    argtypes = list(fn.argtypes or [])
    assert len(argtypes) == len(params), (name, len(argtypes), params)
    for i, (p, ct) in enumerate(zip(params, argtypes)):
        assert _compatible(_c_type(p), ct), f"{name} parameter {i} '{p}' bound as {ct}"
    if ret.replace(" ", "") == "constchar*":
        assert fn.restype is ctypes.c_char_p, name
    else:
        assert fn.restype in (ctypes.c_int, ctypes.c_int32), name


def test_enum_values_and_limits():
    src = _header()
    vals = dict((k, int(v)) for k, v in re.findall(r"\b(LA_[A-Z0-9_]+)\s*=\s*(\d+)", src))
    assert vals["LA_OK"] == B.LA_OK
    assert vals["LA_ERR_INVALID_ARG"] == B.LA_ERR_INVALID_ARG
    assert vals["LA_ERR_UNSUPPORTED"] == B.LA_ERR_UNSUPPORTED
    assert vals["LA_ERR_HIP"] == B.LA_ERR_HIP
    assert vals["LA_BF16"] == B.LA_BF16
    assert vals["LA_FP32"] == B.LA_FP32
    m = re.search(r"#define\s+LA_MAX_HEADS\s+(\d+)", src)
    assert m and int(m.group(1)) == B.LA_MAX_HEADS


def test_la_norm_layout():
    m = re.search(r"typedef\s+struct\s+la_norm\s*\{([^}]*)\}\s*la_norm\s*;", _header())
    assert m
    fields = [f.strip() for f in m.group(1).split(";") if f.strip()]
    names = [re.findall(r"(\w+)\s*$", f)[0] for f in fields]
    assert names == [n for n, _ in B.LaNorm._fields_]
    for f, (_, ct) in zip(fields, B.LaNorm._fields_):
        t = _c_type(f)
        if t.endswith("*"):
            assert ct is ctypes.c_void_p, f
        else:
            assert ct is _SCALARS[t], f
    # pointer, float, pointer: 8 + 4 (+4 padding) + 8 on LP64
    assert ctypes.sizeof(B.LaNorm) == 24
    assert B.LaNorm.gate.offset == 16
