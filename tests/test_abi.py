"""The C ABI library loads, exports every declared symbol and validates
arguments on the host (no GPU needed)."""
import ctypes
import os
import re

import pytest

from unstructured_sparse_feedforward_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "sffn.h")).read()
    return sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(sffn_\w+)\s*\(", src, re.M)))


def test_header_and_binding_agree():
    assert set(_declared()) == set(B.EXPORTS)


def test_library_exports_every_symbol():
    lib = B.load_library()
    for name in _declared():
        assert hasattr(lib, name), name


def test_probe_library_exports_its_header():
    src = open(os.path.join(ROOT, "include", "sffn_probe.h")).read()
    names = sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(sffn_\w+)\s*\(", src, re.M)))
    assert names == ["sffn_probe_rates"]
    lib = ctypes.CDLL(os.path.join(ROOT, "unstructured_sparse_feedforward_amd",
                                   "libsffn_probe.so"))
    for name in names:
        assert hasattr(lib, name), name


def test_status_strings():
    lib = B.load_library()
    assert lib.sffn_status_string(0) == b"SFFN_OK"
    assert lib.sffn_status_string(-4) == b"SFFN_E_CAPACITY"


def _create(**kw):
    lib = B.load_library()
    base = dict(d=2048, d_ff=5632, gated=1, tile=128, twell_cap=8, ell_cap=0,
                dtype=B.SFFN_BF16)
    base.update(kw)
    desc = B.SffnDesc(**base)
    h = ctypes.c_void_p()
    st = lib.sffn_create(ctypes.byref(desc), ctypes.byref(h))
    if h.value:
        lib.sffn_destroy(h)
    return st


@pytest.mark.parametrize("kw,expect", [
    (dict(d=0), B.SFFN_E_ARG),
    (dict(d_ff=-128), B.SFFN_E_ARG),
    (dict(gated=2), B.SFFN_E_ARG),
    (dict(dtype=7), B.SFFN_E_ARG),
    (dict(twell_cap=0), B.SFFN_E_ARG),
    (dict(ell_cap=-1), B.SFFN_E_ARG),
    (dict(dense_rows=-1), B.SFFN_E_ARG),
    (dict(store_dtype=5), B.SFFN_E_ARG),
    (dict(updown=2), B.SFFN_E_ARG),
    (dict(updown=1, dtype=B.SFFN_F32, d=256), B.SFFN_E_UNSUPPORTED),
    (dict(dense_above=-1.0), B.SFFN_E_ARG),
    (dict(store_dtype=B.SFFN_BF16, dtype=B.SFFN_F32, d=256), B.SFFN_E_UNSUPPORTED),
    (dict(tile=64), B.SFFN_E_UNSUPPORTED),
    (dict(d_ff=5600), B.SFFN_E_UNSUPPORTED),
    (dict(d_ff=65536), B.SFFN_E_UNSUPPORTED),
    (dict(twell_cap=129), B.SFFN_E_UNSUPPORTED),
    (dict(d=1000), B.SFFN_E_UNSUPPORTED),
    (dict(d=256), B.SFFN_E_UNSUPPORTED),           # bf16 needs d % 512 == 0
    (dict(d=8192), B.SFFN_E_UNSUPPORTED),
    (dict(d=768, dtype=B.SFFN_F32), B.SFFN_E_UNSUPPORTED),
])
def test_descriptor_validation(kw, expect):
    assert _create(**kw) == expect


def test_null_arguments():
    lib = B.load_library()
    h = ctypes.c_void_p()
    assert lib.sffn_create(None, ctypes.byref(h)) == B.SFFN_E_ARG
    desc = B.SffnDesc(2048, 5632, 1, 128, 8, 0, B.SFFN_BF16)
    assert lib.sffn_create(ctypes.byref(desc), None) == B.SFFN_E_ARG
    n = ctypes.c_size_t()
    assert lib.sffn_workspace_bytes(None, 1, 0, ctypes.byref(n)) == B.SFFN_E_ARG
    assert lib.sffn_forward(None, None, None, None, None, 1, None, None, 0, None, 0,
                            None) == B.SFFN_E_ARG
    assert lib.sffn_pack_twell(None, None, 1, None, None, 0, None) == B.SFFN_E_ARG
    assert lib.sffn_check(None, None) == B.SFFN_E_ARG
    assert lib.sffn_last_error(None) == b""
    lib.sffn_destroy(None)


def test_create_without_gpu_reports_hip_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    assert _create() == B.SFFN_E_HIP
