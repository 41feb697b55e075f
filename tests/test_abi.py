"""The C ABI without a GPU: the library loads, exports what include/sdm.h
declares, and rejects invalid arguments before making any HIP call."""
import ctypes
import os
import re

import pytest

import sparse_memory_linear_select_amd as sdm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x100000  # a 16-byte-aligned non-null address; validation never dereferences it


def declared_functions():
    text = open(os.path.join(ROOT, "include", "sdm.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sdm_\w+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(sdm.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = sdm.lib()
    for name in declared_functions():
        assert hasattr(L, name), name


def test_status_strings():
    L = sdm.lib()
    for code in range(5):
        assert L.sdm_status_string(code)
    assert L.sdm_status_string(99) == b"unknown status"


def _create(M0=FAKE, H=2, S=16, D=32, W=4, R=4):
    h = ctypes.c_void_p()
    st = sdm.lib().sdm_create(ctypes.c_void_p(M0) if M0 else None, H, S, D, W, R, ctypes.byref(h))
    return st, h


@pytest.mark.parametrize("kw,status", [
    (dict(M0=0), 1), (dict(M0=FAKE + 4), 1), (dict(H=0), 1), (dict(S=0), 1), (dict(D=0), 1),
    (dict(W=0), 1), (dict(R=0), 1), (dict(W=17), 1), (dict(R=17), 1),
    (dict(S=2048, W=4, R=4), 2), (dict(S=128, W=65, R=4), 2),
])
def test_create_rejects(kw, status):
    st, h = _create(**kw)
    assert st == status
    assert h.value is None
    assert sdm.lib().sdm_last_error()


def test_create_destroy_and_workspace_size():
    L = sdm.lib()
    st, h = _create()
    assert st == 0 and h.value
    n = ctypes.c_size_t()
    assert L.sdm_workspace_size(h, 2, 100, sdm.F32, sdm.AUTO, ctypes.byref(n)) == 0
    # one record per (chain, token): 4*64 + 2*64 dwords
    assert n.value >= 2 * 2 * 100 * (4 * 64 + 2 * 64) * 4
    assert L.sdm_workspace_size(h, 0, 100, sdm.F32, sdm.AUTO, ctypes.byref(n)) == 1
    assert L.sdm_workspace_size(h, 2, 0, sdm.F32, sdm.AUTO, ctypes.byref(n)) == 1
    assert L.sdm_workspace_size(h, 2, 10, 7, sdm.AUTO, ctypes.byref(n)) == 1
    assert L.sdm_workspace_size(h, 2, 10, sdm.F32, 9, ctypes.byref(n)) == 1
    assert L.sdm_workspace_size(h, 1 << 20, 1 << 20, sdm.F32, sdm.AUTO, ctypes.byref(n)) == 2
    assert L.sdm_destroy(h) == 0
    assert L.sdm_destroy(None) == 0


def _forward(h, B=1, T=8, ptrs=None, dtype=sdm.F32, variant=sdm.AUTO, flags=0, ws=1 << 20):
    p = dict(kp=FAKE, qp=FAKE, v=FAKE, alpha=FAKE, beta=FAKE, ws=FAKE, y=FAKE, M=FAKE)
    p.update(ptrs or {})
    c = lambda x: ctypes.c_void_p(x) if x else None
    return sdm.lib().sdm_forward(h, B, T, c(p["kp"]), c(p["qp"]), c(p["v"]), c(p["alpha"]),
                                 c(p["beta"]), dtype, variant, flags, c(p["ws"]), ws, c(p["y"]),
                                 c(p["M"]), None)


def test_forward_rejects_before_any_device_work():
    st, h = _create()
    assert st == 0
    try:
        for name in ("kp", "qp", "v", "alpha", "beta", "ws", "y", "M"):
            assert _forward(h, ptrs={name: 0}) == 1, name
            assert _forward(h, ptrs={name: FAKE + 8}) == 1, name
        assert _forward(None) == 1
        assert _forward(h, B=0) == 1
        assert _forward(h, T=0) == 1
        assert _forward(h, dtype=5) == 1
        assert _forward(h, variant=7) == 1
        assert _forward(h, flags=4) == 1
        assert _forward(h, ws=64) == 3  # workspace too small
        assert b"workspace" in sdm.lib().sdm_last_error()
    finally:
        sdm.lib().sdm_destroy(h)


def _forward_noalloc(h, B=1, T=8, ptrs=None, flags=0):
    p = dict(kp=FAKE, qp=FAKE, v=FAKE, alpha=FAKE, beta=FAKE, y=FAKE, M=FAKE)
    p.update(ptrs or {})
    c = lambda x: ctypes.c_void_p(x) if x else None
    return sdm.lib().sdm_forward_noalloc(h, B, T, c(p["kp"]), c(p["qp"]), c(p["v"]),
                                         c(p["alpha"]), c(p["beta"]), sdm.F32, sdm.AUTO, flags,
                                         c(p["y"]), c(p["M"]), None)


def test_forward_noalloc_rejects_before_any_device_work():
    """Invalid arguments, and calls whose scratch would exceed the static
    array, fail before the first HIP call (no device is needed to see it)."""
    st, h = _create()
    L = sdm.lib()
    try:
        for name in ("kp", "qp", "v", "alpha", "beta", "y", "M"):
            assert _forward_noalloc(h, ptrs={name: 0}) == 1, name
            assert _forward_noalloc(h, ptrs={name: FAKE + 8}) == 1, name
        assert _forward_noalloc(None) == 1
        assert _forward_noalloc(h, B=0) == 1
        assert _forward_noalloc(h, flags=4) == 1
        n = ctypes.c_size_t()
        assert L.sdm_workspace_size(h, 64, 4096, sdm.F32, sdm.AUTO, ctypes.byref(n)) == 0
        assert n.value > sdm.NOALLOC_MAX_BYTES
        assert _forward_noalloc(h, B=64, T=4096) == 2
        assert b"static scratch" in L.sdm_last_error()
    finally:
        L.sdm_destroy(h)


def test_noalloc_limit_matches_header():
    text = open(os.path.join(ROOT, "include", "sdm.h")).read()
    m = re.search(r"#define SDM_NOALLOC_MAX_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == sdm.NOALLOC_MAX_BYTES


def test_select_rejects_before_any_device_work():
    st, h = _create()
    L = sdm.lib()
    c = ctypes.c_void_p
    try:
        base = [c(FAKE)] * 6
        for k in range(6):
            args = list(base)
            args[k] = None
            assert L.sdm_select(h, 1, 4, args[0], args[1], sdm.F32, *args[2:], None) == 1
            args[k] = c(FAKE + 4)
            assert L.sdm_select(h, 1, 4, args[0], args[1], sdm.F32, *args[2:], None) == 1
        assert L.sdm_select(h, 1, 0, *base[:2], sdm.F32, *base[2:], None) == 1
        assert L.sdm_select(h, 1, 4, *base[:2], 3, *base[2:], None) == 1
    finally:
        L.sdm_destroy(h)


def test_histogram_rejects_before_any_device_work():
    st, h = _create()
    L = sdm.lib()
    c = ctypes.c_void_p
    try:
        assert L.sdm_write_histogram(h, 1, 4, None, sdm.F32, c(FAKE), None) == 1
        assert L.sdm_write_histogram(h, 1, 4, c(FAKE), sdm.F32, None, None) == 1
        assert L.sdm_write_histogram(h, 1, 4, c(FAKE + 4), sdm.F32, c(FAKE), None) == 1
        assert L.sdm_write_histogram(h, 0, 4, c(FAKE), sdm.F32, c(FAKE), None) == 1
        assert L.sdm_write_histogram(None, 1, 4, c(FAKE), sdm.F32, c(FAKE), None) == 1
    finally:
        L.sdm_destroy(h)


def test_prepare_apply_reject_before_any_device_work():
    st, h = _create()
    L = sdm.lib()
    c = ctypes.c_void_p
    try:
        ok = [c(FAKE)] * 5
        # prepare(h, B, T, kp, qp, alpha, beta, dtype, variant, flags, ws, ws_bytes, M, stream)
        assert L.sdm_prepare(h, 1, 8, *ok[:4], sdm.F32, sdm.AUTO, 0, c(FAKE), 1 << 20, None, None) == 1
        assert L.sdm_prepare(h, 1, 8, *ok[:4], sdm.F32, sdm.AUTO, 2, c(FAKE), 1 << 20, c(FAKE), None) == 1
        assert L.sdm_prepare(h, 1, 8, *ok[:4], sdm.F32, sdm.AUTO, 0, c(FAKE), 16, c(FAKE), None) == 3
        # apply(h, B, T, v, dtype, variant, ws, ws_bytes, y, M, stream)
        assert L.sdm_apply(h, 1, 8, None, sdm.F32, sdm.AUTO, c(FAKE), 1 << 20, c(FAKE), c(FAKE), None) == 1
        assert L.sdm_apply(h, 1, 8, c(FAKE), sdm.F32, sdm.AUTO, c(FAKE), 16, c(FAKE), c(FAKE), None) == 3
        assert L.sdm_apply(h, 1, 8, c(FAKE), sdm.F32, 5, c(FAKE), 1 << 20, c(FAKE), c(FAKE), None) == 1
    finally:
        L.sdm_destroy(h)


def test_python_binding_refuses_cpu_tensors():
    import torch
    with pytest.raises(sdm.SDMError):
        sdm.SDM(torch.zeros(1, 16, 4), 2, 2)


def test_bf16_state_handle():
    """sdm_create_ex takes the state type; a bfloat16 state needs the
    time-parallel schedule, which the checks report without a GPU."""
    L = sdm.lib()
    h = ctypes.c_void_p()
    assert L.sdm_create_ex(ctypes.c_void_p(FAKE), 2, 16, 32, 4, 4, 7, ctypes.byref(h)) == 1
    assert h.value is None
    assert L.sdm_create_ex(ctypes.c_void_p(FAKE), 2, 16, 32, 4, 4, sdm.BF16, ctypes.byref(h)) == 0
    n = ctypes.c_size_t()
    try:
        assert L.sdm_workspace_size(h, 2, 100, sdm.F32, sdm.TIMEPAR, ctypes.byref(n)) == 0
        ntp = n.value
        assert L.sdm_workspace_size(h, 2, 100, sdm.F32, sdm.AUTO, ctypes.byref(n)) == 0
        assert n.value == ntp  # AUTO picks the time-parallel schedule
        assert L.sdm_workspace_size(h, 2, 100, sdm.F32, sdm.SERIAL, ctypes.byref(n)) == 2
        assert b"bfloat16" in L.sdm_last_error()
    finally:
        L.sdm_destroy(h)
    # d_v % 4 != 0: no schedule can hold a bfloat16 state
    assert L.sdm_create_ex(ctypes.c_void_p(FAKE), 1, 16, 30, 4, 4, sdm.BF16, ctypes.byref(h)) == 0
    try:
        assert L.sdm_workspace_size(h, 1, 10, sdm.F32, sdm.AUTO, ctypes.byref(n)) == 2
    finally:
        L.sdm_destroy(h)
