"""The C-ABI library loads, exports what include/qsa.h declares, and validates on
the host before touching a device (CPU only: no compute call needs a GPU here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    from token_indexed_sparse_amd import qsa
    if not os.path.exists(qsa.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return qsa.library()


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "qsa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qsa_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for n in ("qsa_forward", "qsa_backward", "qsa_preprocess", "qsa_forward_workspace_bytes",
              "qsa_backward_workspace_bytes", "qsa_preprocess_workspace_bytes",
              "qsa_status_string", "qsa_version"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for n in _declared_functions():
        assert hasattr(lib, n), n
    assert lib.qsa_version() >> 16 == 1


def _dims(**kw):
    from token_indexed_sparse_amd import qsa
    base = dict(B=1, Sq=256, Skv=256, Hq=12, Hkv=1, D=256, W=36, route_is_i64=0, flags=0)
    base.update(kw)
    return qsa.Dims(**base)


def test_workspace_sizes(lib):
    from token_indexed_sparse_amd import qsa
    d = _dims()
    f, b, p = (qsa.forward_workspace_bytes(d), qsa.backward_workspace_bytes(d),
               qsa.preprocess_workspace_bytes(d))
    assert f > 0 and b > f and 0 < p
    d4 = _dims(Sq=32768, Skv=32768, W=2052)
    # forward: both row key lists (all keys, partial-tile keys); the byte
    # membership table is an output of qsa_preprocess only
    f4 = qsa.forward_workspace_bytes(d4)
    assert 2 * 32768 * 2052 * 4 <= f4 < 32768 * 32768
    # backward: the dK/dV partial sums stay within their budget (4 GiB)
    b4 = qsa.backward_workspace_bytes(d4)
    assert b4 > f4 and b4 < f4 + (5 << 30)
    assert qsa.forward_workspace_bytes(_dims(D=128)) == 0
    assert qsa.forward_workspace_bytes(_dims(Hq=24, Hkv=2)) > 0


@pytest.mark.parametrize("kw,status", [
    (dict(D=128), 4), (dict(Hq=16), 3), (dict(Hq=24, Hkv=1), 3), (dict(Hkv=0, Hq=0), 3),
    (dict(B=0), 2), (dict(Sq=0), 2), (dict(Skv=0), 2), (dict(W=0), 2),
    (dict(Skv=(1 << 19) + 1), 2), (dict(route_is_i64=2), 7), (dict(flags=2), 7),
])
def test_validation_errors_before_any_launch(lib, kw, status):
    d = _dims(**kw)
    fake = ctypes.c_void_p(4096)
    st = lib.qsa_forward(ctypes.byref(d), fake, fake, fake, fake, 0.0625, fake, fake, fake, fake,
                         1 << 40, None)
    assert st == status
    st = lib.qsa_backward(ctypes.byref(d), fake, fake, fake, fake, fake, fake, fake, 0.0625, fake,
                          fake, fake, fake, 1 << 40, None)
    assert st == status


def test_pointer_scale_alignment_and_workspace_errors(lib):
    d = _dims()
    a = ctypes.c_void_p(4096)
    ws = lib.qsa_forward_workspace_bytes(ctypes.byref(d))
    call = lambda *args: lib.qsa_forward(ctypes.byref(d), *args)  # noqa: E731
    assert call(None, a, a, a, 0.0625, a, a, a, a, ws, None) == 1
    assert call(a, a, a, a, float("nan"), a, a, a, a, ws, None) == 5
    assert call(a, a, a, a, -1.0, a, a, a, a, ws, None) == 5
    assert call(a, a, a, a, 0.0, a, a, a, a, ws, None) == 5
    assert call(ctypes.c_void_p(4097), a, a, a, 0.0625, a, a, a, a, ws, None) == 6
    assert call(a, a, a, ctypes.c_void_p(4098), 0.0625, a, a, a, a, ws, None) == 6
    assert call(a, a, a, a, 0.0625, a, a, a, a, ws - 1, None) == 8
    assert call(a, a, a, a, 0.0625, a, a, a, None, ws, None) == 8
    for s in range(11):
        assert lib.qsa_status_string(s)


def test_no_gpu_here_reports_device_error(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    d = _dims()
    a = ctypes.c_void_p(4096)
    ws = lib.qsa_forward_workspace_bytes(ctypes.byref(d))
    assert lib.qsa_forward(ctypes.byref(d), a, a, a, a, 0.0625, a, a, a, a, ws, None) == 9
