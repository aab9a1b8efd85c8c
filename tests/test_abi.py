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
    inc = os.path.join(ROOT, "include")
    text = "".join(open(os.path.join(inc, f)).read() for f in sorted(os.listdir(inc))
                   if f.endswith(".h"))
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qsa_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for n in ("qsa_forward", "qsa_backward", "qsa_preprocess", "qsa_forward_workspace_bytes",
              "qsa_backward_workspace_bytes", "qsa_preprocess_workspace_bytes",
              "qsa_status_string", "qsa_version", "qsa_forward_noalloc",
              "qsa_forward_timed", "qsa_backward_timed", "qsa_bench_gather",
              "qsa_plan_bytes", "qsa_plan_build", "qsa_forward_planned", "qsa_backward_planned",
              "qsa_forward_planned_workspace_bytes", "qsa_backward_planned_workspace_bytes",
              "qsa_plan_tables", "qsa_forward_planned_timed", "qsa_backward_planned_timed",
              "qsa_block_plan_bytes", "qsa_block_plan_build", "qsa_block_forward",
              "qsa_block_backward", "qsa_block_forward_workspace_bytes",
              "qsa_block_backward_workspace_bytes", "qsa_doc_plan_bytes", "qsa_doc_plan_build",
              "qsa_doc_forward", "qsa_doc_backward", "qsa_doc_forward_workspace_bytes",
              "qsa_doc_backward_workspace_bytes", "qsa_select", "qsa_select_workspace_bytes",
              "qsa_select_timed"):
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
    for s in range(13):
        assert lib.qsa_status_string(s) != b"unknown status"
    assert lib.qsa_status_string(13) == b"unknown status"


def test_no_gpu_here_reports_device_error(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    d = _dims()
    a = ctypes.c_void_p(4096)
    ws = lib.qsa_forward_workspace_bytes(ctypes.byref(d))
    assert lib.qsa_forward(ctypes.byref(d), a, a, a, a, 0.0625, a, a, a, a, ws, None) == 9

def test_noalloc_validates_before_touching_the_device(lib):
    fake = ctypes.c_void_p(4096)
    args = (fake, fake, fake, fake, 0.0625, fake, fake, fake, None)
    # invalid calls: the same status as qsa_forward
    for kw, status in ((dict(D=128), 4), (dict(Hq=16), 3), (dict(B=0), 2), (dict(flags=2), 7)):
        d = _dims(**kw)
        assert lib.qsa_forward_noalloc(ctypes.byref(d), *args) == status
    d = _dims()
    assert lib.qsa_forward_noalloc(ctypes.byref(d), None, *args[1:]) == 1
    assert lib.qsa_forward_noalloc(ctypes.byref(d), *args[:4], float("nan"), *args[5:]) == 5
    # a call whose workspace exceeds the fixed scratch: the scratch error, on the host
    big = _dims(Sq=32768, Skv=32768, W=2052)
    assert lib.qsa_forward_workspace_bytes(ctypes.byref(big)) > (64 << 20)
    assert lib.qsa_forward_noalloc(ctypes.byref(big), *args) == 11
    assert b"scratch" in lib.qsa_status_string(11)
    # the workloads up to 8192 tokens (and the 4096-query shard) fit the scratch
    for kw in (dict(Sq=8192, Skv=8192, W=260), dict(B=4, Sq=4096, Skv=4096, Hq=24, Hkv=2, W=260),
               dict(Sq=4096, Skv=32768, W=1028)):
        assert lib.qsa_forward_workspace_bytes(ctypes.byref(_dims(**kw))) <= (64 << 20)


def test_plan_sizes_split_the_plain_workspaces(lib):
    """The plan holds the preprocessing of both calls; the planned calls' scratch is
    the rest. Plan and backward keep the membership bits and build the partial-tile
    key lists from them, the plain forward keeps the full key lists instead: plan +
    planned scratch is the plain backward exactly, and the plain forward with the
    bits in place of the full key lists."""
    from token_indexed_sparse_amd import qsa
    for kw in (dict(), dict(Sq=32768, Skv=32768, W=2052), dict(B=4, Sq=4096, Skv=4096, Hq=24,
                                                              Hkv=2, W=260)):
        d = _dims(**kw)
        plan = lib.qsa_plan_bytes(ctypes.byref(d))
        pf = lib.qsa_forward_planned_workspace_bytes(ctypes.byref(d))
        pb = lib.qsa_backward_planned_workspace_bytes(ctypes.byref(d))
        f, b = qsa.forward_workspace_bytes(d), qsa.backward_workspace_bytes(d)
        assert 0 < pf < f and 0 < pb < b
        assert plan + pb == b
        def r256(n):
            return -(-n // 256) * 256
        bits = r256(d.B * d.Sq * (-(-d.Skv // 128) * 4) * 4)
        keys = r256(d.B * d.Sq * d.W * 4) + r256(d.B * d.Sq * 4)
        assert plan + pf == f + bits - keys
    bad = _dims(D=128)
    for n in ("qsa_plan_bytes", "qsa_forward_planned_workspace_bytes",
              "qsa_backward_planned_workspace_bytes"):
        assert getattr(lib, n)(ctypes.byref(bad)) == 0


def _plan(**kw):
    from token_indexed_sparse_amd import qsa
    return qsa.PlanStruct(**kw)


def test_plan_build_validates_before_touching_the_device(lib):
    import torch
    fake = ctypes.c_void_p(4096)
    d = _dims()
    need = lib.qsa_plan_bytes(ctypes.byref(d))
    pl = _plan(tag=7, bytes=5)
    assert lib.qsa_plan_build(ctypes.byref(d), fake, fake, need, None, None) == 1
    for kw, status in ((dict(D=128), 4), (dict(Hq=16), 3), (dict(B=0), 2), (dict(flags=2), 7)):
        pl = _plan(tag=7)
        assert lib.qsa_plan_build(ctypes.byref(_dims(**kw)), fake, fake, need, ctypes.byref(pl),
                                  None) == status
        assert pl.tag == 0  # cleared first: a failed build leaves no usable plan
    pl = _plan()
    assert lib.qsa_plan_build(ctypes.byref(d), None, fake, need, ctypes.byref(pl), None) == 1
    assert lib.qsa_plan_build(ctypes.byref(d), ctypes.c_void_p(4098), fake, need,
                              ctypes.byref(pl), None) == 6
    assert lib.qsa_plan_build(ctypes.byref(d), fake, fake, need - 1, ctypes.byref(pl), None) == 8
    assert lib.qsa_plan_build(ctypes.byref(d), fake, None, need, ctypes.byref(pl), None) == 8
    assert lib.qsa_plan_build(ctypes.byref(d), fake, ctypes.c_void_p(4100), need,
                              ctypes.byref(pl), None) == 6
    if not torch.cuda.is_available():
        assert lib.qsa_plan_build(ctypes.byref(d), fake, fake, need, ctypes.byref(pl), None) == 9
        assert pl.tag == 0


def test_planned_calls_reject_unbuilt_or_edited_plans(lib):
    import torch
    from token_indexed_sparse_amd import qsa
    a = ctypes.c_void_p(4096)
    d = _dims()
    need = lib.qsa_plan_bytes(ctypes.byref(d))
    fws = lib.qsa_forward_planned_workspace_bytes(ctypes.byref(d))
    bws = lib.qsa_backward_planned_workspace_bytes(ctypes.byref(d))

    def fwd(pl, scale=0.0625, ws=fws):
        return lib.qsa_forward_planned(pl, a, a, a, scale, a, a, a, a, ws, None)

    def bwd(pl, scale=0.0625, ws=bws):
        return lib.qsa_backward_planned(pl, a, a, a, a, a, a, scale, a, a, a, a, ws, None)

    def tables(pl):
        return lib.qsa_plan_tables(pl, *([a] * 12), None)

    for call in (fwd, bwd, tables):
        assert call(None) == 1
        assert call(ctypes.byref(_plan())) == qsa.ERR_PLAN  # never built
        built = _plan(dims=d, mem=4096, bytes=need, device=0, tag=qsa.PLAN_TAG)
        built.bytes = need - 1  # edited: the buffer no longer fits the dims
        assert call(ctypes.byref(built)) == qsa.ERR_PLAN
        bad_dims = _plan(dims=_dims(D=128), mem=4096, bytes=need, device=0, tag=qsa.PLAN_TAG)
        assert call(ctypes.byref(bad_dims)) == 4
    ok = _plan(dims=d, mem=4096, bytes=need, device=0, tag=qsa.PLAN_TAG)
    assert fwd(ctypes.byref(ok), scale=float("nan")) == 5
    assert bwd(ctypes.byref(ok), scale=-1.0) == 5
    assert fwd(ctypes.byref(ok), ws=fws - 1) == 8
    assert bwd(ctypes.byref(ok), ws=bws - 1) == 8
    assert lib.qsa_forward_planned(ctypes.byref(ok), a, ctypes.c_void_p(4097), a, 0.0625, a, a,
                                   a, a, fws, None) == 6
    assert lib.qsa_plan_tables(ctypes.byref(ok), *([a] * 11), None, None) == 1
    assert lib.qsa_plan_tables(ctypes.byref(ok), ctypes.c_void_p(4098), *([a] * 11), None) == 6
    if not torch.cuda.is_available():
        assert fwd(ctypes.byref(ok)) == 9
        assert bwd(ctypes.byref(ok)) == 9
        assert tables(ctypes.byref(ok)) == 9


def test_block_entries_validate_before_touching_the_device(lib):
    import torch
    from token_indexed_sparse_amd import qsa
    a = ctypes.c_void_p(4096)
    bd = qsa.block_dims(300, 80)
    need_f = lib.qsa_block_forward_workspace_bytes(ctypes.byref(bd))
    need_b = lib.qsa_block_backward_workspace_bytes(ctypes.byref(bd))
    plan = lib.qsa_block_plan_bytes(ctypes.byref(bd))
    # the per-row key capacity is min(T, 4 NB): the plan equals a route plan of that width
    d = _dims(Sq=300, Skv=300, W=300)
    assert plan == lib.qsa_plan_bytes(ctypes.byref(d))
    assert lib.qsa_block_plan_bytes(ctypes.byref(qsa.block_dims(300, 20))) == \
        lib.qsa_plan_bytes(ctypes.byref(_dims(Sq=300, Skv=300, W=80)))
    assert need_f == plan + lib.qsa_forward_planned_workspace_bytes(ctypes.byref(d))
    assert need_b == plan + lib.qsa_backward_planned_workspace_bytes(ctypes.byref(d))

    def fwd(bd, meta=(a,) * 7, ws=need_f, scale=0.0625):
        return lib.qsa_block_forward(ctypes.byref(bd), a, a, a, *meta, scale, a, a, a, a, ws, None)

    def bwd(bd, meta=(a,) * 7, ws=need_b, scale=0.0625):
        return lib.qsa_block_backward(ctypes.byref(bd), a, a, a, a, a, a, *meta, scale, a, a, a, a,
                                      ws, None)

    def build(bd, meta=(a,) * 7, nbytes=plan):
        pl = qsa.PlanStruct(tag=5)
        st = lib.qsa_block_plan_build(ctypes.byref(bd), *meta, a, nbytes, ctypes.byref(pl), None)
        assert pl.tag == 0
        return st

    for call in (fwd, bwd, build):
        assert call(qsa.block_dims(300, 80, block_size=2)) == 2
        assert call(qsa.block_dims(0, 80)) == 2
        assert call(qsa.block_dims(300, 0)) == 2
        assert call(qsa.block_dims(300, 1 << 31)) == 2
        assert call(qsa.BlockDims(300, 80, 16, 1, 256, 4, 0)) == 3
        assert call(qsa.BlockDims(300, 80, 12, 1, 128, 4, 0)) == 4
        assert call(qsa.block_dims(300, 80, deterministic=True)) != 7
        assert call(qsa.BlockDims(300, 80, 12, 1, 256, 4, 2)) == 7
        for x in range(7):  # every metadata pointer is required
            meta = [a] * 7
            meta[x] = None
            assert call(bd, meta=tuple(meta)) == 1
        for x in range(1, 7):  # int32 metadata are 4-byte aligned; the uint8 bitmap is not
            meta = [a] * 7
            meta[x] = ctypes.c_void_p(4098)
            assert call(bd, meta=tuple(meta)) == 6
    assert fwd(bd, ws=need_f - 1) == 8
    assert bwd(bd, ws=need_b - 1) == 8
    assert build(bd, nbytes=plan - 1) == 8
    assert fwd(bd, scale=float("inf")) == 5
    assert lib.qsa_block_plan_build(ctypes.byref(bd), *([a] * 7), a, plan, None, None) == 1
    if not torch.cuda.is_available():
        unaligned_sel = (ctypes.c_void_p(4097),) + (a,) * 6
        assert fwd(bd, meta=unaligned_sel) == 9
        assert bwd(bd) == 9
        assert build(bd) == 9


def test_doc_entries_validate_before_touching_the_device(lib):
    import torch
    from token_indexed_sparse_amd import qsa
    a = ctypes.c_void_p(4096)

    def dd(**kw):
        base = dict(B=1, Sq=300, Skv=700, Hq=12, Hkv=1, D=256, q_global_start=400, flags=0,
                    reserved=0)
        base.update(kw)
        return qsa.DocDims(**base)

    d = dd()
    plan = lib.qsa_doc_plan_bytes(ctypes.byref(d))
    # per-row capacity min(Skv, q_global_start + Sq): a route plan of that width
    assert plan == lib.qsa_plan_bytes(ctypes.byref(_dims(Sq=300, Skv=700, W=700)))
    assert lib.qsa_doc_plan_bytes(ctypes.byref(dd(q_global_start=0))) == \
        lib.qsa_plan_bytes(ctypes.byref(_dims(Sq=300, Skv=700, W=300)))
    pf = lib.qsa_doc_forward_workspace_bytes(ctypes.byref(d))
    pb = lib.qsa_doc_backward_workspace_bytes(ctypes.byref(d))
    assert pf > plan and pb > pf

    def fwd(d, ids=(a, a), ws=pf, scale=0.0625):
        return lib.qsa_doc_forward(ctypes.byref(d), a, a, a, *ids, scale, a, a, a, a, ws, None)

    def bwd(d, ids=(a, a), ws=pb, scale=0.0625):
        return lib.qsa_doc_backward(ctypes.byref(d), a, a, a, a, a, a, *ids, scale, a, a, a, a,
                                    ws, None)

    def build(d, ids=(a, a), nbytes=plan):
        pl = qsa.PlanStruct(tag=5)
        st = lib.qsa_doc_plan_build(ctypes.byref(d), *ids, a, nbytes, ctypes.byref(pl), None)
        assert pl.tag == 0
        return st

    for call in (fwd, bwd, build):
        assert call(dd(q_global_start=-1)) == 2
        assert call(dd(Sq=0)) == 2
        assert call(dd(D=128)) == 4
        assert call(dd(Hq=16)) == 3
        assert call(dd(flags=4)) == 7
        assert call(dd(reserved=1)) == 7
        assert call(d, ids=(None, a)) == 1
        assert call(d, ids=(a, None)) == 1
        assert call(d, ids=(ctypes.c_void_p(4098), a)) == 6
    assert fwd(d, ws=pf - 1) == 8
    assert bwd(d, ws=pb - 1) == 8
    assert build(d, nbytes=plan - 1) == 8
    assert fwd(d, scale=float("nan")) == 5
    if not torch.cuda.is_available():
        assert fwd(d) == 9 and bwd(d) == 9 and build(d) == 9


def test_select_validates_before_touching_the_device(lib):
    import torch
    from token_indexed_sparse_amd import qsa
    a = ctypes.c_void_p(4096)

    def sd(**kw):
        base = dict(B=2, Sq=300, NB=80, q_offset=0, H=64, D=128, top_k=16, flags=0)
        base.update(kw)
        return qsa.SelectDims(**base)

    d = sd()
    need = lib.qsa_select_workspace_bytes(ctypes.byref(d))
    assert need == 2 * 300 * 80 * 4
    assert lib.qsa_select_workspace_bytes(ctypes.byref(sd(D=64))) == 0

    def call(d, q=a, kb=a, meta=(None, None), scale=0.5, outs=(a, a, None), ws=a, wsb=need):
        return lib.qsa_select(ctypes.byref(d), q, kb, *meta, scale, *outs, ws, wsb, None)

    assert call(sd(D=64)) == 4
    for bad in (dict(B=0), dict(Sq=0), dict(NB=0), dict(NB=32769), dict(H=0), dict(H=65),
                dict(top_k=0), dict(top_k=4097), dict(q_offset=-1),
                dict(q_offset=2 ** 31 - 300)):
        assert call(sd(**bad)) == 2, bad
    assert call(sd(flags=1)) == 7
    assert call(d, q=None) == 1 and call(d, kb=None) == 1
    assert call(d, outs=(None, None, None)) == 1
    assert call(d, scale=0.0) == 5 and call(d, scale=float("inf")) == 5
    assert call(d, q=ctypes.c_void_p(4104)) == 6
    assert call(d, outs=(a, ctypes.c_void_p(4100), None)) == 6      # routes need 16 bytes
    assert call(d, outs=(ctypes.c_void_p(4098), a, None)) == 6
    assert call(d, meta=(ctypes.c_void_p(4098), None)) == 6
    assert call(d, wsb=need - 1) == 8
    assert call(d, ws=None) == 8
    if not torch.cuda.is_available():
        assert call(d) == 9
        # a caller's scores buffer replaces the workspace
        assert call(d, outs=(a, None, a), ws=None, wsb=0) == 9
