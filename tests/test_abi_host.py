"""Host-side tests of the C ABI (no GPU needed, no kernel is launched).

The library must load, export every function include/rlk_logp.h declares, and
reject every host-detectable argument error with its documented status before
any HIP call is made (so these calls return without touching a device). The
pointers passed here are fake, aligned, non-null addresses that the library
never dereferences on the host.
"""
import ctypes

import pytest

import invariant_token_log_fp32_amd as rlk
from invariant_token_log_fp32_amd import VocabLayout

OK, NULL, ALIGN, SHAPE, GROUPS, WS, HIP, SCRATCH = 0, -1, -2, -3, -4, -5, -6, -7
P = 0x10000  # fake 64 KiB-aligned device address


@pytest.fixture(scope="module")
def lib():
    return rlk.load_library()


def lay(vp=1024, vr=1000, stride=None, shards=8, groups=1):
    return VocabLayout(vp, vr, stride if stride is not None else vp, shards, groups)


def full(lib, logits=P, n=4, L=None, t=P + 0x100, tg=P + 0x200, out=P + 0x300, lse=None, ws=None, wsb=0):
    L = L if L is not None else lay()
    return lib.rlk_logp_full(logits, n, ctypes.byref(L) if L is not False else None, t, tg, out, lse,
                             ws, wsb, None)


def nuc(lib, logits=P, n=4, L=None, t=P + 0x100, p=P + 0x140, k=P + 0x180, tg=P + 0x200, pol=P + 0x300,
        ref=P + 0x400, lse=None, state=None, ws=P + 0x1000, wsb=1 << 20):
    L = L if L is not None else lay()
    return lib.rlk_logp_nucleus(logits, n, ctypes.byref(L) if L is not False else None, t, p, k, tg, pol, ref,
                                lse, state, ws, wsb, None)


def bwd(lib, logits=P, n=4, L=None, t=P + 0x100, tg=P + 0x200, ref=P + 0x300, lse=P + 0x340, gr=P + 0x380,
        pol=P + 0x400, state=P + 0x500, gp=P + 0x600, out=P + 0x10000, stride=1024):
    L = L if L is not None else lay()
    return lib.rlk_logp_backward(logits, n, ctypes.byref(L) if L is not False else None, t, tg, ref, lse, gr,
                                 pol, state, gp, out, stride, None)


def test_every_declared_function_is_exported(lib):
    names = rlk.declared_functions()
    assert set(names) == {"rlk_logp_full", "rlk_logp_nucleus", "rlk_logp_workspace_bytes", "rlk_status_string",
                          "rlk_logp_shard_summaries", "rlk_logp_merge", "rlk_logp_summary_bytes",
                          "rlk_logp_backward", "rlk_l2norm", "rlk_l2norm_zero", "rlk_l2norm_accumulate",
                          "rlk_l2norm_finalize", "rlk_linear", "rlk_linear_logp", "rlk_linear_logp_workspace_bytes",
                          "rlk_linear_logp_summaries", "rlk_linear_logp_merge", "rlk_linear_logp_summary_bytes",
                          "rlk_logp_nucleus_noalloc"}
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code in (OK, NULL, ALIGN, SHAPE, GROUPS, WS, HIP):
        s = rlk.status_string(code)
        assert s and s != "unknown status"
    assert rlk.status_string(12345) == "unknown status"


def test_zero_rows_is_ok_without_launch(lib):
    assert full(lib, n=0) == OK
    assert nuc(lib, n=0, wsb=0) == OK
    assert full(lib, n=0, L=lay(groups=4), ws=P + 0x2000, wsb=0) == OK
    # empty arrays may come with NULL pointers
    assert full(lib, n=0, logits=None, t=None, tg=None, out=None) == OK
    assert nuc(lib, n=0, logits=None, p=None, k=None, ws=None, wsb=0) == OK
    # the layout is still validated
    assert full(lib, n=0, L=lay(groups=3)) == GROUPS


@pytest.mark.parametrize("kw,code", [
    (dict(logits=None), NULL), (dict(t=None), NULL), (dict(tg=None), NULL), (dict(out=None), NULL),
    (dict(L=False), NULL),
    (dict(logits=P + 2), ALIGN), (dict(logits=P + 8), ALIGN), (dict(t=P + 2), ALIGN), (dict(tg=P + 4), ALIGN),
    (dict(out=P + 1), ALIGN), (dict(lse=P + 3), ALIGN),
    (dict(n=-1), SHAPE), (dict(n=(1 << 22) + 1), SHAPE),
    (dict(L=lay(shards=4)), SHAPE), (dict(L=lay(vp=1000, vr=1000)), SHAPE), (dict(L=lay(vp=32, vr=32)), SHAPE),
    (dict(L=lay(vr=0)), SHAPE), (dict(L=lay(vr=1025)), SHAPE), (dict(L=lay(stride=1020)), SHAPE),
    (dict(L=lay(stride=1028)), SHAPE), (dict(L=lay(vp=(1 << 30) + 64, vr=10)), SHAPE),
    (dict(L=lay(groups=3)), GROUPS), (dict(L=lay(groups=16)), GROUPS), (dict(L=lay(groups=0)), GROUPS),
    (dict(L=lay(groups=2)), WS), (dict(L=lay(groups=2), ws=P + 0x2000, wsb=4 * 8 * 16 - 1), WS),
    (dict(L=lay(groups=8), ws=P + 0x2008, wsb=1 << 20), ALIGN),
    (dict(n=1 << 29, L=lay(groups=8), ws=P, wsb=1 << 40), SHAPE),
])
def test_full_rejects_bad_arguments(lib, kw, code):
    assert full(lib, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(p=None), NULL), (dict(k=None), NULL), (dict(pol=None), NULL), (dict(ref=None), NULL),
    (dict(p=P + 2), ALIGN), (dict(k=P + 1), ALIGN), (dict(pol=P + 2), ALIGN), (dict(ref=P + 2), ALIGN),
    (dict(ws=None, L=lay(groups=2)), WS), (dict(wsb=4 * 8 * 16 - 1, L=lay(groups=2)), WS),
    (dict(ws=P + 4, L=lay(groups=2)), ALIGN), (dict(logits=None), NULL),
    (dict(L=lay(groups=5)), GROUPS), (dict(n=-3), SHAPE), (dict(L=lay(vr=2000)), SHAPE),
    (dict(lse=P + 0x502), ALIGN), (dict(state=P + 0x508), ALIGN),
    (dict(L=lay(vp=1 << 24, vr=1 << 24, stride=1 << 24)), SHAPE),
    (dict(L=lay(vp=(1 << 24) + 1024, vr=(1 << 24) + 7, stride=(1 << 24) + 1024)), SHAPE),
    # the support search's limit: fewer than 2^24 - 2^20 real tokens
    (dict(L=lay(vp=15728640, vr=15728640, stride=15728640)), SHAPE),
    (dict(L=lay(vp=15728704, vr=15728641, stride=15728704)), SHAPE),
    (dict(n=0, L=lay(vp=1 << 25, vr=1 << 25, stride=1 << 25)), SHAPE),
])
def test_nucleus_rejects_bad_arguments(lib, kw, code):
    assert nuc(lib, **kw) == code


def test_nucleus_accepts_the_largest_vocabulary(lib):
    # 2^24 - 2^20 - 1 real tokens pass the checks (an empty batch enqueues nothing)
    assert nuc(lib, n=0, wsb=0, L=lay(vp=15728640, vr=15728639, stride=15728640)) == OK
    assert noalloc(lib, n=0, L=lay(vp=15728640, vr=15728639, stride=15728640)) == OK


@pytest.mark.parametrize("kw,code", [
    (dict(logits=None), NULL), (dict(t=None), NULL), (dict(tg=None), NULL), (dict(out=None), NULL),
    (dict(L=False), NULL), (dict(gr=None, gp=None), NULL),
    (dict(ref=None), NULL), (dict(lse=None), NULL), (dict(pol=None), NULL), (dict(state=None), NULL),
    (dict(logits=P + 8), ALIGN), (dict(out=P + 0x10008), ALIGN), (dict(t=P + 0x102), ALIGN),
    (dict(tg=P + 0x204), ALIGN), (dict(ref=P + 0x301), ALIGN), (dict(lse=P + 0x342), ALIGN),
    (dict(gr=P + 0x381), ALIGN), (dict(pol=P + 0x402), ALIGN), (dict(state=P + 0x508), ALIGN),
    (dict(gp=P + 0x601), ALIGN),
    (dict(stride=1016), SHAPE), (dict(stride=1028), SHAPE), (dict(n=-1), SHAPE),
    (dict(L=lay(vr=0)), SHAPE), (dict(L=lay(groups=3)), GROUPS),
    (dict(n=1 << 20, stride=1 << 44), SHAPE), (dict(n=(1 << 22) + 1), SHAPE),
])
def test_backward_rejects_bad_arguments(lib, kw, code):
    assert bwd(lib, **kw) == code


def test_backward_optional_terms_and_zero_rows(lib):
    # a term whose upstream gradient is NULL needs none of its statistics
    assert bwd(lib, n=0) == OK
    assert bwd(lib, n=0, logits=None, t=None, tg=None, ref=None, lse=None, gr=None, pol=None, state=None,
               gp=None, out=None) == OK
    assert bwd(lib, n=0, stride=1000) == SHAPE


def test_workspace_sizes(lib):
    assert rlk.workspace_bytes(8192, 152576, 151936) == 0
    for g in (2, 4, 8):
        assert rlk.workspace_bytes(8192, 152576, 151936, groups=g) == 8192 * 8 * 16
    assert rlk.workspace_bytes(8192, 152576, 151936, nucleus=True) == 0
    assert rlk.workspace_bytes(8192, 152576, 151936, groups=4, nucleus=True) == 8192 * 8 * 16
    assert rlk.workspace_bytes(-1, 152576, 151936) == 0
    assert rlk.workspace_bytes(10, 152576, 151936, groups=3) == 0
    L = lay()
    assert lib.rlk_logp_workspace_bytes(5, None, 0) == 0
    assert lib.rlk_logp_workspace_bytes(5, ctypes.byref(L), 1) == 0
    L2 = lay(groups=2)
    assert lib.rlk_logp_workspace_bytes(5, ctypes.byref(L2), 1) == 5 * 128


def test_binding_fails_loudly_without_library(tmp_path):
    import importlib
    mod = importlib.import_module("invariant_token_log_fp32_amd")
    with pytest.raises(RuntimeError, match="missing"):
        saved = mod._lib
        try:
            mod._lib = None
            mod.load_library(str(tmp_path / "nope.so"))
        finally:
            mod._lib = saved


def shard(lib, logits=P, n=4, L=None, rank=0, stride=1024, t=P + 0x100, tg=P + 0x200, out=P + 0x1000, ob=1 << 20):
    L = L if L is not None else lay()
    return lib.rlk_logp_shard_summaries(logits, n, ctypes.byref(L) if L is not False else None, rank, stride, t, tg,
                                        out, ob, None)


def merge(lib, summ=P + 0x1000, sb=1 << 20, n=4, L=None, t=P + 0x100, tg=P + 0x200, out=P + 0x300, lse=None):
    L = L if L is not None else lay()
    return lib.rlk_logp_merge(summ, sb, n, ctypes.byref(L) if L is not False else None, t, tg, out, lse, None)


def test_shard_api_zero_rows_and_sizes(lib):
    assert shard(lib, n=0, logits=None, t=None, tg=None, out=None, ob=0) == OK
    assert merge(lib, n=0, summ=None, sb=0, t=None, tg=None, out=None) == OK
    for g in (1, 2, 4, 8):
        assert rlk.summary_bytes(8192, 152576, 151936, groups=g) == 8192 * (8 // g) * 16


@pytest.mark.parametrize("kw,code", [
    (dict(logits=None), NULL), (dict(t=None), NULL), (dict(tg=None), NULL), (dict(out=None), NULL),
    (dict(L=False), NULL), (dict(logits=P + 8), ALIGN), (dict(out=P + 8), ALIGN), (dict(tg=P + 4), ALIGN),
    (dict(rank=-1), SHAPE), (dict(rank=1), SHAPE), (dict(L=lay(groups=2), rank=2), SHAPE),
    (dict(stride=1020), SHAPE), (dict(L=lay(groups=4), stride=250), SHAPE), (dict(L=lay(groups=4), stride=252), SHAPE),
    (dict(ob=4 * 8 * 16 - 1), WS), (dict(L=lay(groups=2), ob=4 * 4 * 16 - 1), WS),
    (dict(L=lay(groups=6)), GROUPS), (dict(n=-1), SHAPE),
])
def test_shard_summaries_rejects_bad_arguments(lib, kw, code):
    assert shard(lib, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(summ=None), NULL), (dict(t=None), NULL), (dict(out=None), NULL), (dict(summ=P + 8), ALIGN),
    (dict(lse=P + 2), ALIGN), (dict(sb=4 * 128 - 1), WS), (dict(L=lay(groups=3)), GROUPS), (dict(n=-2), SHAPE),
])
def test_merge_rejects_bad_arguments(lib, kw, code):
    assert merge(lib, **kw) == code


@pytest.mark.parametrize("call,code", [
    (lambda L: L.rlk_l2norm_zero(None, None), NULL),
    (lambda L: L.rlk_l2norm_zero(P + 4, None), ALIGN),
    (lambda L: L.rlk_l2norm_accumulate(P, -1, P + 0x1000, None), SHAPE),
    (lambda L: L.rlk_l2norm_accumulate(P, 1 << 39, P + 0x1000, None), SHAPE),
    (lambda L: L.rlk_l2norm_accumulate(None, 0, None, None), OK),
    (lambda L: L.rlk_l2norm_accumulate(None, 5, P + 0x1000, None), NULL),
    (lambda L: L.rlk_l2norm_accumulate(P, 5, None, None), NULL),
    (lambda L: L.rlk_l2norm_accumulate(P + 2, 5, P + 0x1000, None), ALIGN),
    (lambda L: L.rlk_l2norm_accumulate(P, 5, P + 0x1004, None), ALIGN),
    (lambda L: L.rlk_l2norm_finalize(None, P, P + 0x100, None), NULL),
    (lambda L: L.rlk_l2norm_finalize(P + 0x1000, None, None, None), NULL),
    (lambda L: L.rlk_l2norm_finalize(P + 0x1000, P + 4, None, None), ALIGN),
    (lambda L: L.rlk_l2norm_finalize(P + 0x1000, None, P + 2, None), ALIGN),
    (lambda L: L.rlk_l2norm(P, -1, P + 0x1000, P, P + 0x100, None), SHAPE),
    (lambda L: L.rlk_l2norm(P, 5, None, P, P + 0x100, None), NULL),
    (lambda L: L.rlk_l2norm(P, 5, P + 0x1000, None, None, None), NULL),
    (lambda L: L.rlk_l2norm(None, 5, P + 0x1000, P, P + 0x100, None), NULL),
    (lambda L: L.rlk_l2norm(P + 1, 5, P + 0x1000, P, P + 0x100, None), ALIGN),
    (lambda L: L.rlk_l2norm(P, 5, P + 0x1000, P + 4, None, None), ALIGN),
])
def test_l2norm_rejects_bad_arguments(lib, call, code):
    assert call(lib) == code


def lin(lib, h=P, n=4, d=128, ldh=128, w=P + 0x100000, ldw=128, L=None, out=P + 0x200000):
    L = L if L is not None else lay()
    return lib.rlk_linear(h, n, d, ldh, w, ldw, ctypes.byref(L) if L is not False else None, out, None)


def linlogp(lib, h=P, n=4, d=128, ldh=128, w=P + 0x100000, ldw=128, L=None, t=P + 0x300000, tg=P + 0x300100,
            out=P + 0x300200, lse=None, ws=P + 0x400000, wsb=1 << 20):
    L = L if L is not None else lay()
    return lib.rlk_linear_logp(h, n, d, ldh, w, ldw, ctypes.byref(L) if L is not False else None, t, tg, out, lse,
                               ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(h=None), NULL), (dict(w=None), NULL), (dict(out=None), NULL), (dict(L=False), NULL),
    (dict(d=32, ldh=32, ldw=32), SHAPE), (dict(d=100, ldh=104, ldw=104), SHAPE),
    (dict(d=65600, ldh=65600, ldw=65600), SHAPE), (dict(ldh=120), SHAPE), (dict(ldh=132), SHAPE),
    (dict(ldw=64), SHAPE), (dict(ldw=130), SHAPE), (dict(n=(1 << 22) + 1), SHAPE), (dict(n=-1), SHAPE),
    (dict(L=lay(groups=3)), GROUPS), (dict(L=lay(vp=1000, vr=1000)), SHAPE), (dict(L=lay(stride=1020)), SHAPE),
    (dict(h=P + 8), ALIGN), (dict(w=P + 0x100008), ALIGN), (dict(out=P + 0x200004), ALIGN),
    # row strides above 2^21 elements: a 256-row panel's byte offsets would not fit the buffer offsets
    (dict(ldh=(1 << 21) + 8), SHAPE), (dict(ldw=(1 << 21) + 8), SHAPE),
])
def test_linear_rejects_bad_arguments(lib, kw, code):
    assert lin(lib, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(h=None), NULL), (dict(w=None), NULL), (dict(t=None), NULL), (dict(tg=None), NULL), (dict(out=None), NULL),
    (dict(ws=None), NULL), (dict(wsb=4 * 8 * 16 - 1), WS), (dict(ws=P + 0x400008), ALIGN),
    (dict(t=P + 0x300002), ALIGN), (dict(tg=P + 0x300104), ALIGN), (dict(out=P + 0x300201), ALIGN),
    (dict(lse=P + 0x300302), ALIGN), (dict(d=96, ldh=96, ldw=96), SHAPE), (dict(L=lay(groups=6)), GROUPS),
    (dict(ldh=(1 << 21) + 8), SHAPE), (dict(ldw=(1 << 21) + 8), SHAPE),
])
def test_linear_logp_rejects_bad_arguments(lib, kw, code):
    assert linlogp(lib, **kw) == code


def test_linear_zero_rows_and_workspace_size(lib):
    assert lin(lib, n=0, h=None, w=None, out=None) == OK
    assert linlogp(lib, n=0, h=None, w=None, t=None, tg=None, out=None, ws=None, wsb=0) == OK
    L = lay(vp=152576, vr=151936)
    assert lib.rlk_linear_logp_workspace_bytes(8192, ctypes.byref(L)) == 8192 * 1192 * 16
    L2 = lay(vp=1088, vr=1000)
    assert lib.rlk_linear_logp_workspace_bytes(3, ctypes.byref(L2)) == 3 * 9 * 16
    assert lib.rlk_linear_logp_workspace_bytes(-1, ctypes.byref(L2)) == 0


def linsum(lib, h=P, n=4, d=128, ldh=128, w=P + 0x100000, ldw=128, L=None, rank=0, t=P + 0x300000,
           tg=P + 0x300100, out=P + 0x400000, ob=1 << 20):
    L = L if L is not None else lay(groups=2)
    return lib.rlk_linear_logp_summaries(h, n, d, ldh, w, ldw, ctypes.byref(L) if L is not False else None, rank, t,
                                         tg, out, ob, None)


def linmerge(lib, summ=P + 0x400000, sb=1 << 20, n=4, L=None, t=P + 0x300000, tg=P + 0x300100, out=P + 0x300200,
             lse=None):
    L = L if L is not None else lay(groups=2)
    return lib.rlk_linear_logp_merge(summ, sb, n, ctypes.byref(L) if L is not False else None, t, tg, out, lse, None)


@pytest.mark.parametrize("kw,code", [
    (dict(rank=-1), SHAPE), (dict(rank=2), SHAPE), (dict(L=lay(vp=1088, vr=1000, groups=8)), SHAPE),
    (dict(h=None), NULL), (dict(w=None), NULL), (dict(t=None), NULL), (dict(tg=None), NULL), (dict(out=None), NULL),
    (dict(out=P + 0x400008), ALIGN), (dict(w=P + 0x100004), ALIGN), (dict(ob=4 * 4 * 16 - 1), WS),
    (dict(L=lay(groups=3)), GROUPS), (dict(d=48, ldh=48, ldw=48), SHAPE),
])
def test_linear_logp_summaries_rejects_bad_arguments(lib, kw, code):
    assert linsum(lib, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(summ=None), NULL), (dict(t=None), NULL), (dict(out=None), NULL), (dict(summ=P + 0x400004), ALIGN),
    (dict(lse=P + 0x300302), ALIGN), (dict(sb=4 * 8 * 16 - 1), WS), (dict(L=lay(vp=1088, vr=1000, groups=8)), SHAPE),
])
def test_linear_logp_merge_rejects_bad_arguments(lib, kw, code):
    assert linmerge(lib, **kw) == code


def test_linear_logp_summary_sizes(lib):
    assert linsum(lib, n=0, h=None, w=None, t=None, tg=None, out=None, ob=0) == OK
    assert linmerge(lib, n=0, summ=None, sb=0, t=None, tg=None, out=None) == OK
    for g in (1, 2, 4, 8):
        L = lay(vp=152576, vr=151936, groups=g)
        assert lib.rlk_linear_logp_summary_bytes(8192, ctypes.byref(L)) == 8192 * (1192 // g) * 16
    L = lay(vp=1088, vr=1000, groups=8)
    assert lib.rlk_linear_logp_summary_bytes(8, ctypes.byref(L)) == 0


def noalloc(lib, logits=P, n=4, L=None, t=P + 0x100, p=P + 0x140, k=P + 0x180, tg=P + 0x200, pol=P + 0x300,
            ref=P + 0x400, lse=None, state=None):
    L = L if L is not None else lay()
    return lib.rlk_logp_nucleus_noalloc(logits, n, ctypes.byref(L) if L is not False else None, t, p, k, tg, pol,
                                        ref, lse, state, None)


@pytest.mark.parametrize("kw,code", [
    (dict(L=False), NULL), (dict(logits=None), NULL), (dict(pol=None), NULL), (dict(ref=None), NULL),
    (dict(logits=P + 2), ALIGN), (dict(state=P + 8), ALIGN), (dict(n=-1), SHAPE),
    (dict(L=lay(groups=3)), GROUPS), (dict(L=lay(vp=1 << 25, vr=1 << 24)), SHAPE),
    (dict(n=rlk.NOALLOC_MAX_ROWS + 1, L=lay(groups=2)), SCRATCH),
    (dict(n=rlk.NOALLOC_MAX_ROWS + 1, L=lay(groups=8)), SCRATCH),
])
def test_noalloc_rejects_bad_arguments(lib, kw, code):
    assert noalloc(lib, **kw) == code


def test_noalloc_limits_and_status(lib):
    assert noalloc(lib, n=0, L=lay(groups=4)) == OK
    assert noalloc(lib, n=0, logits=None, pol=None, ref=None) == OK
    assert "static scratch" in rlk.status_string(SCRATCH)
    assert rlk.STATUS_NAMES[SCRATCH] == "RLK_ERR_SCRATCH"
    text = open(rlk.HEADER_PATH).read()
    assert f"#define RLK_NOALLOC_MAX_ROWS {rlk.NOALLOC_MAX_ROWS}" in text
