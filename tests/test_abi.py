"""Host-side checks of the C ABI (no GPU needed, no kernel is launched).

* libprism.so loads and exports every function include/prism.h declares.
* Every argument check runs before any HIP call and returns its status code
  with a message (pointers below are never dereferenced: validation fails
  first).
* Workspace queries are monotone in T and L.
"""
import ctypes
import os
import re

import pytest
import torch

from linear_recurrent_sequence_shortconv_amd import prism as P

# The calls below pass fake device pointers that validation must reject; they
# are never run where a GPU is visible, so a mistake in a test cannot launch a
# kernel on real memory.
pytestmark = pytest.mark.skipif(torch.cuda.is_available(),
                                reason="fake-pointer ABI checks run on hosts without a GPU")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "prism.h")

OK, E_NULL, E_SHAPE, E_UNSUP, E_ALIGN, E_WS = 0, 1, 2, 3, 4, 5


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(prism_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    L = P.lib()
    names = declared_functions()
    assert set(names) == set(P.EXPORTS), names
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    L = P.lib()
    for code, name in P.STATUS.items():
        assert L.prism_status_string(code).decode() == name


def _fwd(desc, ptrs=None, ws=None, nbytes=0):
    """Call prism_forward with fake (never dereferenced) 16-byte aligned pointers."""
    L = P.lib()
    fake = ctypes.c_void_p(0x10000)
    p = [fake] * 15 if ptrs is None else ptrs
    return L.prism_forward(ctypes.byref(desc) if desc is not None else None, *p,
                           ws if ws is not None else fake, ctypes.c_size_t(nbytes), None)


def _err():
    return P.lib().prism_last_error().decode()


def good_desc(**kw):
    d = dict(B=2, T=100, H=4, dk=64, dv=64, L=2, chunk=64, dtype=P.PRISM_BF16)
    d.update(kw)
    return P.make_desc(d["B"], d["T"], d["H"], d["dk"], d["dv"], d["L"], d["chunk"], d["dtype"])


@pytest.mark.parametrize("field,value,code", [
    ("B", 0, E_SHAPE), ("T", 0, E_SHAPE), ("H", -1, E_SHAPE),
    ("dk", 48, E_UNSUP), ("dv", 32, E_UNSUP), ("L", 9, E_UNSUP), ("L", -1, E_SHAPE),
    ("chunk", 128, E_UNSUP), ("chunk", 8, E_UNSUP), ("dtype", 7, E_UNSUP),
    ("H", (1 << 22) // 64 + 1, E_SHAPE),
])
def test_descriptor_checks(field, value, code):
    d = good_desc(**{field: value})
    n = ctypes.c_size_t(123)
    assert P.lib().prism_forward_workspace(ctypes.byref(d), ctypes.byref(n)) == code
    assert n.value == 0
    assert _err()
    assert _fwd(d) == code


def test_conv_width_and_fp32_envelope():
    d = good_desc()
    d.conv_width = 3
    assert _fwd(d) == E_UNSUP
    assert _fwd(good_desc(dtype=P.PRISM_F32, dk=128, dv=128)) == E_UNSUP
    assert _fwd(good_desc(dtype=P.PRISM_F32, dk=64, dv=64, chunk=64)) == E_UNSUP
    n = ctypes.c_size_t(0)
    d = good_desc(dtype=P.PRISM_F32, dk=64, dv=64, chunk=32)
    assert P.lib().prism_forward_workspace(ctypes.byref(d), ctypes.byref(n)) == OK and n.value > 0


def test_variant_fields():
    """activation in {GELU, identity} and conv_offset in {0, 1}; anything else
    is rejected; the strictly-past taps own one token less per backward tile,
    so the backward workspace grows, while the training buffer does not change."""
    for act, off in ((0, 0), (1, 0), (0, 1), (1, 1)):
        d = good_desc()
        d.activation, d.conv_offset = act, off
        n = ctypes.c_size_t(0)
        assert P.lib().prism_forward_workspace(ctypes.byref(d), ctypes.byref(n)) == OK
    for field, value in (("activation", 2), ("activation", -1), ("conv_offset", 2),
                         ("conv_offset", -1)):
        d = good_desc()
        setattr(d, field, value)
        assert _fwd(d) == E_UNSUP and field in _err()
    with pytest.raises(ValueError):
        P.make_desc(1, 8, 1, 16, 16, 1, 16, P.PRISM_BF16, activation="relu")
    d0, d1 = good_desc(T=4096), good_desc(T=4096)
    d1.conv_offset = 1
    assert P.backward_workspace_bytes(d1) > P.backward_workspace_bytes(d0)
    assert P.saved_bytes(d1) == P.saved_bytes(d0)


def test_null_desc_and_pointers():
    # forward pointers: q k v alpha beta Wk Wp wbeta conv S0 conv_hist cu_seqlens o ST
    # conv_hist_out
    assert _fwd(None) == E_NULL
    fake = ctypes.c_void_p(0x10000)
    for i, name in enumerate(["q", "k", "v", "alpha", "beta", "Wk", "Wp", "wbeta", "conv"]):
        p = [fake] * 15
        p[i] = None
        assert _fwd(good_desc(), p) == E_NULL, name
        assert name in _err()
    # with L = 0 the weights may be NULL (then the workspace check fails next)
    p = [fake] * 15
    p[5] = p[6] = p[7] = p[8] = None
    assert _fwd(good_desc(L=0), p, nbytes=0) == E_WS
    # output o is required; S0, conv_hist, cu_seqlens, ST and conv_hist_out are optional
    p = [fake] * 15
    p[12] = None
    assert _fwd(good_desc(), p) == E_NULL
    p = [fake] * 15
    p[9] = p[10] = p[11] = p[13] = p[14] = None
    assert _fwd(good_desc(), p, nbytes=0) == E_WS
    # the history buffers are checked for alignment like every tensor; the
    # packed-batch offsets need 4 bytes
    for i, name in ((10, "conv_hist"), (14, "conv_hist_out"), (11, "cu_seqlens")):
        p = [fake] * 15
        p[i] = ctypes.c_void_p(0x10002)
        assert _fwd(good_desc(), p) == E_ALIGN and name in _err()
    p = [fake] * 15
    p[11] = ctypes.c_void_p(0x10004)   # 4-byte aligned offsets pass
    assert _fwd(good_desc(), p, nbytes=0) == E_WS


def test_alignment_and_workspace():
    fake = ctypes.c_void_p(0x10000)
    p = [fake] * 15
    p[2] = ctypes.c_void_p(0x10008)
    assert _fwd(good_desc(), p) == E_ALIGN and "v" in _err()
    assert _fwd(good_desc(), ws=ctypes.c_void_p(0x10010), nbytes=1 << 40) == E_ALIGN
    d = good_desc()
    need = P.forward_workspace_bytes(d)
    assert _fwd(d, nbytes=need - 1) == E_WS and str(need) in _err()
    L = P.lib()
    p = [fake] * 25
    assert L.prism_backward(ctypes.byref(d), *p, fake, ctypes.c_size_t(0), None) == E_WS
    # order: q k v alpha beta Wk Wp wbeta conv S0 conv_hist cu_seqlens dO dST dq ...
    p[12] = None   # dO
    assert L.prism_backward(ctypes.byref(d), *p, fake, ctypes.c_size_t(1 << 40), None) == E_NULL
    p = [fake] * 25
    p[14] = None   # dq
    assert L.prism_backward(ctypes.byref(d), *p, fake, ctypes.c_size_t(1 << 40), None) == E_NULL
    p = [fake] * 25
    p[10] = p[11] = p[23] = p[24] = None   # conv_hist, cu_seqlens, dS0, dconv_hist are optional
    assert L.prism_backward(ctypes.byref(d), *p, fake, ctypes.c_size_t(0), None) == E_WS


def test_workspace_monotone():
    prev_f = prev_b = 0
    for T in (1, 63, 64, 65, 1000, 4096):
        d = good_desc(T=T)
        f, b = P.forward_workspace_bytes(d), P.backward_workspace_bytes(d)
        assert f >= prev_f and b >= prev_b and b > f
        prev_f, prev_b = f, b
    prev = 0
    for L in range(0, 9):
        b = P.backward_workspace_bytes(good_desc(L=L))
        assert b >= prev
        prev = b


def test_workspace_query_null_output():
    d = good_desc()
    assert P.lib().prism_forward_workspace(ctypes.byref(d), None) == E_NULL


def test_training_pair_checks():
    """prism_forward_train / prism_backward_train validate the kept buffer
    before any HIP call."""
    L = P.lib()
    d = good_desc()
    need = P.saved_bytes(d)
    assert need > 0
    fake = ctypes.c_void_p(0x10000)
    ws_ok = ctypes.c_size_t(1 << 40)
    p14 = [fake] * 15
    # saved NULL, misaligned, too small
    assert L.prism_forward_train(ctypes.byref(d), *p14, None, ctypes.c_size_t(need), fake, ws_ok,
                                 None) == E_WS
    assert "saved" in _err()
    assert L.prism_forward_train(ctypes.byref(d), *p14, ctypes.c_void_p(0x10010),
                                 ctypes.c_size_t(need), fake, ws_ok, None) == E_ALIGN
    assert L.prism_forward_train(ctypes.byref(d), *p14, fake, ctypes.c_size_t(need - 1), fake, ws_ok,
                                 None) == E_WS
    assert str(need) in _err()
    p11 = [fake] * 12   # q k v alpha beta Wk Wp wbeta conv S0 conv_hist cu_seqlens
    p13 = [fake] * 13   # dO dST dq dk dv dalpha dbeta dWk dWp dwbeta dconv dS0 dconv_hist
    assert L.prism_backward_train(ctypes.byref(d), *p11, None, ctypes.c_size_t(need), *p13, fake,
                                  ws_ok, None) == E_WS
    assert "saved" in _err()
    # the workspace check still applies
    assert L.prism_backward_train(ctypes.byref(d), *p11, fake, ctypes.c_size_t(need), *p13, fake,
                                  ctypes.c_size_t(0), None) == E_WS
    assert "workspace" in _err()
    # saved size grows with T and L
    assert P.saved_bytes(good_desc(T=4096)) > need and P.saved_bytes(good_desc(L=4)) > need


def test_step_checks():
    """prism_step: q k v alpha beta Wk Wp wbeta conv S conv_state o; S and o
    are required, conv_state is optional; checks come before any HIP call."""
    L = P.lib()
    fake = ctypes.c_void_p(0x10000)
    d = good_desc(T=1)
    need = P.step_workspace_bytes(d)
    assert need == 2 * ((2 * 4 * 2 * 64 * 2 + 255) // 256 * 256)   # pairs [B,H,L,T,D] bf16
    ws = (fake, ctypes.c_size_t(need), None)
    for i, name in ((0, "q"), (5, "Wk"), (9, "S"), (11, "o")):
        p = [fake] * 12
        p[i] = None
        assert L.prism_step(ctypes.byref(d), *p, *ws) == E_NULL and name in _err()
    p = [fake] * 12
    p[10] = ctypes.c_void_p(0x10002)
    assert L.prism_step(ctypes.byref(d), *p, *ws) == E_ALIGN and "conv_state" in _err()
    bad = good_desc(T=1, L=9)
    assert L.prism_step(ctypes.byref(bad), *([fake] * 12), *ws) == E_UNSUP
    assert L.prism_step(ctypes.byref(d), *([fake] * 12), fake, ctypes.c_size_t(need - 1),
                        None) == E_WS
    assert P.step_workspace_bytes(good_desc(T=1, L=0)) == 0


def test_train_workspaces():
    """The training pair keeps the forward intermediates in its saved buffer,
    so its workspaces are smaller than the stateless ones; the train entry
    points accept exactly their own size."""
    L = P.lib()
    d = good_desc(T=2048, dk=128, dv=128, L=3)
    f, b = P.forward_workspace_bytes(d), P.backward_workspace_bytes(d)
    ft, bt = P.forward_train_workspace_bytes(d), P.backward_train_workspace_bytes(d)
    assert 0 < ft < f and 0 < bt < b
    fake = ctypes.c_void_p(0x10000)
    need = P.saved_bytes(d)
    p15 = [fake] * 15
    assert L.prism_forward_train(ctypes.byref(d), *p15, fake, ctypes.c_size_t(need), fake,
                                 ctypes.c_size_t(ft - 1), None) == E_WS
    assert str(ft) in _err()
    p12, p13 = [fake] * 12, [fake] * 13
    assert L.prism_backward_train(ctypes.byref(d), *p12, fake, ctypes.c_size_t(need), *p13, fake,
                                  ctypes.c_size_t(bt - 1), None) == E_WS
    assert str(bt) in _err()
    n = ctypes.c_size_t(7)
    assert L.prism_forward_train_workspace(ctypes.byref(good_desc(B=0)), ctypes.byref(n)) == E_SHAPE
    assert n.value == 0
    assert L.prism_backward_train_workspace(ctypes.byref(d), None) == E_NULL


def test_packed_tokens_checked():
    """With cu_seqlens the packed row count N (packed_tokens) must be >= 0;
    without offsets the field is ignored."""
    fake = ctypes.c_void_p(0x10000)
    d = good_desc()
    d.packed_tokens = -1
    p = [fake] * 15
    assert _fwd(d, p) == E_SHAPE and "packed_tokens" in _err()
    p[11] = None                     # dense batch: the field is not used
    assert _fwd(d, p, nbytes=0) == E_WS


def test_step_noalloc_checks():
    """prism_step_noalloc validates like prism_step and refuses, before any
    HIP call, a call whose refinement pairs exceed its fixed 16 MiB array."""
    L = P.lib()
    fake = ctypes.c_void_p(0x10000)
    d = P.make_desc(4096, 1, 16, 128, 128, 8, 16, P.PRISM_BF16)
    assert P.step_workspace_bytes(d) > (16 << 20)
    assert L.prism_step_noalloc(ctypes.byref(d), *([fake] * 12), None) == E_WS
    assert "fixed device array" in _err()
    p = [fake] * 12
    p[9] = None
    assert L.prism_step_noalloc(ctypes.byref(good_desc(T=1)), *p, None) == E_NULL and "S" in _err()
    assert L.prism_step_noalloc(ctypes.byref(good_desc(T=1, L=9)), *([fake] * 12), None) == E_UNSUP
