"""Thin ctypes binding of libprism.so (the C ABI in include/prism.h).

Argument marshalling only: every step of the layer runs in the HIP kernels
behind the C ABI.  PyTorch provides device memory (outputs, workspace) and
the current stream.  There is no fallback: if the library is missing or a
call fails, a RuntimeError is raised.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libprism.so")

PRISM_F32 = 0
PRISM_BF16 = 1
STATUS = {0: "PRISM_OK", 1: "PRISM_ERR_NULL", 2: "PRISM_ERR_SHAPE", 3: "PRISM_ERR_UNSUPPORTED",
          4: "PRISM_ERR_ALIGN", 5: "PRISM_ERR_WORKSPACE", 6: "PRISM_ERR_HIP"}

EXPORTS = ("prism_forward_workspace", "prism_backward_workspace",
           "prism_forward_train_workspace", "prism_backward_train_workspace", "prism_forward",
           "prism_backward", "prism_saved_bytes", "prism_forward_train", "prism_backward_train",
           "prism_step_workspace", "prism_step", "prism_step_noalloc", "prism_status_string", "prism_last_error", "prism_timing_begin",
           "prism_timing_end")


class Desc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("T", ctypes.c_int), ("H", ctypes.c_int),
                ("dk", ctypes.c_int), ("dv", ctypes.c_int), ("L", ctypes.c_int),
                ("chunk", ctypes.c_int), ("conv_width", ctypes.c_int), ("dtype", ctypes.c_int),
                ("activation", ctypes.c_int), ("conv_offset", ctypes.c_int),
                ("packed_tokens", ctypes.c_int)]


_lib = None
_P = ctypes.c_void_p


def lib():
    """Load libprism.so once.  torch is imported first so that its HIP runtime
    (same SONAME as the system one) is the single runtime in the process."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run "
                               "`python -m linear_recurrent_sequence_shortconv_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.prism_forward_workspace.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(ctypes.c_size_t)]
        L.prism_backward_workspace.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(ctypes.c_size_t)]
        L.prism_forward_train_workspace.argtypes = [ctypes.POINTER(Desc),
                                                    ctypes.POINTER(ctypes.c_size_t)]
        L.prism_backward_train_workspace.argtypes = [ctypes.POINTER(Desc),
                                                     ctypes.POINTER(ctypes.c_size_t)]
        # inputs q..conv, S0, conv_hist, cu_seqlens (12); forward outputs o, ST,
        # conv_hist_out (3); backward: dO, dST, then 11 gradients (dq..dconv, dS0, dconv_hist)
        L.prism_forward.argtypes = [ctypes.POINTER(Desc)] + [_P] * 15 + [_P, ctypes.c_size_t, _P]
        L.prism_backward.argtypes = [ctypes.POINTER(Desc)] + [_P] * 25 + [_P, ctypes.c_size_t, _P]
        L.prism_saved_bytes.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(ctypes.c_size_t)]
        L.prism_forward_train.argtypes = ([ctypes.POINTER(Desc)] + [_P] * 15
                                          + [_P, ctypes.c_size_t, _P, ctypes.c_size_t, _P])
        L.prism_backward_train.argtypes = ([ctypes.POINTER(Desc)] + [_P] * 12 + [_P, ctypes.c_size_t]
                                           + [_P] * 13 + [_P, ctypes.c_size_t, _P])
        L.prism_step_workspace.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(ctypes.c_size_t)]
        L.prism_step.argtypes = [ctypes.POINTER(Desc)] + [_P] * 12 + [_P, ctypes.c_size_t, _P]
        L.prism_step_noalloc.argtypes = [ctypes.POINTER(Desc)] + [_P] * 12 + [_P]
        for f in ("prism_forward_workspace", "prism_backward_workspace",
                  "prism_forward_train_workspace", "prism_backward_train_workspace", "prism_forward",
                  "prism_backward", "prism_saved_bytes", "prism_forward_train",
                  "prism_backward_train", "prism_step_workspace", "prism_step",
                  "prism_step_noalloc"):
            getattr(L, f).restype = ctypes.c_int
        L.prism_status_string.argtypes = [ctypes.c_int]
        L.prism_status_string.restype = ctypes.c_char_p
        L.prism_last_error.restype = ctypes.c_char_p
        L.prism_timing_end.argtypes = [ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_double),
                                       ctypes.POINTER(ctypes.c_int), ctypes.c_int]
        L.prism_timing_end.restype = ctypes.c_int
        _lib = L
    return _lib


ACTIVATIONS = {"gelu": 0, "identity": 1}


def make_desc(B, T, H, dk, dv, L, chunk, dtype, conv_width=4, activation="gelu", conv_offset=0,
              packed_tokens=0):
    if activation not in ACTIVATIONS:
        raise ValueError(f"activation must be one of {sorted(ACTIVATIONS)}, got {activation!r}")
    return Desc(B, T, H, dk, dv, L, chunk, conv_width, dtype, ACTIVATIONS[activation],
                int(conv_offset), int(packed_tokens))


def _check(status):
    if status != 0:
        msg = lib().prism_last_error().decode()
        raise RuntimeError(f"{STATUS.get(status, status)}: {msg}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return PRISM_BF16
    if t.dtype == torch.float32:
        return PRISM_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _req(t, name, dtype, device):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name}: expected device {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _desc_from(q, v, Wk, chunk, activation="gelu", conv_offset=0, cu_seqlens=None,
               max_seqlen=None):
    """Descriptor of a dense batch (q [B,T,H,dk]) or, with cu_seqlens, of a
    packed one (q [N,H,dk], B = len(cu_seqlens) - 1, T = max_seqlen, N rows)."""
    N = 0
    if cu_seqlens is None:
        if q.dim() != 4:
            raise ValueError(f"q: expected [B, T, H, dk], got shape {tuple(q.shape)}")
        B, T, H, dk = q.shape
    else:
        if max_seqlen is None:
            raise ValueError("max_seqlen is required with cu_seqlens")
        N, H, dk = q.shape
        B, T = cu_seqlens.numel() - 1, int(max_seqlen)
    dv = v.shape[-1]
    L = 0 if Wk is None else Wk.shape[1]
    return make_desc(B, T, H, dk, dv, L, chunk, _dtype_code(q), activation=activation,
                     conv_offset=conv_offset, packed_tokens=N)


def _shape(t, name, shape):
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")


def _check_shapes(desc, packed, k, v, alpha, beta, Wk, Wp, wbeta, conv, S0, extra=(),
                  state_name="S0"):
    """Every tensor's shape against the descriptor, on the host, before the
    library sees a pointer: the C ABI cannot see shapes, and a wrong one
    would make the kernels read or write outside the tensor."""
    B, T, H, d, L = desc.B, desc.T, desc.H, desc.dk, desc.L
    tok = (desc.packed_tokens, H) if packed else (B, T, H)
    _shape(k, "k", tok + (d,))
    _shape(v, "v", tok + (d,))
    _shape(alpha, "alpha", tok)
    _shape(beta, "beta", tok)
    if L > 0:
        _shape(Wk, "Wk", (H, L, d, d))
        _shape(Wp, "Wp", (H, L, d, d))
        _shape(wbeta, "wbeta", (H, L, d))
        _shape(conv, "conv", (H, d, 4))
    _shape(S0, state_name, (B, H, d, d))
    for name, t, kind in extra:
        _shape(t, name, tok + (d,) if kind == "tok" else (B, H, d, d))


def _on_gpu(q):
    if q.device.type != "cuda":
        raise ValueError(f"tensors must be on a GPU device, got {q.device}")


def _req_cu(cu, q):
    if cu is None:
        return
    if cu.dtype != torch.int32 or cu.device != q.device or not cu.is_contiguous() or cu.dim() != 1:
        raise ValueError("cu_seqlens must be a contiguous 1-D int32 tensor on q's device")
    if q.dim() != 3:
        raise ValueError("with cu_seqlens, q, k, v are packed [N, H, d]")


def _workspace(nbytes, device):
    ws = torch.empty(max(int(nbytes), 256) + 256, dtype=torch.uint8, device=device)
    off = (-ws.data_ptr()) % 256
    return ws, ws[off:]


def forward_workspace_bytes(desc):
    n = ctypes.c_size_t(0)
    _check(lib().prism_forward_workspace(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def backward_workspace_bytes(desc):
    n = ctypes.c_size_t(0)
    _check(lib().prism_backward_workspace(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def forward_train_workspace_bytes(desc):
    n = ctypes.c_size_t(0)
    _check(lib().prism_forward_train_workspace(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def backward_train_workspace_bytes(desc):
    n = ctypes.c_size_t(0)
    _check(lib().prism_backward_train_workspace(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def saved_bytes(desc):
    n = ctypes.c_size_t(0)
    _check(lib().prism_saved_bytes(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def _validate_inputs(q, k, v, alpha, beta, Wk, Wp, wbeta, conv, S0):
    dev, dt = q.device, q.dtype
    for name, t in (("q", q), ("k", k), ("v", v)):
        _req(t, name, dt, dev)
    for name, t in (("alpha", alpha), ("beta", beta)):
        _req(t, name, torch.float32, dev)
    if Wk is not None:
        for name, t in (("Wk", Wk), ("Wp", Wp), ("wbeta", wbeta), ("conv", conv)):
            if t is None:
                raise ValueError(f"{name} is required when Wk is given")
            _req(t, name, dt, dev)
    if S0 is not None:
        _req(S0, "S0", torch.float32, dev)


def _req_hist(h, name, q, v, B=None):
    B = v.shape[0] if B is None else B
    H = v.shape[-2]
    _req(h, name, q.dtype, q.device)
    if tuple(h.shape) != (B, 4, H, v.shape[-1]):
        raise ValueError(f"{name}: expected shape {(B, 4, H, v.shape[-1])}, got {tuple(h.shape)}")


def forward(q, k, v, alpha, beta, Wk=None, Wp=None, wbeta=None, conv=None, S0=None, chunk=64,
            workspace=None, saved=None, activation="gelu", conv_offset=0, conv_hist=None,
            conv_hist_out=None, cu_seqlens=None, max_seqlen=None):
    """PRISM layer forward.  Returns (o, S_T).

    q, k [B,T,H,dk], v [B,T,H,dv] (bf16 or fp32); alpha, beta [B,T,H] fp32;
    Wk [H,L,dk,dv], Wp [H,L,dv,dv], wbeta [H,L,dv], conv [H,dv,4] in q's
    dtype (all None for L = 0); S0 [B,H,dv,dk] fp32 or None.
    activation: "gelu" (delta = GELU(p r)) or "identity" (delta = p r);
    conv_offset: 0 (tap j on v_{t-j}) or 1 (tap j on v_{t-1-j}).
    conv_hist [B,4,H,dv] (v's dtype): the four values of v before the
    sequence (None: zeros); conv_hist_out (same shape, may be conv_hist)
    receives them for the next call.  cu_seqlens (int32 [B+1] on the device)
    with max_seqlen packs B sequences of different lengths: q, k, v are then
    [N, H, d], alpha, beta [N, H].
    With `saved` (a buffer from saved_buffer()) this is the training forward
    (prism_forward_train): the buffer then holds what backward(saved=...)
    needs.
    """
    _validate_inputs(q, k, v, alpha, beta, Wk, Wp, wbeta, conv, S0)
    _req_cu(cu_seqlens, q)
    desc = _desc_from(q, v, Wk, chunk, activation, conv_offset, cu_seqlens, max_seqlen)
    _check_shapes(desc, cu_seqlens is not None, k, v, alpha, beta, Wk, Wp, wbeta, conv, S0)
    B, H, dk, dv = desc.B, desc.H, desc.dk, desc.dv
    for name, h in (("conv_hist", conv_hist), ("conv_hist_out", conv_hist_out)):
        if h is not None:
            _req_hist(h, name, q, v, B)
    _on_gpu(q)
    o = torch.empty_like(v)
    ST = torch.empty((B, H, dv, dk), dtype=torch.float32, device=q.device)
    need = forward_workspace_bytes(desc) if saved is None else forward_train_workspace_bytes(desc)
    if workspace is None:
        _, ws = _workspace(need, q.device)
    else:
        ws = workspace
    stream = torch.cuda.current_stream(q.device).cuda_stream
    if saved is None:
        _check(lib().prism_forward(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                   _ptr(beta), _ptr(Wk), _ptr(Wp), _ptr(wbeta), _ptr(conv),
                                   _ptr(S0), _ptr(conv_hist), _ptr(cu_seqlens), _ptr(o), _ptr(ST),
                                   _ptr(conv_hist_out), _ptr(ws), ctypes.c_size_t(ws.numel()),
                                   ctypes.c_void_p(stream)))
    else:
        _check(lib().prism_forward_train(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                         _ptr(beta), _ptr(Wk), _ptr(Wp), _ptr(wbeta), _ptr(conv),
                                         _ptr(S0), _ptr(conv_hist), _ptr(cu_seqlens), _ptr(o),
                                         _ptr(ST), _ptr(conv_hist_out), _ptr(saved),
                                         ctypes.c_size_t(saved.numel()), _ptr(ws),
                                         ctypes.c_size_t(ws.numel()), ctypes.c_void_p(stream)))
    return o, ST


def saved_buffer(q, v, Wk=None, chunk=64, cu_seqlens=None, max_seqlen=None):
    """A 256-byte aligned device buffer for the training pair (uint8 view);
    its size does not depend on the activation or the tap offset."""
    desc = _desc_from(q, v, Wk, chunk, cu_seqlens=cu_seqlens, max_seqlen=max_seqlen)
    return _workspace(saved_bytes(desc), q.device)[1]


def backward(q, k, v, alpha, beta, Wk=None, Wp=None, wbeta=None, conv=None, S0=None, dO=None,
             dST=None, chunk=64, need_dS0=False, workspace=None, saved=None, activation="gelu",
             conv_offset=0, conv_hist=None, need_dconv_hist=False, cu_seqlens=None,
             max_seqlen=None):
    """Gradients of <dO, o> + <dST, S_T> with respect to every input.

    Returns a dict: dq, dk, dv (input dtype), dalpha, dbeta (fp32), and for
    L > 0 dWk, dWp, dwbeta, dconv (fp32); dS0 (fp32) when need_dS0.
    With `saved` (filled by forward(..., saved=...) on the same inputs) this is
    prism_backward_train, which skips the forward recompute.  activation,
    conv_offset and conv_hist as in forward() (and equal to the forward's
    with `saved`); need_dconv_hist adds dconv_hist [B,4,H,dv] fp32.
    cu_seqlens and max_seqlen as in forward().
    """
    _validate_inputs(q, k, v, alpha, beta, Wk, Wp, wbeta, conv, S0)
    if dO is None:
        raise ValueError("dO is required")
    _req(dO, "dO", q.dtype, q.device)
    _req_cu(cu_seqlens, q)
    desc = _desc_from(q, v, Wk, chunk, activation, conv_offset, cu_seqlens, max_seqlen)
    if dST is not None:
        _req(dST, "dST", torch.float32, q.device)
    _check_shapes(desc, cu_seqlens is not None, k, v, alpha, beta, Wk, Wp, wbeta, conv, S0,
                  extra=(("dO", dO, "tok"), ("dST", dST, "state")))
    B, H, dk, dv_ = desc.B, desc.H, desc.dk, desc.dv
    if conv_hist is not None:
        _req_hist(conv_hist, "conv_hist", q, v, B)
    _on_gpu(q)
    dev = q.device
    g = {"dq": torch.empty_like(q), "dk": torch.empty_like(k), "dv": torch.empty_like(v),
         "dalpha": torch.empty_like(alpha), "dbeta": torch.empty_like(beta)}
    if Wk is not None:
        g["dWk"] = torch.empty(Wk.shape, dtype=torch.float32, device=dev)
        g["dWp"] = torch.empty(Wp.shape, dtype=torch.float32, device=dev)
        g["dwbeta"] = torch.empty(wbeta.shape, dtype=torch.float32, device=dev)
        g["dconv"] = torch.empty(conv.shape, dtype=torch.float32, device=dev)
    if need_dS0:
        g["dS0"] = torch.empty((B, H, dv_, dk), dtype=torch.float32, device=dev)
    if need_dconv_hist:
        g["dconv_hist"] = torch.empty((B, 4, H, dv_), dtype=torch.float32, device=dev)
    need = backward_workspace_bytes(desc) if saved is None else backward_train_workspace_bytes(desc)
    if workspace is None:
        _, ws = _workspace(need, dev)
    else:
        ws = workspace
    stream = torch.cuda.current_stream(dev).cuda_stream
    grads = (_ptr(g["dq"]), _ptr(g["dk"]), _ptr(g["dv"]), _ptr(g["dalpha"]), _ptr(g["dbeta"]),
             _ptr(g.get("dWk")), _ptr(g.get("dWp")), _ptr(g.get("dwbeta")), _ptr(g.get("dconv")),
             _ptr(g.get("dS0")), _ptr(g.get("dconv_hist")))
    inputs = (_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(Wk), _ptr(Wp),
              _ptr(wbeta), _ptr(conv), _ptr(S0), _ptr(conv_hist), _ptr(cu_seqlens))
    if saved is None:
        _check(lib().prism_backward(ctypes.byref(desc), *inputs, _ptr(dO), _ptr(dST), *grads,
                                    _ptr(ws), ctypes.c_size_t(ws.numel()), ctypes.c_void_p(stream)))
    else:
        _check(lib().prism_backward_train(ctypes.byref(desc), *inputs, _ptr(saved),
                                          ctypes.c_size_t(saved.numel()), _ptr(dO), _ptr(dST),
                                          *grads, _ptr(ws), ctypes.c_size_t(ws.numel()),
                                          ctypes.c_void_p(stream)))
    return g


def step_workspace_bytes(desc):
    n = ctypes.c_size_t(0)
    _check(lib().prism_step_workspace(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def step(q, k, v, alpha, beta, Wk=None, Wp=None, wbeta=None, conv=None, S=None, conv_state=None,
         activation="gelu", conv_offset=0, workspace=None, noalloc=False):
    """Recurrent form (prism_step): the T tokens of each sequence in order,
    token by token.  S [B,H,dv,dk] fp32 is required and updated in place
    (S_0 in, S_T out); conv_state [B,4,H,dv] (v's dtype) likewise, or None
    for a zero history that is not kept.  Returns o [B,T,H,dv].  With T = 1
    this is one decode step.  noalloc=True calls prism_step_noalloc (the
    pairs go to the library's fixed device array; no workspace, nothing
    allocated but the output)."""
    _validate_inputs(q, k, v, alpha, beta, Wk, Wp, wbeta, conv, S)
    if S is None:
        raise ValueError("S is required")
    desc = _desc_from(q, v, Wk, 16, activation, conv_offset)
    _check_shapes(desc, False, k, v, alpha, beta, Wk, Wp, wbeta, conv, S, state_name="S")
    if conv_state is not None:
        _req_hist(conv_state, "conv_state", q, v)
    _on_gpu(q)
    o = torch.empty_like(v)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    if noalloc:
        _check(lib().prism_step_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                        _ptr(beta), _ptr(Wk), _ptr(Wp), _ptr(wbeta), _ptr(conv),
                                        _ptr(S), _ptr(conv_state), _ptr(o), ctypes.c_void_p(stream)))
        return o
    if workspace is None:
        _, workspace = _workspace(step_workspace_bytes(desc), q.device)
    _check(lib().prism_step(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                            _ptr(beta), _ptr(Wk), _ptr(Wp), _ptr(wbeta), _ptr(conv), _ptr(S),
                            _ptr(conv_state), _ptr(o), _ptr(workspace),
                            ctypes.c_size_t(workspace.numel()), ctypes.c_void_p(stream)))
    return o


class KernelTimer:
    """Context manager: event-measured duration of every library kernel
    launched inside the block (prism_timing_begin / prism_timing_end)."""

    def __enter__(self):
        lib().prism_timing_begin()
        self.result = {}
        return self

    def __exit__(self, *exc):
        cap = 64
        names = (ctypes.c_char_p * cap)()
        ms = (ctypes.c_double * cap)()
        cnt = (ctypes.c_int * cap)()
        n = lib().prism_timing_end(names, ms, cnt, cap)
        self.result = {names[i].decode(): (ms[i], cnt[i]) for i in range(min(n, cap))}
        return False
