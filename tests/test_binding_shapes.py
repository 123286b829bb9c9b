"""Host-side shape checks of the Python binding (no GPU, no library call).

The C ABI sees only pointers and the descriptor, so the binding checks every
tensor's shape against the descriptor before a pointer leaves Python: a
mismatch raises ValueError naming the tensor.  Tensors on a non-GPU device are
refused after the shape checks.  All calls here use CPU tensors and stop at a
ValueError before any library call.
"""
import pytest
import torch

from linear_recurrent_sequence_shortconv_amd import prism as P

B, T, H, D, L = 2, 12, 3, 16, 2
BF = torch.bfloat16


def _inputs(**over):
    x = {
        "q": torch.zeros(B, T, H, D, dtype=BF), "k": torch.zeros(B, T, H, D, dtype=BF),
        "v": torch.zeros(B, T, H, D, dtype=BF),
        "alpha": torch.ones(B, T, H), "beta": torch.zeros(B, T, H),
        "Wk": torch.zeros(H, L, D, D, dtype=BF), "Wp": torch.zeros(H, L, D, D, dtype=BF),
        "wbeta": torch.zeros(H, L, D, dtype=BF), "conv": torch.zeros(H, D, 4, dtype=BF),
        "S0": torch.zeros(B, H, D, D),
    }
    x.update(over)
    return x


def _fwd(x, **kw):
    return P.forward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["Wk"], x["Wp"], x["wbeta"],
                     x["conv"], S0=x["S0"], chunk=16, **kw)


def _bwd(x, dO, dST=None):
    return P.backward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["Wk"], x["Wp"],
                      x["wbeta"], x["conv"], S0=x["S0"], dO=dO, dST=dST, chunk=16)


BAD = [
    ("k", torch.zeros(B, T + 1, H, D, dtype=BF)),
    ("v", torch.zeros(B, T, H, D + 16, dtype=BF)),
    ("alpha", torch.ones(B, T, H + 1)),
    ("beta", torch.zeros(B, T)),
    ("Wk", torch.zeros(H, L, D, D + 16, dtype=BF)),
    ("Wp", torch.zeros(H, L + 1, D, D, dtype=BF)),
    ("wbeta", torch.zeros(H, L + 1, D, dtype=BF)),
    ("conv", torch.zeros(H, D, 3, dtype=BF)),
    ("S0", torch.zeros(B, H, D, D + 1)),
]


@pytest.mark.parametrize("name,bad", BAD, ids=[n for n, _ in BAD])
def test_forward_rejects_wrong_shape(name, bad):
    with pytest.raises(ValueError, match=name):
        _fwd(_inputs(**{name: bad}))


@pytest.mark.parametrize("name,bad", BAD, ids=[n for n, _ in BAD])
def test_backward_rejects_wrong_shape(name, bad):
    with pytest.raises(ValueError, match=name):
        _bwd(_inputs(**{name: bad}), torch.zeros(B, T, H, D, dtype=BF))


def test_backward_rejects_wrong_dO_and_dST():
    x = _inputs()
    with pytest.raises(ValueError, match="dO"):
        _bwd(x, torch.zeros(B, T - 1, H, D, dtype=BF))
    with pytest.raises(ValueError, match="dST"):
        _bwd(x, torch.zeros(B, T, H, D, dtype=BF), dST=torch.zeros(B, H + 1, D, D))


def test_q_rank_and_history_shape():
    x = _inputs(q=torch.zeros(B * T, H, D, dtype=BF))
    with pytest.raises(ValueError, match="q"):
        _fwd(x)
    x = _inputs()
    with pytest.raises(ValueError, match="conv_hist"):
        _fwd(x, conv_hist=torch.zeros(B, 3, H, D, dtype=BF))


def test_packed_batch_shapes():
    N = 17
    cu = torch.tensor([0, 5, 17], dtype=torch.int32)
    x = _inputs(q=torch.zeros(N, H, D, dtype=BF), k=torch.zeros(N, H, D, dtype=BF),
                v=torch.zeros(N, H, D, dtype=BF), alpha=torch.ones(N, H),
                beta=torch.zeros(N, H))
    with pytest.raises(ValueError, match="alpha"):
        _fwd(dict(x, alpha=torch.ones(N + 1, H)), cu_seqlens=cu, max_seqlen=12)
    with pytest.raises(ValueError, match="k"):
        _fwd(dict(x, k=torch.zeros(N - 1, H, D, dtype=BF)), cu_seqlens=cu, max_seqlen=12)
    with pytest.raises(ValueError, match="GPU"):   # shapes fine: refused as CPU tensors
        _fwd(x, cu_seqlens=cu, max_seqlen=12)


def test_step_shapes():
    x = _inputs(q=torch.zeros(B, 1, H, D, dtype=BF), k=torch.zeros(B, 1, H, D, dtype=BF),
                v=torch.zeros(B, 1, H, D, dtype=BF), alpha=torch.ones(B, 1, H),
                beta=torch.zeros(B, 1, H))
    args = [x[n] for n in ("q", "k", "v", "alpha", "beta", "Wk", "Wp", "wbeta", "conv")]
    with pytest.raises(ValueError, match="S: expected"):
        P.step(*args, S=torch.zeros(B, H, D, D + 1))
    args[3] = torch.ones(B, 2, H)
    with pytest.raises(ValueError, match="alpha"):
        P.step(*args, S=torch.zeros(B, H, D, D))


def test_cpu_tensors_refused_after_shape_checks():
    with pytest.raises(ValueError, match="GPU"):
        _fwd(_inputs())
    with pytest.raises(ValueError, match="GPU"):
        _bwd(_inputs(), torch.zeros(B, T, H, D, dtype=BF))
