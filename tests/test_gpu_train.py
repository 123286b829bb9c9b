"""GPU parity of the training pair (prism_forward_train / prism_backward_train).

The training forward runs the same kernels as prism_forward (plus two extra
stores), so its outputs must be bitwise equal to the plain forward's.  The
training backward starts from the kept intermediates and must meet the same
bars against the float64 oracle as the stateless backward (max relative
error 1e-4 for fp32 storage, 2e-2 for bf16), on every gradient.
"""
import numpy as np
import pytest
import torch

from oracle import prism_oracle as O
from linear_recurrent_sequence_shortconv_amd.workloads import make_inputs, workloads
from tests.parity import relerr

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
TDT = {"f32": torch.float32, "bf16": torch.bfloat16}
SEQ_GRADS = ("dq", "dk", "dv", "dalpha", "dbeta")
W_GRADS = ("dWk", "dWp", "dwbeta", "dconv")


def _dev(a, dtype):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(dtype)


def _args(x, dtype, L):
    t, f = TDT[dtype], torch.float32
    w = (lambda n: _dev(x[n], t)) if L > 0 else (lambda n: None)
    return (_dev(x["q"], t), _dev(x["k"], t), _dev(x["v"], t), _dev(x["alpha"], f),
            _dev(x["beta"], f), w("Wk"), w("Wp"), w("wbeta"), w("conv"))


def train_pair(x, dtype, chunk, L):
    from linear_recurrent_sequence_shortconv_amd import prism as P
    a = _args(x, dtype, L)
    S0 = _dev(x["S0"], torch.float32)
    saved = P.saved_buffer(a[0], a[2], a[5], chunk)
    o, ST = P.forward(*a, S0=S0, chunk=chunk, saved=saved)
    g = P.backward(*a, S0=S0, dO=_dev(x["dO"], TDT[dtype]), dST=_dev(x["dST"], torch.float32),
                   chunk=chunk, need_dS0=True, saved=saved)
    torch.cuda.synchronize()
    return o, ST, g


@pytest.mark.parametrize("dtype,d,chunk", [("f32", 32, 32), ("bf16", 128, 64), ("bf16", 64, 16)])
def test_train_forward_bitwise_equals_forward(dtype, d, chunk):
    from linear_recurrent_sequence_shortconv_amd import prism as P
    x = make_inputs(2, 97, 2, d, 2, dtype, seed=31 + d, random_S0=True, with_dST=True)
    print(f"\n[train forward {dtype} d={d} chunk={chunk}]", flush=True)
    a = _args(x, dtype, 2)
    S0 = _dev(x["S0"], torch.float32)
    o1, s1 = P.forward(*a, S0=S0, chunk=chunk)
    o2, s2, _ = train_pair(x, dtype, chunk, 2)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


@pytest.mark.parametrize("dtype,d,chunk,L", [("f32", 16, 16, 2), ("f32", 32, 32, 3), ("f32", 64, 32, 0),
                                             ("bf16", 128, 64, 3), ("bf16", 128, 32, 1),
                                             ("bf16", 64, 64, 2)])
def test_train_backward_matches_oracle(dtype, d, chunk, L):
    x = make_inputs(2, 90, 2, d, L, dtype, seed=41 + d + L, random_S0=True, with_dST=True)
    print(f"\n[train backward {dtype} d={d} chunk={chunk} L={L} T=90]", flush=True)
    o, ST, g = train_pair(x, dtype, chunk, L)
    Wn = [x[n] for n in ("Wk", "Wp", "wbeta", "conv")] if L > 0 else [None] * 4
    oo, so = O.forward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], *Wn, S0=x["S0"])
    go = O.backward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], *Wn, S0=x["S0"], dO=x["dO"],
                    dST=x["dST"])
    errs = {"o": relerr(o.double().cpu().numpy(), oo), "ST": relerr(ST.double().cpu().numpy(), so)}
    for n in SEQ_GRADS + (W_GRADS if L > 0 else ()) + ("dS0",):
        errs[n] = relerr(g[n].double().cpu().numpy(), go[n])
    print("  " + "  ".join(f"{n} {e:.2e}" for n, e in errs.items()), flush=True)
    bad = {n: e for n, e in errs.items() if not e <= TOL[dtype]}
    assert not bad, bad


def test_train_pair_lm_workload_sampled():
    """The timed training pair at its full size (B=8, H=16, T=2048, d=128,
    L=3): two sequences' gradients and dS0, and one head's weight and tap
    gradients (sums over all eight sequences of that head)."""
    w = workloads()["lm-T2048"]
    x = make_inputs(w.B, w.T, w.H, w.d, w.L, w.dtype, seed=0)
    print(f"\n[{w.name} train pair, sequences (3,7), (6,12), weights of head 12]", flush=True)
    _, _, g = train_pair(x, w.dtype, w.chunk, w.L)
    g = {n: t.double().cpu().numpy() for n, t in g.items()}
    for n in SEQ_GRADS + W_GRADS + ("dS0",):
        assert np.all(np.isfinite(g[n])), n
    for b, h in [(3, 7), (6, 12)]:
        s = lambda n: x[n][b:b + 1, :, h:h + 1]
        Wn = [x[n][h:h + 1] for n in ("Wk", "Wp", "wbeta", "conv")]
        go = O.backward(s("q"), s("k"), s("v"), s("alpha"), s("beta"), *Wn, dO=s("dO"))
        errs = {n: relerr(g[n][b:b + 1, :, h:h + 1], go[n]) for n in SEQ_GRADS}
        errs["dS0"] = relerr(g["dS0"][b:b + 1, h:h + 1], go["dS0"])
        print(f"  (b={b},h={h}) " + "  ".join(f"{n} {e:.2e}" for n, e in errs.items()), flush=True)
        assert all(e <= TOL[w.dtype] for e in errs.values()), errs
    hh = 12
    s = lambda n: x[n][:, :, hh:hh + 1]
    Wn = [x[n][hh:hh + 1] for n in ("Wk", "Wp", "wbeta", "conv")]
    go = O.backward(s("q"), s("k"), s("v"), s("alpha"), s("beta"), *Wn, dO=s("dO"))
    errs = {n: relerr(g[n][hh:hh + 1], go[n]) for n in W_GRADS}
    print(f"  (weights, h={hh}) " + "  ".join(f"{n} {e:.2e}" for n, e in errs.items()), flush=True)
    assert all(e <= TOL[w.dtype] for e in errs.values()), errs


@pytest.mark.parametrize("B,H", [(1, 4), (4, 16), (8, 16)], ids=["rows16", "rows32", "rows64"])
def test_state_row_block_widths(B, H):
    """At d = 128 the state passes split the state into row blocks of 16, 32
    or 64 rows depending on how many sequence-heads fill the chip (B H = 4,
    64, 128 here): each width against the oracle, forward and training pair."""
    x = make_inputs(B, 50, H, 128, 1, "bf16", seed=90 + B * H, random_S0=True, with_dST=True)
    print(f"\n[state row blocks B={B} H={H} d=128 T=50]", flush=True)
    o, ST, g = train_pair(x, "bf16", 32, 1)
    Wn = [x[n] for n in ("Wk", "Wp", "wbeta", "conv")]
    oo, so = O.forward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], *Wn, S0=x["S0"])
    go = O.backward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], *Wn, S0=x["S0"], dO=x["dO"],
                    dST=x["dST"])
    errs = {"o": relerr(o.double().cpu().numpy(), oo), "ST": relerr(ST.double().cpu().numpy(), so)}
    for n in SEQ_GRADS + ("dS0",):
        errs[n] = relerr(g[n].double().cpu().numpy(), go[n])
    print("  " + "  ".join(f"{n} {e:.2e}" for n, e in errs.items()), flush=True)
    assert all(e <= TOL["bf16"] for e in errs.values()), errs
