"""GPU parity of the layer variants against the float64 oracle.

Variants of the PRISM summary §2.2: the refinement step without the GELU
(delta = p * r, the ablation of the nonlinearity) and the ShortConv anchor on
strictly past tokens (tap j on v_{t-1-j}).  Each is checked on the forward
(o, S_T), the stateless backward and the training pair, on every gradient, to
the same bars as the method itself (max relative error 1e-4 for fp32
storage, 2e-2 for bf16).  Sequence lengths span several refinement tiles
(64 tokens forward, 28-29 backward) and end in a ragged tail.
"""
import numpy as np
import pytest
import torch

from oracle import prism_oracle as O
from linear_recurrent_sequence_shortconv_amd.workloads import make_inputs
from tests.parity import relerr

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
TDT = {"f32": torch.float32, "bf16": torch.bfloat16}
GRADS = ("dq", "dk", "dv", "dalpha", "dbeta", "dWk", "dWp", "dwbeta", "dconv", "dS0")
VARIANTS = [("identity", 0), ("gelu", 1), ("identity", 1)]
SHAPES = [("f32", 32, 32, 2, 150), ("f32", 16, 16, 5, 45), ("bf16", 128, 64, 3, 150),
          ("bf16", 64, 16, 1, 61), ("bf16", 32, 32, 2, 3)]


def _dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(dtype)


@pytest.mark.parametrize("act,off", VARIANTS, ids=[f"{a}-off{o}" for a, o in VARIANTS])
@pytest.mark.parametrize("dtype,d,chunk,L,T", SHAPES,
                         ids=[f"{s[0]}-d{s[1]}-c{s[2]}-L{s[3]}-T{s[4]}" for s in SHAPES])
def test_variant_matches_oracle(act, off, dtype, d, chunk, L, T):
    from linear_recurrent_sequence_shortconv_amd import prism as P
    print(f"\n[variant {act} conv_offset={off} {dtype} d={d} chunk={chunk} L={L} T={T}]", flush=True)
    x = make_inputs(2, T, 2, d, L, dtype, seed=300 + 7 * d + L + off, random_S0=True, with_dST=True)
    t, f = TDT[dtype], torch.float32
    a = tuple(_dev(x[n], t) for n in ("q", "k", "v")) + tuple(
        _dev(x[n], f) for n in ("alpha", "beta")) + tuple(
        _dev(x[n], t) for n in ("Wk", "Wp", "wbeta", "conv"))
    S0, dO, dST = _dev(x["S0"], f), _dev(x["dO"], t), _dev(x["dST"], f)
    kw = dict(chunk=chunk, activation=act, conv_offset=off)
    o, ST = P.forward(*a, S0=S0, **kw)
    g = P.backward(*a, S0=S0, dO=dO, dST=dST, need_dS0=True, **kw)
    saved = P.saved_buffer(a[0], a[2], a[5], chunk)
    o2, ST2 = P.forward(*a, S0=S0, saved=saved, **kw)
    g2 = P.backward(*a, S0=S0, dO=dO, dST=dST, need_dS0=True, saved=saved, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(ST, ST2)

    W = [x[n] for n in ("Wk", "Wp", "wbeta", "conv")]
    okw = dict(S0=x["S0"], activation=act, conv_offset=off)
    oo, so = O.forward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], *W, **okw)
    go = O.backward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], *W, dO=x["dO"], dST=x["dST"],
                    **okw)
    errs = {"o": relerr(o.double().cpu().numpy(), oo), "ST": relerr(ST.double().cpu().numpy(), so)}
    for n in GRADS:
        errs[n] = relerr(g[n].double().cpu().numpy(), go[n])
        errs[n + "(train)"] = relerr(g2[n].double().cpu().numpy(), go[n])
    print("  " + "  ".join(f"{n} {e:.2e}" for n, e in errs.items()), flush=True)
    bad = {n: e for n, e in errs.items() if not e <= TOL[dtype]}
    assert not bad, bad


def test_default_fields_are_the_method():
    """activation="gelu", conv_offset=0 runs the same kernels as the defaults."""
    from linear_recurrent_sequence_shortconv_amd import prism as P
    x = make_inputs(1, 70, 2, 64, 2, "bf16", seed=5)
    a = tuple(_dev(x[n], torch.bfloat16) for n in ("q", "k", "v")) + tuple(
        _dev(x[n], torch.float32) for n in ("alpha", "beta")) + tuple(
        _dev(x[n], torch.bfloat16) for n in ("Wk", "Wp", "wbeta", "conv"))
    o1, s1 = P.forward(*a, chunk=32)
    o2, s2 = P.forward(*a, chunk=32, activation="gelu", conv_offset=0)
    o3, _ = P.forward(*a, chunk=32, conv_offset=1)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    assert not torch.equal(o1, o3)
