"""prism_step_noalloc (the recurrent step for callers that cannot allocate:
its refinement pairs live in the library's fixed device array) against
prism_step with a caller workspace, through the C ABI.

Both run the same kernels in the same order, so the outputs, the updated
state and the updated ShortConv history must be bitwise equal.  Two calls in
a row, the second with a smaller batch and fewer tokens, so the second reads
an array that still holds the first call's (larger) contents; then a check
against the float64 oracle on the second call, to the bf16 bar (2e-2).
"""
import numpy as np
import pytest
import torch

from oracle import prism_oracle as O
from linear_recurrent_sequence_shortconv_amd.workloads import make_inputs
from tests.parity import relerr

pytestmark = pytest.mark.gpu


def _dev(a, t):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(t)


def _run(P, x, noalloc, S0, hist):
    t, f = torch.bfloat16, torch.float32
    args = [_dev(x[n], t) for n in ("q", "k", "v")] + [_dev(x[n], f) for n in ("alpha", "beta")]
    args += [_dev(x[n], t) for n in ("Wk", "Wp", "wbeta", "conv")]
    S = S0.clone()
    cs = hist.clone()
    o = P.step(*args, S=S, conv_state=cs, noalloc=noalloc)
    torch.cuda.synchronize()
    return o, S, cs


@pytest.mark.parametrize("d,L", [(128, 3), (64, 2)])
def test_noalloc_step_equals_step(d, L):
    from linear_recurrent_sequence_shortconv_amd import prism as P
    assert "prism_step_noalloc" in P.EXPORTS
    H = 4
    for call, (B, T) in enumerate(((48, 5), (20, 1))):
        print(f"\n[noalloc call {call}: B={B} T={T} H={H} d={d} L={L}]", flush=True)
        x = make_inputs(B, T, H, d, L, "bf16", seed=300 + call + d, random_S0=True)
        S0 = _dev(x["S0"], torch.float32)
        rng = np.random.default_rng(9 + call)
        hist = _dev(rng.standard_normal((B, 4, H, d)), torch.bfloat16)
        o1, S1, c1 = _run(P, x, False, S0, hist)
        o2, S2, c2 = _run(P, x, True, S0, hist)
        assert torch.equal(o1, o2) and torch.equal(S1, S2) and torch.equal(c1, c2)
    # the second (smaller) call against the oracle
    h64 = hist.double().cpu().numpy()
    oo, so = O.forward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["Wk"], x["Wp"],
                       x["wbeta"], x["conv"], S0=x["S0"], conv_hist=h64)
    eo, es = relerr(o2.double().cpu().numpy(), oo), relerr(S2.double().cpu().numpy(), so)
    print(f"  o {eo:.2e}  S {es:.2e}", flush=True)
    assert eo <= 2e-2 and es <= 2e-2

