"""The chunked algebra the kernels implement equals the token recurrence.

Compares tests/chunked_model.py (float64 chunked affine maps and their
adjoint) with the float64 oracle, for several chunk sizes, ragged lengths and
refinement depths.  Agreement to ~1e-11 shows the rearrangement is exact
(the PRISM summary, §2.2 last paragraph: the update depends on the input
only, which is what allows chunking / prefix scanning).
"""
import numpy as np
import pytest

from oracle import prism_oracle as O
from linear_recurrent_sequence_shortconv_amd.workloads import make_inputs
from tests import chunked_model as CM


def _oracle(x, L):
    a = dict(x)
    if L == 0:
        a.update(Wk=None, Wp=None, wbeta=None, conv=None)
    o, s = O.forward(a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["Wk"], a["Wp"],
                     a["wbeta"], a["conv"], S0=a["S0"])
    g = O.backward(a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["Wk"], a["Wp"],
                   a["wbeta"], a["conv"], S0=a["S0"], dO=a["dO"], dST=a["dST"])
    return o, s, g


@pytest.mark.parametrize("C,T,L", [(1, 7, 2), (2, 9, 1), (3, 10, 3), (4, 16, 0),
                                   (16, 37, 2), (16, 64, 3), (37, 37, 1)])
def test_chunked_equals_oracle(C, T, L):
    x = make_inputs(2, T, 2, 5, L, "f32", seed=100 + C + T + L, random_S0=True, with_dST=True)
    o, s, g = _oracle(x, L)
    oc, sc, gc = CM.forward_backward(x, C, dST=x["dST"])
    scale = lambda a: max(1.0, np.max(np.abs(a)))
    assert np.max(np.abs(oc - o)) / scale(o) < 1e-11
    assert np.max(np.abs(sc - s)) / scale(s) < 1e-11
    for key in g:
        err = np.max(np.abs(gc[key] - g[key])) / scale(g[key])
        assert err < 1e-10, (key, err)


def test_chunked_long_memory():
    """alpha close to 1 (logit mean 6): memory spans many chunks."""
    x = make_inputs(1, 50, 1, 4, 2, "f32", seed=9, alpha_logit_mean=6.0, with_dST=True)
    o, s, g = _oracle(x, 2)
    oc, sc, gc = CM.forward_backward(x, 8, dST=x["dST"])
    assert np.max(np.abs(oc - o)) < 1e-11 and np.max(np.abs(sc - s)) < 1e-11
    for key in g:
        assert np.max(np.abs(gc[key] - g[key])) < 1e-9, key
