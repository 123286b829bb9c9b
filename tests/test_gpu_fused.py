"""GPU checks of the fused inference forward.

prism_forward without a saved buffer forms the refinement pairs (ShortConv
anchor, projections, activation chain, step gates of the PRISM summary
§2.2) inside the chunk kernel instead of writing them to HBM and reading
them back.  The fused kernel repeats the separate refinement kernel's
arithmetic in the same order and rounding, so its outputs are compared
bitwise with the training forward (which keeps the separate kernels), on
every head size and chunk length, both activations and tap offsets, with and
without a ShortConv history, dense and packed.  Sequence lengths end in a
ragged tail and include lengths shorter than the ShortConv reach.  A second
set compares the bf16 path at d = 16 (16-wide MFMA in the projections)
with the float64 oracle, forward and both backward paths.
"""
import numpy as np
import pytest
import torch

from oracle import prism_oracle as O
from linear_recurrent_sequence_shortconv_amd.workloads import make_inputs
from tests.parity import relerr

pytestmark = pytest.mark.gpu

TDT = {"f32": torch.float32, "bf16": torch.bfloat16}
WN = ("Wk", "Wp", "wbeta", "conv")


def _dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(dtype)


def _args(x, dtype):
    t, f = TDT[dtype], torch.float32
    return tuple(_dev(x[n], t) for n in ("q", "k", "v")) + tuple(
        _dev(x[n], f) for n in ("alpha", "beta")) + tuple(_dev(x[n], t) for n in WN)


# (dtype, d, chunk, L, T): every (d, chunk) the kernels take, several depths
SHAPES = [("bf16", 128, 64, 3, 200), ("bf16", 128, 32, 2, 97), ("bf16", 128, 16, 1, 50),
          ("bf16", 64, 64, 4, 130), ("bf16", 64, 16, 8, 33), ("bf16", 32, 32, 2, 70),
          ("bf16", 16, 64, 3, 90), ("bf16", 16, 16, 2, 2), ("f32", 64, 32, 3, 77),
          ("f32", 32, 64, 2, 65), ("f32", 16, 16, 5, 3), ("bf16", 128, 64, 1, 1)]
VARIANTS = [("gelu", 0), ("identity", 1)]


@pytest.mark.parametrize("act,off", VARIANTS, ids=[f"{a}-off{o}" for a, o in VARIANTS])
@pytest.mark.parametrize("dtype,d,chunk,L,T", SHAPES,
                         ids=[f"{s[0]}-d{s[1]}-c{s[2]}-L{s[3]}-T{s[4]}" for s in SHAPES])
def test_fused_forward_equals_separate_kernels(act, off, dtype, d, chunk, L, T):
    from linear_recurrent_sequence_shortconv_amd import prism as P
    print(f"\n[fused {dtype} d={d} chunk={chunk} L={L} T={T} {act} conv_offset={off}]", flush=True)
    B, H = 2, 3
    x = make_inputs(B, T, H, d, L, dtype, seed=500 + d + chunk + L + off, random_S0=True)
    a = _args(x, dtype)
    rng = np.random.default_rng(d + L)
    hist = _dev(rng.standard_normal((B, 4, H, d)), TDT[dtype])
    S0 = _dev(x["S0"], torch.float32)
    for h in (None, hist):
        kw = dict(chunk=chunk, activation=act, conv_offset=off, S0=S0, conv_hist=h)
        o1, s1 = P.forward(*a, **kw)                       # fused
        saved = P.saved_buffer(a[0], a[2], a[5], chunk)
        o2, s2 = P.forward(*a, saved=saved, **kw)          # separate refinement kernel
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(s1, s2), "history" if h is not None else "zeros"


def test_fused_forward_packed_equals_separate_kernels():
    from linear_recurrent_sequence_shortconv_amd import prism as P
    lengths = [130, 0, 1, 64, 3, 200, 65]
    d, H, L, chunk = 128, 2, 3, 64
    print(f"\n[fused packed bf16 d={d} lengths={lengths}]", flush=True)
    N = sum(lengths)
    x = make_inputs(1, N, H, d, L, "bf16", seed=77)
    a = tuple(t[0] if i < 5 else t for i, t in enumerate(_args(x, "bf16")))
    cu = _dev(np.concatenate([[0], np.cumsum(lengths)]), torch.int32)
    hist = _dev(np.random.default_rng(3).standard_normal((len(lengths), 4, H, d)), torch.bfloat16)
    kw = dict(chunk=chunk, cu_seqlens=cu, max_seqlen=max(lengths), conv_hist=hist)
    o1, s1 = P.forward(*a, **kw)
    saved = P.saved_buffer(a[0], a[2], a[5], chunk, cu_seqlens=cu, max_seqlen=max(lengths))
    o2, s2 = P.forward(*a, saved=saved, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


@pytest.mark.parametrize("chunk,L,T", [(16, 2, 45), (64, 3, 130), (32, 8, 7)])
def test_bf16_d16_matches_oracle(chunk, L, T):
    """bf16 at d = 16: projections on the 16x16x16 MFMA, forward and both
    backward paths against the float64 oracle at the bf16 bar (2e-2)."""
    from linear_recurrent_sequence_shortconv_amd import prism as P
    print(f"\n[bf16 d=16 chunk={chunk} L={L} T={T}]", flush=True)
    x = make_inputs(2, T, 2, 16, L, "bf16", seed=40 + chunk + L, random_S0=True, with_dST=True)
    a = _args(x, "bf16")
    S0, dO, dST = (_dev(x["S0"], torch.float32), _dev(x["dO"], torch.bfloat16),
                   _dev(x["dST"], torch.float32))
    o, ST = P.forward(*a, S0=S0, chunk=chunk)
    g = P.backward(*a, S0=S0, dO=dO, dST=dST, need_dS0=True, chunk=chunk)
    saved = P.saved_buffer(a[0], a[2], a[5], chunk)
    P.forward(*a, S0=S0, chunk=chunk, saved=saved)
    g2 = P.backward(*a, S0=S0, dO=dO, dST=dST, need_dS0=True, chunk=chunk, saved=saved)
    torch.cuda.synchronize()
    W = [x[n] for n in WN]
    oo, so = O.forward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], *W, S0=x["S0"])
    go = O.backward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], *W, S0=x["S0"], dO=x["dO"],
                    dST=x["dST"])
    errs = {"o": relerr(o.double().cpu().numpy(), oo), "ST": relerr(ST.double().cpu().numpy(), so)}
    for n in ("dq", "dk", "dv", "dalpha", "dbeta", "dWk", "dWp", "dwbeta", "dconv", "dS0"):
        errs[n] = relerr(g[n].double().cpu().numpy(), go[n])
        errs[n + "(train)"] = relerr(g2[n].double().cpu().numpy(), go[n])
    print("  " + "  ".join(f"{n} {e:.2e}" for n, e in errs.items()), flush=True)
    bad = {n: e for n, e in errs.items() if not e <= 2e-2}
    assert not bad, bad


def test_bf16_d16_decode_step_matches_oracle():
    """The decode step's projections at d = 16 in bf16 (16x16x16 MFMA)."""
    from linear_recurrent_sequence_shortconv_amd import prism as P
    B, H, d, L, T = 5, 2, 16, 3, 6
    print(f"\n[bf16 d=16 step B={B} T={T} L={L}]", flush=True)
    x = make_inputs(B, T, H, d, L, "bf16", seed=91, random_S0=True)
    a = _args(x, "bf16")
    S = _dev(x["S0"], torch.float32)
    cs = torch.zeros((B, 4, H, d), dtype=torch.bfloat16, device="cuda")
    outs = []
    for t in range(T):
        tok = tuple(z[:, t:t + 1].contiguous() for z in a[:5])
        outs.append(P.step(*tok, *a[5:], S=S, conv_state=cs))
    torch.cuda.synchronize()
    o = torch.cat(outs, dim=1)
    W = [x[n] for n in WN]
    oo, so = O.forward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], *W, S0=x["S0"])
    eo, es = relerr(o.double().cpu().numpy(), oo), relerr(S.double().cpu().numpy(), so)
    print(f"  o {eo:.2e}  S {es:.2e}", flush=True)
    assert eo <= 2e-2 and es <= 2e-2
