"""GPU backward parity: every gradient from the HIP library (through the C
ABI) against the float64 oracle's hand-derived reverse pass (itself pinned to
central finite differences in test_oracle_pins.py).

Metric per gradient tensor: max |x - y| / max |y|; tolerances 1e-4 for fp32
storage, 2e-2 for bf16 storage.  At full workload sizes the oracle runs on a
few (b, h) sequences (per-sequence gradients), and on every sequence of one
head for that head's weight and tap gradients (sums over the batch).
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


def gpu_backward(x, dtype, chunk, L):
    from linear_recurrent_sequence_shortconv_amd import prism as P
    t, f = TDT[dtype], torch.float32
    w = (lambda n: _dev(x[n], t)) if L > 0 else (lambda n: None)
    g = P.backward(_dev(x["q"], t), _dev(x["k"], t), _dev(x["v"], t), _dev(x["alpha"], f),
                   _dev(x["beta"], f), w("Wk"), w("Wp"), w("wbeta"), w("conv"), _dev(x["S0"], f),
                   dO=_dev(x["dO"], t), dST=_dev(x["dST"], f), chunk=chunk, need_dS0=True)
    torch.cuda.synchronize()
    return {k_: v_.double().cpu().numpy() for k_, v_ in g.items()}


def oracle_backward(x, L, sl_b=slice(None), sl_h=slice(None)):
    W = [x[n][sl_h] for n in ("Wk", "Wp", "wbeta", "conv")] if L > 0 else [None] * 4
    s = lambda n: None if x[n] is None else x[n][sl_b, :, sl_h]
    s0 = None if x["S0"] is None else x["S0"][sl_b, sl_h]
    dst = None if x["dST"] is None else x["dST"][sl_b, sl_h]
    return O.backward(s("q"), s("k"), s("v"), s("alpha"), s("beta"), *W, S0=s0, dO=s("dO"),
                      dST=dst, segment=64)


def _compare(gg, go, names, tol, tag=""):
    errs = {n: relerr(gg[n], go[n]) for n in names}
    print(f"  {tag} " + "  ".join(f"{n} {e:.2e}" for n, e in errs.items()), flush=True)
    bad = {n: e for n, e in errs.items() if not e <= tol}
    assert not bad, bad


def _check_full(x, dtype, chunk, L):
    gg = gpu_backward(x, dtype, chunk, L)
    go = oracle_backward(x, L)
    names = SEQ_GRADS + (W_GRADS if L > 0 else ()) + ("dS0",)
    _compare(gg, go, names, TOL[dtype])
    return gg, go


@pytest.mark.parametrize("d,chunk", [(16, 16), (16, 64), (32, 32), (64, 16), (64, 32)])
@pytest.mark.parametrize("L", [0, 2])
def test_fp32_backward_ragged(d, chunk, L):
    x = make_inputs(2, 50, 2, d, L, "f32", seed=d + chunk + L, random_S0=True, with_dST=True)
    print(f"\n[fp32 bwd d={d} chunk={chunk} T=50 L={L}]", flush=True)
    _check_full(x, "f32", chunk, L)


@pytest.mark.parametrize("L", [1, 3, 4, 5, 8])
def test_fp32_backward_depths(L):
    x = make_inputs(1, 40, 2, 16, L, "f32", seed=70 + L, random_S0=True, with_dST=True)
    print(f"\n[fp32 bwd d=16 chunk=16 T=40 L={L}]", flush=True)
    _check_full(x, "f32", 16, L)


def test_tiny_fp32_workload_backward():
    w = workloads()["tiny-fp32"]
    x = make_inputs(w.B, w.T, w.H, w.d, w.L, w.dtype, seed=0)
    print(f"\n[{w.name} bwd]", flush=True)
    _check_full(x, w.dtype, w.chunk, w.L)


@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_bf16_d128_backward(chunk):
    x = make_inputs(2, 150, 2, 128, 3, "bf16", seed=5 + chunk, random_S0=True, with_dST=True)
    print(f"\n[bf16 bwd d=128 chunk={chunk} T=150 L=3]", flush=True)
    _check_full(x, "bf16", chunk, 3)


@pytest.mark.parametrize("chunk", [16, 32])
def test_bf16_d128_backward_many_chunks(chunk):
    """More chunks than resident workgroups at d = 128 (B H NC = 520), so
    the persistent chunk-backward workgroups each take several chunks, with a
    ragged last chunk: one sequence's gradients and dS0 against the oracle."""
    T = 64 * chunk + 7
    x = make_inputs(2, T, 4, 128, 3, "bf16", seed=70 + chunk, random_S0=True, with_dST=True)
    print(f"\n[bf16 bwd d=128 chunk={chunk} T={T} H=4 L=3, sequence (1, 2)]", flush=True)
    gg = gpu_backward(x, "bf16", chunk, 3)
    go = oracle_backward(x, 3, slice(1, 2), slice(2, 3))
    gs = {n: gg[n][1:2, :, 2:3] for n in SEQ_GRADS}
    gs["dS0"] = gg["dS0"][1:2, 2:3]
    _compare(gs, go, SEQ_GRADS + ("dS0",), TOL["bf16"], tag="(b=1,h=2)")


def test_bf16_d128_backward_four_steps():
    # the four-step refinement backward keeps one replayed residual for the
    # next reverse step (a kernel instance of its own)
    x = make_inputs(2, 150, 2, 128, 4, "bf16", seed=44, random_S0=True, with_dST=True)
    print("\n[bf16 bwd d=128 chunk=64 T=150 L=4]", flush=True)
    _check_full(x, "bf16", 64, 4)


def test_bf16_backward_long_memory():
    x = make_inputs(2, 300, 2, 64, 2, "bf16", seed=8, alpha_logit_mean=6.0, with_dST=True)
    print("\n[bf16 bwd long memory d=64 T=300 L=2]", flush=True)
    gg, go = _check_full(x, "bf16", 64, 2)
    # The gradient of the refinement values dW_l is kept in fp32 between the
    # chunk and refinement backward kernels: it enters beta^(l) dW_l - dL/dr,
    # which can nearly cancel.  Held in bf16 it gave 1.5e-2 here (5.5e-3 in
    # fp32); this bound keeps that margin.
    assert relerr(gg["dWp"], go["dWp"]) <= 1e-2


def _check_workload(name, pairs, weight_head):
    w = workloads()[name]
    x = make_inputs(w.B, w.T, w.H, w.d, w.L, w.dtype, seed=0)
    print(f"\n[{name} bwd, sequences {pairs}, weight grads of head {weight_head}]", flush=True)
    gg = gpu_backward(x, w.dtype, w.chunk, w.L)
    for n in SEQ_GRADS + ("dS0",):
        assert np.all(np.isfinite(gg[n])), n
    for b, h in pairs:
        go = oracle_backward(x, w.L, slice(b, b + 1), slice(h, h + 1))
        gs = {n: gg[n][b:b + 1, :, h:h + 1] for n in SEQ_GRADS}
        gs["dS0"] = gg["dS0"][b:b + 1, h:h + 1]
        _compare(gs, go, SEQ_GRADS + ("dS0",), TOL[w.dtype], tag=f"(b={b},h={h})")
    if w.L > 0:
        hh = weight_head
        go = oracle_backward(x, w.L, slice(None), slice(hh, hh + 1))
        gw = {n: gg[n][hh:hh + 1] for n in W_GRADS}
        _compare(gw, go, W_GRADS, TOL[w.dtype], tag=f"(weights, h={hh})")


def test_lm_workload_backward():
    _check_workload("lm-T2048", [(0, 0), (5, 9)], weight_head=3)


@pytest.mark.parametrize("L", [0, 1, 2, 4, 8])
def test_depth_backward(L):
    """Refinement-depth sweep at its own shape (B = 4, T = 4096, d = 128):
    every refinement-backward instance (two, three, four and eight steps)."""
    _check_workload(f"depth-L{L}", [(1, 2)], weight_head=14)


@pytest.mark.parametrize("T", [4096, 8192, 16384])
def test_long_context_backward(T):
    """Long-context sweep (B = 16384 / T): the reverse state pass runs over
    up to 256 chunks with 16-row state blocks (B H = 16 at T = 16384); the
    last sequence's gradients and dS0, one head's weight and tap gradients."""
    B = 16384 // T
    _check_workload(f"long-T{T}", [(B - 1, 5)], weight_head=9)


def test_backward_deterministic():
    """Two runs give bitwise identical gradients (no atomics, fixed-order sums)."""
    x = make_inputs(2, 130, 3, 64, 2, "bf16", seed=21, with_dST=True)
    g1 = gpu_backward(x, "bf16", 64, 2)
    g2 = gpu_backward(x, "bf16", 64, 2)
    for n in g1:
        assert np.array_equal(g1[n], g2[n]), n
