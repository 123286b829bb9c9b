"""Pins of the float64 oracle against things other than itself.

Each test ties one part of the oracle to a textbook routine, a closed form, a
brute-force evaluation or finite differences, so that a dropped term, a wrong
sign, a transposed operand or a wrong index fails at least one test.  The
method follows the PRISM technical summary (gist.science, 2602.10796):
§2.1 Write-Forget Decoupling, §2.2 Input-Anchored Loop Unrolling, §3 item 3.
"""
import math
import os

import numpy as np
import pytest
from scipy.special import expit

from oracle import prism_oracle as O
from linear_recurrent_sequence_shortconv_amd.workloads import make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _inputs(B=2, T=9, H=2, d=4, L=2, seed=0, **kw):
    return make_inputs(B, T, H, d, L, "f32", seed, **kw)


def _fwd(x, L=None, **kw):
    args = dict(x)
    if L == 0:
        args.update(Wk=None, Wp=None, wbeta=None, conv=None)
    return O.forward(args["q"], args["k"], args["v"], args["alpha"], args["beta"],
                     args["Wk"], args["Wp"], args["wbeta"], args["conv"],
                     S0=args.get("S0"), **kw)


# ---------------------------------------------------------------------------
# GELU: exact erf form (§2.2 "Residual Update"), pinned to tabulated Phi
# ---------------------------------------------------------------------------
def test_gelu_matches_normal_cdf_table():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "normal_cdf.txt"))
            if l.strip() and not l.startswith("#")]
    for xs, phis in rows:
        x, phi = float(xs), float(phis)
        assert abs(O.gelu(np.float64(x)) - x * phi) < 1e-15, x


def test_gelu_grad_is_derivative():
    z = np.linspace(-4, 4, 81)
    h = 1e-6
    fd = (O.gelu(z + h) - O.gelu(z - h)) / (2 * h)
    assert np.max(np.abs(fd - O.gelu_grad(z))) < 1e-8
    assert O.gelu_grad(np.float64(0.0)) == 0.5


# ---------------------------------------------------------------------------
# Stage 1: ShortConv (§2.2 Stage 1) against numpy's full convolution
# ---------------------------------------------------------------------------
def test_shortconv_is_causal_convolution():
    x = _inputs(B=2, T=11, H=3, d=5)
    u = O.shortconv(x["v"], x["conv"])
    for b in range(2):
        for h in range(3):
            for i in range(5):
                ref = np.convolve(x["v"][b, :, h, i], x["conv"][h, i, :])[:11]
                assert np.allclose(u[b, :, h, i], ref, rtol=0, atol=1e-14)


def test_shortconv_impulse_response_and_no_leak_across_batch():
    B, T, H, d = 2, 10, 1, 3
    conv = np.arange(1, 1 + H * d * 4, dtype=np.float64).reshape(H, d, 4)
    v = np.zeros((B, T, H, d))
    v[1, 2, 0, :] = 1.0                         # impulse at t=2 in sequence 1
    u = O.shortconv(v, conv)
    assert np.all(u[0] == 0)                    # nothing leaks into sequence 0
    for j in range(4):
        assert np.array_equal(u[1, 2 + j, 0], conv[0, :, j])   # tap j hits v_{t-j}
    assert np.all(u[1, :2] == 0) and np.all(u[1, 6:] == 0)


def test_shortconv_strictly_past_is_current_taps_on_delayed_input():
    """conv_offset = 1 equals the current-token convolution of v delayed by one
    token (zero first row); an impulse at t reaches u_{t+1+j} through tap j."""
    x = _inputs(B=2, T=11, H=3, d=5)
    vd = np.zeros_like(x["v"])
    vd[:, 1:] = x["v"][:, :-1]
    assert np.array_equal(O.shortconv(x["v"], x["conv"], conv_offset=1),
                          O.shortconv(vd, x["conv"]))
    conv = np.arange(1, 1 + 3 * 4, dtype=np.float64).reshape(1, 3, 4)
    v = np.zeros((1, 9, 1, 3))
    v[0, 2, 0, :] = 1.0
    u = O.shortconv(v, conv, conv_offset=1)
    for j in range(4):
        assert np.array_equal(u[0, 3 + j, 0], conv[0, :, j])
    assert np.all(u[0, :3] == 0) and np.all(u[0, 7:] == 0)
    # first token sees no history at all
    assert np.all(O.shortconv(x["v"], x["conv"], conv_offset=1)[:, 0] == 0)


# ---------------------------------------------------------------------------
# Stage 2: refinement chain (§2.2 Stage 2)
# ---------------------------------------------------------------------------
def test_refinement_identity_activation_closed_form():
    """With delta = p*r (no GELU): r^(l+1) = (1-p^(l)) r^(l), hence
    delta^(l) = p^(l) r^(1) prod_{j<l} (1 - p^(j)); gate = sigmoid(w_beta . u);
    direction k^(l) = W_k^(l) u (matrix times column, not its transpose)."""
    x = _inputs(B=1, T=6, H=2, d=4, L=3)
    u = O.shortconv(x["v"], x["conv"])
    ref = O.refine(u, x["v"], x["Wk"], x["Wp"], x["wbeta"], activation="identity")
    for t in range(6):
        for h in range(2):
            uu = u[0, t, h]
            r1 = x["v"][0, t, h] - uu
            keep = np.ones(4)
            for l in range(3):
                p = np.array([sum(x["Wp"][h, l, i, j] * uu[j] for j in range(4)) for i in range(4)])
                kap = np.array([sum(x["Wk"][h, l, i, j] * uu[j] for j in range(4)) for i in range(4)])
                g = expit(sum(x["wbeta"][h, l, j] * uu[j] for j in range(4)))
                delta = p * r1 * keep
                assert np.allclose(ref["kappa"][l][0, t, h], kap, atol=1e-13)
                assert np.allclose(ref["delta"][l][0, t, h], delta, atol=1e-13)
                assert np.allclose(ref["w"][l][0, t, h], g * delta, atol=1e-13)
                keep = keep * (1.0 - p)


def test_refinement_vanishes_when_anchor_equals_value():
    """Only tap 0 = 1: u = v, r^(1) = 0, every delta = GELU(0) = 0, so the layer
    is Gated DeltaNet whatever the weights."""
    x = _inputs(T=12, L=3)
    conv = np.zeros_like(x["conv"])
    conv[..., 0] = 1.0
    y = dict(x, conv=conv)
    o1, s1 = _fwd(y)
    o0, s0 = _fwd(x, L=0)
    assert np.max(np.abs(o1 - o0)) < 1e-14 and np.max(np.abs(s1 - s0)) < 1e-14


def test_refinement_vanishes_with_zero_gain():
    x = _inputs(T=12, L=2)
    y = dict(x, Wp=np.zeros_like(x["Wp"]))
    o1, s1 = _fwd(y)
    o0, s0 = _fwd(x, L=0)
    assert np.max(np.abs(o1 - o0)) < 1e-14 and np.max(np.abs(s1 - s0)) < 1e-14


# ---------------------------------------------------------------------------
# recurrence: L = 0 is Gated DeltaNet (§3 item 3); §2.1 product order
# ---------------------------------------------------------------------------
def _gdn_textbook(q, k, v, alpha, beta, S0=None):
    """Gated DeltaNet as usually written: decay the memory by alpha_t, then one
    delta-rule step towards v_t along k_t; read out with the new memory."""
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    ST = np.zeros((B, H, dv, dk))
    for b in range(B):
        for h in range(H):
            S = np.zeros((dv, dk)) if S0 is None else S0[b, h].copy()
            for t in range(T):
                S = alpha[b, t, h] * S
                pred = S @ k[b, t, h]
                S = S + beta[b, t, h] * np.outer(v[b, t, h] - pred, k[b, t, h])
                o[b, t, h] = S @ q[b, t, h]
            ST[b, h] = S
    return o, ST


@pytest.mark.parametrize("random_S0", [False, True])
def test_L0_is_gated_deltanet(random_S0):
    x = _inputs(B=2, T=23, H=3, d=5, L=0, random_S0=random_S0)
    o, s = _fwd(x, L=0)
    og, sg = _gdn_textbook(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["S0"])
    assert np.max(np.abs(o - og)) < 1e-12 and np.max(np.abs(s - sg)) < 1e-12


def test_delta_rule_overwrites_along_unit_key():
    """L = 0, beta = 1, |k| = 1: after the step the memory maps k_t to v_t exactly."""
    rng = np.random.default_rng(5)
    B, T, H, d = 1, 10, 2, 6
    k = rng.standard_normal((B, T, H, d))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q = rng.standard_normal((B, T, H, d))
    v = rng.standard_normal((B, T, H, d))
    alpha = rng.uniform(0.2, 1.0, (B, T, H))
    _, _, states = O.forward(q, k, v, alpha, np.ones((B, T, H)), return_states=True)
    Sk = np.einsum("bthij,bthj->bthi", states, k)
    assert np.max(np.abs(Sk - v)) < 1e-12


def _write_and_forget(x, activation="gelu"):
    """Materialise A_t = alpha_t (I - beta_t k_t k_t^T) and
    B_t = beta_t v_t k_t^T + sum_l w^(l) k^(l)^T as d x d matrices."""
    B, T, H, d = x["k"].shape
    I = np.eye(d)
    A = x["alpha"][..., None, None] * (I - x["beta"][..., None, None]
                                       * x["k"][..., :, None] * x["k"][..., None, :])
    Bm = x["beta"][..., None, None] * x["v"][..., :, None] * x["k"][..., None, :]
    if x["Wk"] is not None and x["Wk"].shape[1] > 0:
        Bm = Bm + O.injection(x["v"], x["Wk"], x["Wp"], x["wbeta"], x["conv"], activation)
    return A, Bm


def test_brute_force_product_of_forget_operators():
    """S_t = S_0 A_1 ... A_t + sum_{s<=t} B_s A_{s+1} ... A_t for every prefix
    t <= 8, with explicit d x d products (§2.1, right multiplication)."""
    x = _inputs(B=1, T=8, H=2, d=4, L=2, random_S0=True)
    _, _, states = _fwd(x, return_states=True)
    A, Bm = _write_and_forget(x)
    for h in range(2):
        for t in range(8):
            P = np.eye(4)
            for s in range(t + 1):
                P = P @ A[0, s, h]
            S = x["S0"][0, h] @ P
            for s in range(t + 1):
                P = np.eye(4)
                for r in range(s + 1, t + 1):
                    P = P @ A[0, r, h]
                S = S + Bm[0, s, h] @ P
            assert np.max(np.abs(S - states[0, t, h])) < 1e-12, (h, t)


def _tree_scan(items):
    """Inclusive scan of affine maps S -> S A + B, combining in tree order:
    (A, B) then (A', B') is (A A', B A' + B')."""
    if len(items) == 1:
        return items
    mid = len(items) // 2
    left = _tree_scan(items[:mid])
    right = _tree_scan(items[mid:])
    At, Bt = left[-1]
    return left + [(At @ A2, Bt @ A2 + B2) for A2, B2 in right]


def test_parallel_scan_equals_sequential():
    """The update depends on the input only (§2.2 last paragraph), so the
    maps compose associatively and any scan order gives the same states."""
    x = _inputs(B=1, T=16, H=1, d=4, L=3, random_S0=True)
    _, _, states = _fwd(x, return_states=True)
    A, Bm = _write_and_forget(x)
    pref = _tree_scan([(A[0, t, 0], Bm[0, t, 0]) for t in range(16)])
    for t in range(16):
        S = x["S0"][0, 0] @ pref[t][0] + pref[t][1]
        assert np.max(np.abs(S - states[0, t, 0])) < 1e-12


def test_write_path_closed_form_without_forgetting():
    """alpha = 1, beta = 0: S_t = S_0 + sum_{s<=t} sum_l w_s^(l) k_s^(l)^T, so
    o_t = S_0 q_t + sum_{s<=t} sum_l w_s^(l) (k_s^(l) . q_t)."""
    x = _inputs(B=2, T=10, H=2, d=4, L=3, random_S0=True)
    x = dict(x, alpha=np.ones_like(x["alpha"]), beta=np.zeros_like(x["beta"]))
    o, s = _fwd(x)
    ref = O.refine(O.shortconv(x["v"], x["conv"]), x["v"], x["Wk"], x["Wp"], x["wbeta"])
    for b in range(2):
        for h in range(2):
            for t in range(10):
                acc = x["S0"][b, h] @ x["q"][b, t, h]
                for s_ in range(t + 1):
                    for l in range(3):
                        acc = acc + ref["w"][l][b, s_, h] * np.dot(ref["kappa"][l][b, s_, h], x["q"][b, t, h])
                assert np.max(np.abs(acc - o[b, t, h])) < 1e-12


def test_injection_rank():
    """§2.1/§3: the refinement injection has rank <= L per token (and exactly L
    for generic inputs); with the Gated-DeltaNet base term the write has rank
    <= L + 1."""
    L = 3
    x = _inputs(B=1, T=12, H=2, d=6, L=L)
    inj = O.injection(x["v"], x["Wk"], x["Wp"], x["wbeta"], x["conv"])
    _, Bm = _write_and_forget(x)
    for t in range(4, 12):          # from t = 4 the conv window is full
        for h in range(2):
            s = np.linalg.svd(inj[0, t, h], compute_uv=False)
            assert s[L] / s[0] < 1e-12 and s[L - 1] / s[0] > 1e-6
            s = np.linalg.svd(Bm[0, t, h], compute_uv=False)
            assert s[L + 1] / s[0] < 1e-12 and s[L] / s[0] > 1e-6


# ---------------------------------------------------------------------------
# backward: central finite differences in float64
# ---------------------------------------------------------------------------
def _loss(x, dO, dST, L, **kw):
    o, s = _fwd(x, L=L, **kw)
    return float(np.sum(dO * o) + np.sum(dST * s))


@pytest.mark.parametrize("L,kw", [(0, {}), (1, {}), (2, {}),
                                  (2, {"activation": "identity"}),
                                  (2, {"conv_offset": 1}),
                                  (2, {"conv_offset": 1, "conv_hist": True}),
                                  (1, {"conv_hist": True})],
                         ids=["L0", "L1", "L2", "L2-identity", "L2-past-conv",
                              "L2-past-conv-history", "L1-history"])
def test_backward_matches_finite_differences(L, kw):
    x = make_inputs(1, 7, 2, 3, L, "f32", seed=11 + L, random_S0=True, with_dST=True)
    x = {k_: (None if v_ is None else v_.copy()) for k_, v_ in x.items()}
    kw = dict(kw)
    if kw.get("conv_hist"):
        x["conv_hist"] = np.random.default_rng(5).standard_normal((1, 4, 2, 3))
        kw["conv_hist"] = x["conv_hist"]          # the array FD perturbs in place
    dO, dST = x["dO"], x["dST"]
    args = dict(x)
    if L == 0:
        args.update(Wk=None, Wp=None, wbeta=None, conv=None)
    g = O.backward(args["q"], args["k"], args["v"], args["alpha"], args["beta"],
                   args["Wk"], args["Wp"], args["wbeta"], args["conv"], S0=args["S0"],
                   dO=dO, dST=dST, segment=3, **kw)
    names = {"q": "dq", "k": "dk", "v": "dv", "alpha": "dalpha", "beta": "dbeta", "S0": "dS0"}
    if L > 0:
        names.update(Wk="dWk", Wp="dWp", wbeta="dwbeta", conv="dconv")
    if "conv_hist" in kw:
        names.update(conv_hist="dconv_hist")
    h = 1e-6
    for name, gname in names.items():
        X = x[name]
        fd = np.zeros_like(X)
        for idx in np.ndindex(X.shape):
            old = X[idx]
            X[idx] = old + h
            fp = _loss(x, dO, dST, L, **kw)
            X[idx] = old - h
            fm = _loss(x, dO, dST, L, **kw)
            X[idx] = old
            fd[idx] = (fp - fm) / (2 * h)
        err = np.max(np.abs(fd - g[gname])) / max(1e-3, np.max(np.abs(fd)))
        assert err < 1e-6, (name, err)


def test_backward_segmenting_does_not_change_result():
    x = make_inputs(2, 13, 2, 4, 2, "f32", seed=3, random_S0=True, with_dST=True)
    gs = [O.backward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["Wk"], x["Wp"],
                     x["wbeta"], x["conv"], S0=x["S0"], dO=x["dO"], dST=x["dST"],
                     segment=seg) for seg in (1, 4, 64)]
    for key in gs[0]:
        for other in gs[1:]:
            assert np.max(np.abs(gs[0][key] - other[key])) < 1e-12, key


# ---------------------------------------------------------------------------
# continuation: S0 and the ShortConv history carry one call into the next
# ---------------------------------------------------------------------------
def _split_forward(x, cuts, **kw):
    """Run the oracle piece by piece, handing S_T and the conv history on."""
    W = [x[n] for n in ("Wk", "Wp", "wbeta", "conv")]
    S, hist, outs = x["S0"], None, []
    edges = [0] + list(cuts) + [x["q"].shape[1]]
    for a, b in zip(edges[:-1], edges[1:]):
        sl = lambda n: x[n][:, a:b]
        o, S = O.forward(sl("q"), sl("k"), sl("v"), sl("alpha"), sl("beta"), *W, S0=S,
                         conv_hist=hist, **kw)
        hist = O.conv_state(sl("v"), hist)
        outs.append(o)
    return np.concatenate(outs, axis=1), S, hist


@pytest.mark.parametrize("off", [0, 1])
@pytest.mark.parametrize("cuts", [(5,), (1, 2, 3), (2, 4, 6, 8, 10), (11,)])
def test_forward_continuation_is_exact(off, cuts):
    """Splitting a sequence anywhere (pieces shorter than the taps included)
    and carrying S and the last four values of v reproduces the whole run."""
    x = _inputs(B=2, T=12, H=2, d=4, L=2, seed=21, random_S0=True)
    W = [x[n] for n in ("Wk", "Wp", "wbeta", "conv")]
    o, S = O.forward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], *W, S0=x["S0"],
                     conv_offset=off)
    o2, S2, hist = _split_forward(x, cuts, conv_offset=off)
    assert np.max(np.abs(o2 - o)) < 1e-13 and np.max(np.abs(S2 - S)) < 1e-13
    assert np.array_equal(hist, x["v"][:, -4:])


def test_conv_state_of_short_pieces():
    v = np.arange(2 * 3 * 1 * 2, dtype=np.float64).reshape(2, 3, 1, 2) + 1
    h = O.conv_state(v)                      # zero history, 3 tokens: one zero row first
    assert np.all(h[:, 0] == 0) and np.array_equal(h[:, 1:], v)
    h2 = O.conv_state(v[:, :1], h)           # one more token shifts by one
    assert np.array_equal(h2[:, :3], h[:, 1:]) and np.array_equal(h2[:, 3], v[:, 0])


@pytest.mark.parametrize("off", [0, 1])
def test_backward_continuation_is_exact(off):
    """Gradients of a run split in two: the second piece's dS0 is the first
    piece's dST, its dconv_hist adds to dv of the first piece's last four
    tokens, and weight gradients add up; together they equal the whole run's."""
    T, T1 = 11, 6
    x = make_inputs(1, T, 2, 3, 2, "f32", seed=77, random_S0=True, with_dST=True)
    W = [x[n] for n in ("Wk", "Wp", "wbeta", "conv")]
    g = O.backward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], *W, S0=x["S0"], dO=x["dO"],
                   dST=x["dST"], conv_offset=off)
    p1 = {n: x[n][:, :T1] for n in ("q", "k", "v", "alpha", "beta", "dO")}
    p2 = {n: x[n][:, T1:] for n in ("q", "k", "v", "alpha", "beta", "dO")}
    _, S1 = O.forward(p1["q"], p1["k"], p1["v"], p1["alpha"], p1["beta"], *W, S0=x["S0"],
                      conv_offset=off)
    hist = O.conv_state(p1["v"])
    g2 = O.backward(p2["q"], p2["k"], p2["v"], p2["alpha"], p2["beta"], *W, S0=S1, dO=p2["dO"],
                    dST=x["dST"], conv_offset=off, conv_hist=hist)
    g1 = O.backward(p1["q"], p1["k"], p1["v"], p1["alpha"], p1["beta"], *W, S0=x["S0"],
                    dO=p1["dO"], dST=g2["dS0"], conv_offset=off)
    dv1 = g1["dv"].copy()
    dv1[:, T1 - 4:] += g2["dconv_hist"]
    cat = lambda n: np.concatenate([g1[n], g2[n]], axis=1)
    assert np.max(np.abs(np.concatenate([dv1, g2["dv"]], axis=1) - g["dv"])) < 1e-12
    for n in ("dq", "dk", "dalpha", "dbeta"):
        assert np.max(np.abs(cat(n) - g[n])) < 1e-12, n
    for n in ("dWk", "dWp", "dwbeta", "dconv"):
        assert np.max(np.abs(g1[n] + g2[n] - g[n])) < 1e-12, n
    assert np.max(np.abs(g1["dS0"] - g["dS0"])) < 1e-12
