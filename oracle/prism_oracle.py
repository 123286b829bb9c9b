"""PRISM layer oracle: a plain, slow, float64, token-by-token CPU recurrence.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this module: only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` use it, to check and time the HIP library.  It shares no
code with the HIP path (no kernels, helpers, constants or pre/post-processing).

Source of the method: the web summary "Technical Summary: PRISM (Parallel
Residual Iterative Sequence Model)" (gist.science, paper 2602.10796, English
page, and its Dutch, Portuguese, German and Japanese translations).  Sections
cited below are the summary's own numbering:

* §2.1 "Write-Forget Decoupling":      S_t = S_{t-1} A_t + B_t, with the forget
  operator A_t of rank-1 Gated-DeltaNet form.
* §2.2 "Input-Anchored Loop Unrolling", Stage 1: a short convolution over the
  input gives the state-free anchor u_t (a proxy for S_{t-1} k_t).
* §2.2 Stage 2: for l = 1..L, direction k^(l) = W_k^(l) u, gain p^(l) = W_p^(l) u,
  residual step delta^(l) = GELU(p^(l) * r^(l)), r^(l+1) = r^(l) - delta^(l),
  step-size gate beta^(l); injection B_t = sum_l beta^(l) delta^(l) k^(l)^T.
* §3 item 3: with L = 0 the layer reduces to Gated DeltaNet.

Readings where the summary is silent or contradicts itself (binding here and
in the kernels; each is listed with its reason in the design notes):

* R1  The write keeps the Gated-DeltaNet base term:
      B_t = beta_t v_t k_t^T + sum_l beta_t^(l) delta_t^(l) k_t^(l)^T.
      Without it L = 0 would not be Gated DeltaNet (§3 item 3).
* R2  ShortConv: depthwise, causal, width 4, over v, tap j multiplies
      v_{t-j} (j = 0 is the current token), zero history before t = 1,
      no bias, no activation.  conv_offset = 1 selects the strictly-past
      variant, tap j multiplying v_{t-1-j} (the anchor then only sees tokens
      the state S_{t-1} has seen).  A call may continue an earlier one: then
      the four values before the sequence come in as ``conv_hist`` instead of
      zeros, as S0 carries the state.
* R3  r^(1) = v_t - u_t.
* R4  beta_t^(l) = sigmoid(w_beta^(l) . u_t), one scalar per token, head, step.
* R5  GELU is the exact erf form z * Phi(z).
* R6  W_k^(l) is d_k x d_v, W_p^(l) is d_v x d_v, separate per head and step.
* R7  Readout o_t = S_t q_t with the post-update state, no scale.
* R8  A_t = alpha_t (I - beta_t k_t k_t^T); q, k are used as given.

Array layouts (all float64 numpy arrays):
  q, k        [B, T, H, dk]        v        [B, T, H, dv]
  alpha, beta [B, T, H]            S0, S_T  [B, H, dv, dk]
  Wk          [H, L, dk, dv]       Wp       [H, L, dv, dv]
  wbeta       [H, L, dv]           conv     [H, dv, W]   (W = 4)
  conv_hist   [B, 4, H, dv]        (v_{-4} .. v_{-1}, v's own layout)
"""

import math

import numpy as np
from scipy.special import erf

_SQRT2 = math.sqrt(2.0)
_INV_SQRT_2PI = 1.0 / math.sqrt(2.0 * math.pi)


# ---------------------------------------------------------------------------
# elementwise pieces
# ---------------------------------------------------------------------------
def gelu(z):
    """Exact GELU, z * Phi(z) (reading R5; §2.2 Stage 2 "Residual Update")."""
    return 0.5 * z * (1.0 + erf(z / _SQRT2))


def gelu_grad(z):
    """d/dz [z Phi(z)] = Phi(z) + z phi(z)."""
    return 0.5 * (1.0 + erf(z / _SQRT2)) + z * _INV_SQRT_2PI * np.exp(-0.5 * z * z)


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _activation(name):
    if name == "gelu":
        return gelu, gelu_grad
    if name == "identity":  # the "no GELU" ablation of §4, used only as a pin
        return (lambda z: z), (lambda z: np.ones_like(z))
    raise ValueError(f"unknown activation {name!r}")


# ---------------------------------------------------------------------------
# Stage 1: ShortConv anchor (§2.2 Stage 1; reading R2)
# ---------------------------------------------------------------------------
def shortconv(v, conv, conv_offset=0, hist=None):
    """u_t = sum_j conv[:, :, j] * v_{t-o-j} (o = conv_offset).  Before the
    sequence v_s is zero, or, with ``hist`` [B, 4, H, dv], the four values
    v_{-4} .. v_{-1} that preceded it (oldest first)."""
    if hist is not None:
        ext = np.concatenate([hist, v], axis=1)
        return shortconv(ext, conv, conv_offset)[:, hist.shape[1]:]
    B, T, H, dv = v.shape
    W = conv.shape[-1]
    u = np.zeros_like(v)
    for j in range(W):
        s = j + conv_offset
        if s < T:
            u[:, s:] += conv[None, None, :, :, j] * v[:, : T - s]
    return u


# ---------------------------------------------------------------------------
# Stage 2: L refinement steps (§2.2 Stage 2; readings R3, R4, R6)
# ---------------------------------------------------------------------------
def refine(u, v, Wk, Wp, wbeta, activation="gelu"):
    """Per-token refinement.  Depends on the input only, never on the state.

    Returns a dict of per-step lists (length L), each entry [B, T, H, *]:
      kappa  k^(l) = W_k^(l) u           (direction)
      p      p^(l) = W_p^(l) u           (gain)
      gate   beta^(l) = sigmoid(w_beta^(l) . u)   [B, T, H]
      r      r^(l)  (residual entering step l; r^(1) = v - u)
      z      p^(l) * r^(l)
      delta  act(z)
      w      beta^(l) delta^(l)          (value of the l-th injected pair)
    """
    act, _ = _activation(activation)
    L = Wk.shape[1] if Wk is not None else 0
    out = {key: [] for key in ("kappa", "p", "gate", "r", "z", "delta", "w")}
    r = v - u
    for l in range(L):
        kappa = np.einsum("hij,bthj->bthi", Wk[:, l], u)
        p = np.einsum("hij,bthj->bthi", Wp[:, l], u)
        gate = sigmoid(np.einsum("hj,bthj->bth", wbeta[:, l], u))
        z = p * r
        delta = act(z)
        w = gate[..., None] * delta
        for key, val in (("kappa", kappa), ("p", p), ("gate", gate), ("r", r),
                         ("z", z), ("delta", delta), ("w", w)):
            out[key].append(val)
        r = r - delta
    return out


# ---------------------------------------------------------------------------
# the state recurrence (§2.1; readings R1, R7, R8)
# ---------------------------------------------------------------------------
def _step(S, q_t, k_t, v_t, a_t, b_t, kap_t, w_t):
    """One token: S <- S A_t + B_t, then o_t = S q_t.

    S [N, dv, dk]; q_t, k_t [N, dk]; v_t [N, dv]; a_t, b_t [N];
    kap_t, w_t lists over l of [N, dk] / [N, dv].
    S A_t = alpha (S - beta (S k) k^T) is S times alpha (I - beta k k^T).
    """
    Sk = np.einsum("nij,nj->ni", S, k_t)
    S = a_t[:, None, None] * (S - b_t[:, None, None] * Sk[:, :, None] * k_t[:, None, :])
    S = S + b_t[:, None, None] * v_t[:, :, None] * k_t[:, None, :]
    for kap, w in zip(kap_t, w_t):
        S = S + w[:, :, None] * kap[:, None, :]
    o_t = np.einsum("nij,nj->ni", S, q_t)
    return S, o_t


def _flat(x):
    """[B, T, H, ...] -> [T, B*H, ...] so that the loop runs over t."""
    B, T, H = x.shape[:3]
    x = np.moveaxis(x, 1, 0)
    return x.reshape((T, B * H) + x.shape[3:])


def _unflat(x, B, H):
    """[T, B*H, ...] -> [B, T, H, ...]."""
    T = x.shape[0]
    return np.moveaxis(x.reshape((T, B, H) + x.shape[2:]), 0, 1)


def conv_state(v, hist=None):
    """The ShortConv history after the sequence: the last four values of
    (hist or zeros) followed by v, [B, 4, H, dv], oldest first."""
    B, T, H, dv = v.shape
    h = np.zeros((B, 4, H, dv)) if hist is None else hist
    return np.concatenate([h, v], axis=1)[:, -4:]


def forward(q, k, v, alpha, beta, Wk=None, Wp=None, wbeta=None, conv=None,
            S0=None, activation="gelu", return_states=False, conv_offset=0, conv_hist=None):
    """The PRISM layer, token by token.  Returns (o [B,T,H,dv], S_T [B,H,dv,dk]).

    With ``return_states`` also returns S_1..S_T as [B, T, H, dv, dk].
    L = Wk.shape[1]; L = 0 (or Wk None) means no refinement pairs.
    """
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    L = 0 if Wk is None else Wk.shape[1]
    if L > 0:
        u = shortconv(v, conv, conv_offset, conv_hist)
        ref = refine(u, v, Wk, Wp, wbeta, activation)
        kap = [_flat(x) for x in ref["kappa"]]
        w = [_flat(x) for x in ref["w"]]
    else:
        kap, w = [], []
    qf, kf, vf = _flat(q), _flat(k), _flat(v)
    af, bf = _flat(alpha), _flat(beta)
    S = np.zeros((B * H, dv, dk)) if S0 is None else S0.reshape(B * H, dv, dk).copy()
    o = np.zeros((T, B * H, dv))
    states = np.zeros((T, B * H, dv, dk)) if return_states else None
    for t in range(T):
        S, o[t] = _step(S, qf[t], kf[t], vf[t], af[t], bf[t],
                        [x[t] for x in kap], [x[t] for x in w])
        if return_states:
            states[t] = S
    out = (_unflat(o, B, H), S.reshape(B, H, dv, dk))
    if return_states:
        out = out + (_unflat(states, B, H),)
    return out


def injection(v, Wk, Wp, wbeta, conv, activation="gelu", conv_offset=0):
    """The refinement part of the write, sum_l beta^(l) delta^(l) k^(l)^T,
    materialised per token: [B, T, H, dv, dk] (§2.2, final injection matrix)."""
    u = shortconv(v, conv, conv_offset)
    ref = refine(u, v, Wk, Wp, wbeta, activation)
    dv, dk = v.shape[-1], Wk.shape[2]
    out = np.zeros(v.shape[:3] + (dv, dk))
    for kap, w in zip(ref["kappa"], ref["w"]):
        out += w[..., :, None] * kap[..., None, :]
    return out


# ---------------------------------------------------------------------------
# backward: the adjoint of forward(), token by token in reverse
# ---------------------------------------------------------------------------
def backward(q, k, v, alpha, beta, Wk=None, Wp=None, wbeta=None, conv=None,
             S0=None, dO=None, dST=None, activation="gelu", segment=64, conv_offset=0,
             conv_hist=None):
    """Gradients of  <dO, o> + <dST, S_T>  with respect to every input.

    The reverse pass needs S_{t-1} and S_t at each t.  States are recomputed
    segment by segment from snapshots taken every ``segment`` tokens, so
    memory stays at (T/segment + segment) states per sequence.

    Returns a dict with dq, dk, dv, dalpha, dbeta, dS0 and, when L > 0,
    dWk, dWp, dwbeta, dconv (same shapes as the inputs), and dconv_hist when
    ``conv_hist`` is given.
    """
    B, T, H, dk = k.shape
    dv_ = v.shape[-1]
    N = B * H
    L = 0 if Wk is None else Wk.shape[1]
    act, act_grad = _activation(activation)

    if L > 0:
        u = shortconv(v, conv, conv_offset, conv_hist)
        ref = refine(u, v, Wk, Wp, wbeta, activation)
        kap = [_flat(x) for x in ref["kappa"]]
        w = [_flat(x) for x in ref["w"]]
    else:
        kap, w = [], []
    qf, kf, vf = _flat(q), _flat(k), _flat(v)
    af, bf = _flat(alpha), _flat(beta)
    dOf = np.zeros((T, N, dv_)) if dO is None else _flat(dO)

    # forward sweep: keep a snapshot at the start of every segment
    S = np.zeros((N, dv_, dk)) if S0 is None else S0.reshape(N, dv_, dk).copy()
    snaps = {}
    for t in range(T):
        if t % segment == 0:
            snaps[t] = S.copy()
        S, _ = _step(S, qf[t], kf[t], vf[t], af[t], bf[t],
                     [x[t] for x in kap], [x[t] for x in w])

    G = np.zeros((N, dv_, dk)) if dST is None else dST.reshape(N, dv_, dk).copy()
    dq = np.zeros_like(qf)
    dk_ = np.zeros_like(kf)
    dvv = np.zeros_like(vf)
    da = np.zeros_like(af)
    db = np.zeros_like(bf)
    dkap = [np.zeros_like(x) for x in kap]
    dw = [np.zeros_like(x) for x in w]

    for s0 in sorted(snaps, reverse=True):
        s1 = min(s0 + segment, T)
        # recompute S_{s0} .. S_{s1} inside the segment; seg[i] = S before token s0+i
        seg = [snaps[s0]]
        for t in range(s0, s1):
            Sn, _ = _step(seg[-1], qf[t], kf[t], vf[t], af[t], bf[t],
                          [x[t] for x in kap], [x[t] for x in w])
            seg.append(Sn)
        for t in range(s1 - 1, s0 - 1, -1):
            S_prev, S_t = seg[t - s0], seg[t - s0 + 1]
            a_t, b_t = af[t][:, None], bf[t][:, None]
            # o_t = S_t q_t
            G = G + dOf[t][:, :, None] * qf[t][:, None, :]
            dq[t] = np.einsum("nij,ni->nj", S_t, dOf[t])
            x = np.einsum("nij,nj->ni", S_prev, kf[t])          # S_{t-1} k_t
            y = np.einsum("nij,nj->ni", G, kf[t])               # G k_t
            xy = np.sum(x * y, axis=1)
            da[t] = np.einsum("nij,nij->n", G, S_prev) - bf[t] * xy
            db[t] = -af[t] * xy + np.sum(vf[t] * y, axis=1)
            dvv[t] += b_t * y
            Gt_v = np.einsum("nij,ni->nj", G, b_t * vf[t] - a_t * b_t * x)
            dk_[t] = Gt_v - a_t * b_t * np.einsum("nij,ni->nj", S_prev, y)
            for l in range(L):
                dw[l][t] = np.einsum("nij,nj->ni", G, kap[l][t])
                dkap[l][t] = np.einsum("nij,ni->nj", G, w[l][t])
            # G <- G A_t
            G = af[t][:, None, None] * (G - bf[t][:, None, None] * y[:, :, None] * kf[t][:, None, :])

    grads = {
        "dq": _unflat(dq, B, H), "dk": _unflat(dk_, B, H),
        "dalpha": _unflat(da, B, H), "dbeta": _unflat(db, B, H),
        "dS0": G.reshape(B, H, dv_, dk),
    }
    dv_full = _unflat(dvv, B, H)

    if L > 0:
        dkap_b = [_unflat(x, B, H) for x in dkap]
        dw_b = [_unflat(x, B, H) for x in dw]
        dWk = np.zeros_like(Wk)
        dWp = np.zeros_like(Wp)
        dwbeta = np.zeros_like(wbeta)
        du = np.zeros_like(u)
        a = np.zeros_like(v)                       # d loss / d r^(l+1)
        for l in range(L - 1, -1, -1):
            gate = ref["gate"][l]
            dgate = np.sum(ref["delta"][l] * dw_b[l], axis=-1)
            ddelta = gate[..., None] * dw_b[l] - a
            dz = ddelta * act_grad(ref["z"][l])
            dp = dz * ref["r"][l]
            a = a + dz * ref["p"][l]
            dlogit = dgate * gate * (1.0 - gate)
            dwbeta[:, l] += np.einsum("bth,bthj->hj", dlogit, u)
            du += dlogit[..., None] * wbeta[None, None, :, l]
            dWp[:, l] += np.einsum("bthi,bthj->hij", dp, u)
            du += np.einsum("hij,bthi->bthj", Wp[:, l], dp)
            dWk[:, l] += np.einsum("bthi,bthj->hij", dkap_b[l], u)
            du += np.einsum("hij,bthi->bthj", Wk[:, l], dkap_b[l])
        dv_full = dv_full + a
        du = du - a
        # ShortConv: u_t = sum_j c_j * v_{t-o-j}, over the history (zeros
        # without one) followed by the sequence
        hist = np.zeros((B, 4, H, dv_)) if conv_hist is None else conv_hist
        ve = np.concatenate([hist, v], axis=1)
        due = np.concatenate([np.zeros_like(hist), du], axis=1)
        dve = np.zeros_like(ve)
        Te = T + 4
        dconv = np.zeros_like(conv)
        for j in range(conv.shape[-1]):
            s = j + conv_offset
            if s < Te:
                dconv[:, :, j] += np.einsum("bthi,bthi->hi", due[:, s:], ve[:, : Te - s])
                dve[:, : Te - s] += conv[None, None, :, :, j] * due[:, s:]
        dv_full = dv_full + dve[:, 4:]
        if conv_hist is not None:
            grads["dconv_hist"] = dve[:, :4]
        grads.update(dWk=dWk, dWp=dWp, dwbeta=dwbeta, dconv=dconv)
    grads["dv"] = dv_full
    return grads
