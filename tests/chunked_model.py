"""Float64 numpy model of the chunked algorithm that the HIP kernels run.

Not the oracle: a design check.  The tests compare it with the token-by-token
oracle, which shows that the chunked algebra is an exact rearrangement of the
recurrence S_t = S_{t-1} A_t + B_t (PRISM summary §2.1) before any kernel
relies on it.  The update depends on the input only (§2.2, last paragraph), so
a chunk of C tokens acts on the state as one affine map

    S_next = exp(gC) S - S M + H,        O = O_loc + Qt S^T,

with everything on the right computed from the chunk's own inputs:

    g_t  = sum_{j<=t} log alpha_j,  Gam_ti = exp(g_t - g_i) (i <= t),
    D_t  = exp(gC - g_t),           e_t = exp(g_t),
    A    = diag(beta) (Gam * K K^T)_{i<t},  T = (I + A)^{-1},
    V'   = V - sum_l (Gam * K K_l^T)_{i<t} W_l,
    U    = T diag(beta) V',         Wk = T diag(beta e) K,
    M    = Wk^T diag(D) K,          H  = U^T diag(D) K + sum_l W_l^T diag(D) K_l,
    R0   = (Gam * Q K^T)_{i<=t},    R_l = (Gam * Q K_l^T)_{i<=t},
    Qt   = diag(e) Q - R0 Wk,       O_loc = R0 U + sum_l R_l W_l.

(K_l, W_l) are the refinement pairs (k^(l), beta^(l) delta^(l)) per token.
The reverse pass is the adjoint of these formulas, chunk by chunk.
"""

import numpy as np
from scipy.special import erf


# ----------------------------------------------------------------- refinement
def _gelu(z):
    return 0.5 * z * (1.0 + erf(z / np.sqrt(2.0)))


def _gelu_d(z):
    return 0.5 * (1.0 + erf(z / np.sqrt(2.0))) + z * np.exp(-0.5 * z * z) / np.sqrt(2 * np.pi)


def _sig(x):
    return 1.0 / (1.0 + np.exp(-x))


def refine_seq(v, conv, Wk, Wp, wb):
    """One sequence of one head.  v [T, d]; conv [d, 4]; Wk, Wp [L, d, d];
    wb [L, d].  Returns u, Kl [L, T, d], Wl [L, T, d] and the chain cache."""
    T, d = v.shape
    L = Wk.shape[0]
    u = np.zeros_like(v)
    for j in range(4):
        if j < T:
            u[j:] += conv[:, j] * v[: T - j]
    r = v - u
    Kl = np.zeros((L, T, d))
    Wl = np.zeros((L, T, d))
    cache = []
    for l in range(L):
        kap = u @ Wk[l].T
        p = u @ Wp[l].T
        gate = _sig(u @ wb[l])
        z = p * r
        dl = _gelu(z)
        Kl[l] = kap
        Wl[l] = gate[:, None] * dl
        cache.append((p, gate, r, z, dl))
        r = r - dl
    return u, Kl, Wl, cache


def refine_seq_bwd(v, conv, Wk, Wp, wb, u, cache, dKl, dWl, dv):
    """Adjoint of refine_seq; adds into dv and returns weight grads."""
    T, d = v.shape
    L = Wk.shape[0]
    dWk = np.zeros_like(Wk)
    dWp = np.zeros_like(Wp)
    dwb = np.zeros_like(wb)
    du = np.zeros_like(u)
    a = np.zeros_like(v)
    for l in range(L - 1, -1, -1):
        p, gate, r, z, dl = cache[l]
        dgate = np.sum(dl * dWl[l], axis=1)
        ddl = gate[:, None] * dWl[l] - a
        dz = ddl * _gelu_d(z)
        dp = dz * r
        a = a + dz * p
        dlog = dgate * gate * (1 - gate)
        dwb[l] = dlog @ u
        du += dlog[:, None] * wb[l][None, :]
        dWp[l] = dp.T @ u
        du += dp @ Wp[l]
        dWk[l] = dKl[l].T @ u
        du += dKl[l] @ Wk[l]
    dv = dv + a
    du = du - a
    dconv = np.zeros_like(conv)
    for j in range(4):
        if j < T:
            dconv[:, j] = np.sum(du[j:] * v[: T - j], axis=0)
            dv[: T - j] += conv[:, j] * du[j:]
    return dv, dWk, dWp, dwb, dconv


# ----------------------------------------------------------------- chunk maps
def chunk_fwd(Q, K, V, lg, beta, Kl, Wl):
    C = K.shape[0]
    L = Kl.shape[0]
    g = np.cumsum(lg)
    e = np.exp(g)
    gC = g[-1]
    D = np.exp(gC - g)
    incl = np.tril(np.ones((C, C)))
    strict = np.tril(np.ones((C, C)), -1)
    Gam = np.exp(g[:, None] - g[None, :]) * incl
    G0 = K @ K.T
    Y = Gam * G0 * strict
    A = beta[:, None] * Y
    T = np.linalg.inv(np.eye(C) + A)
    F = [Gam * strict * (K @ Kl[l].T) for l in range(L)]
    Vp = V - sum((F[l] @ Wl[l] for l in range(L)), np.zeros_like(V))
    U = T @ (beta[:, None] * Vp)
    Wk = T @ ((beta * e)[:, None] * K)
    M = Wk.T @ (D[:, None] * K)
    H = U.T @ (D[:, None] * K) + sum((Wl[l].T @ (D[:, None] * Kl[l]) for l in range(L)),
                                     np.zeros((V.shape[1], K.shape[1])))
    R0 = Gam * (Q @ K.T)
    R = [Gam * (Q @ Kl[l].T) for l in range(L)]
    Qt = e[:, None] * Q - R0 @ Wk
    Oloc = R0 @ U + sum((R[l] @ Wl[l] for l in range(L)), np.zeros_like(V))
    cache = dict(g=g, e=e, gC=gC, D=D, Gam=Gam, G0=G0, Y=Y, T=T, F=F, Vp=Vp, U=U,
                 Wk=Wk, R0=R0, R=R, strict=strict, incl=incl)
    return M, H, Qt, Oloc, cache


def chunk_bwd(Q, K, V, lg, beta, Kl, Wl, S, dSn, dO, c):
    """Adjoint of one chunk's map given S (state entering the chunk), dSn
    (adjoint of the state leaving it) and dO.  c is chunk_fwd's cache."""
    L = Kl.shape[0]
    g, e, gC, D, Gam = c["g"], c["e"], c["gC"], c["D"], c["Gam"]
    T, U, Wk, Vp, R0, R, F, Y = c["T"], c["U"], c["Wk"], c["Vp"], c["R0"], c["R"], c["F"], c["Y"]
    strict, incl = c["strict"], c["incl"]
    dQt = dO @ S
    dM = -S.T @ dSn
    dgC = np.exp(gC) * np.sum(S * dSn)
    # H and M (state side)
    KdS = K @ dSn.T
    dU = D[:, None] * KdS
    dK = D[:, None] * (U @ dSn)
    dD = np.sum(U * KdS, axis=1)
    dKl = np.zeros_like(Kl)
    dWl = np.zeros_like(Wl)
    for l in range(L):
        KldS = Kl[l] @ dSn.T
        dWl[l] = D[:, None] * KldS
        dKl[l] = D[:, None] * (Wl[l] @ dSn)
        dD += np.sum(Wl[l] * KldS, axis=1)
    KdM = K @ dM.T
    dWk = D[:, None] * KdM
    dK += D[:, None] * (Wk @ dM)
    dD += np.sum(Wk * KdM, axis=1)
    # Qt and O_loc
    dQ = e[:, None] * dQt
    de = np.sum(Q * dQt, axis=1)
    dR0 = -dQt @ Wk.T + dO @ U.T
    dWk += -R0.T @ dQt
    dU += R0.T @ dO
    dg = np.zeros_like(g)
    X = Gam * dR0
    dQ += X @ K
    dK += X.T @ Q
    P = dR0 * R0
    dg += P.sum(1) - P.sum(0)
    for l in range(L):
        dRl = dO @ Wl[l].T
        dWl[l] += R[l].T @ dO
        X = Gam * dRl
        dQ += X @ Kl[l]
        dKl[l] += X.T @ Q
        P = dRl * R[l]
        dg += P.sum(1) - P.sum(0)
    # solve: U = T diag(beta) V', Wk = T diag(beta e) K
    Bv = beta[:, None] * Vp
    Bk = (beta * e)[:, None] * K
    dT = dU @ Bv.T + dWk @ Bk.T
    X1 = T.T @ dU
    X2 = T.T @ dWk
    dVp = beta[:, None] * X1
    dbeta = np.sum(Vp * X1, axis=1) + e * np.sum(K * X2, axis=1)
    dK += (beta * e)[:, None] * X2
    de += beta * np.sum(K * X2, axis=1)
    dA = -(T.T @ dT @ T.T) * strict
    dbeta += np.sum(dA * Y, axis=1)
    dY = beta[:, None] * dA
    dG0 = Gam * dY
    P = dY * Y
    dg += P.sum(1) - P.sum(0)
    dK += (dG0 + dG0.T) @ K
    # fold: V' = V - sum_l F_l W_l
    dV = dVp.copy()
    for l in range(L):
        dWl[l] += -F[l].T @ dVp
        dF = -(dVp @ Wl[l].T) * strict
        dGl = Gam * dF
        dK += dGl @ Kl[l]
        dKl[l] += dGl.T @ K
        P = dF * F[l]
        dg += P.sum(1) - P.sum(0)
    dg += e * de
    dg -= D * dD
    dgC += np.sum(D * dD)
    dg[-1] += dgC
    dlg = np.cumsum(dg[::-1])[::-1]
    return dict(dQ=dQ, dK=dK, dV=dV, dlg=dlg, dbeta=dbeta, dKl=dKl, dWl=dWl)


# ----------------------------------------------------------------- whole layer
def _pad(x, Tp):
    out = np.zeros((Tp,) + x.shape[1:])
    out[: x.shape[0]] = x
    return out


def forward_backward(x, C, dST=None, backward=True):
    """x: dict of float64 arrays as from workloads.make_inputs.  Returns
    (o, S_T, grads-or-None) in the oracle's layouts."""
    q, k, v, al, be = x["q"], x["k"], x["v"], x["alpha"], x["beta"]
    B, T, H, d = k.shape
    L = 0 if x.get("Wk") is None else x["Wk"].shape[1]
    NC = -(-T // C)
    Tp = NC * C
    o = np.zeros_like(v)
    ST = np.zeros((B, H, d, d))
    grads = {n: np.zeros_like(x[m]) for n, m in
             (("dq", "q"), ("dk", "k"), ("dv", "v"), ("dalpha", "alpha"), ("dbeta", "beta"))}
    grads["dS0"] = np.zeros((B, H, d, d))
    if L > 0:
        for n, m in (("dWk", "Wk"), ("dWp", "Wp"), ("dwbeta", "wbeta"), ("dconv", "conv")):
            grads[n] = np.zeros_like(x[m])
    for b in range(B):
        for h in range(H):
            vs = v[b, :, h]
            if L > 0:
                u, Kl, Wl, rc = refine_seq(vs, x["conv"][h], x["Wk"][h], x["Wp"][h], x["wbeta"][h])
            else:
                Kl = np.zeros((0, T, d))
                Wl = np.zeros((0, T, d))
            Qp, Kp, Vp = _pad(q[b, :, h], Tp), _pad(k[b, :, h], Tp), _pad(vs, Tp)
            lg = _pad(np.log(al[b, :, h]), Tp)
            bp = _pad(be[b, :, h], Tp)
            Klp = np.stack([_pad(Kl[l], Tp) for l in range(L)]) if L else np.zeros((0, Tp, d))
            Wlp = np.stack([_pad(Wl[l], Tp) for l in range(L)]) if L else np.zeros((0, Tp, d))
            S = np.zeros((d, d)) if x.get("S0") is None else x["S0"][b, h].copy()
            sl = lambda c: slice(c * C, (c + 1) * C)
            maps, Ss = [], []
            for c in range(NC):
                s = sl(c)
                M, Hc, Qt, Oloc, cache = chunk_fwd(Qp[s], Kp[s], Vp[s], lg[s], bp[s], Klp[:, s], Wlp[:, s])
                Ss.append(S)
                maps.append((M, Qt, cache))
                o_c = Oloc + Qt @ S.T
                n_valid = min(C, T - c * C)
                o[b, c * C: c * C + n_valid, h] = o_c[:n_valid]
                S = np.exp(cache["gC"]) * S - S @ M + Hc
            ST[b, h] = S
            if not backward:
                continue
            dS = np.zeros((d, d)) if dST is None else dST[b, h].copy()
            dOp = _pad(x["dO"][b, :, h], Tp)
            dq = np.zeros((Tp, d)); dk = np.zeros((Tp, d)); dvv = np.zeros((Tp, d))
            dlg = np.zeros(Tp); dbe = np.zeros(Tp)
            dKl = np.zeros((L, Tp, d)); dWl = np.zeros((L, Tp, d))
            for c in range(NC - 1, -1, -1):
                s = sl(c)
                M, Qt, cache = maps[c]
                r = chunk_bwd(Qp[s], Kp[s], Vp[s], lg[s], bp[s], Klp[:, s], Wlp[:, s],
                              Ss[c], dS, dOp[s], cache)
                dq[s], dk[s], dvv[s], dlg[s], dbe[s] = r["dQ"], r["dK"], r["dV"], r["dlg"], r["dbeta"]
                dKl[:, s], dWl[:, s] = r["dKl"], r["dWl"]
                dS = np.exp(cache["gC"]) * dS - dS @ M.T + dOp[s].T @ Qt
            grads["dS0"][b, h] = dS
            grads["dq"][b, :, h] = dq[:T]
            grads["dk"][b, :, h] = dk[:T]
            grads["dalpha"][b, :, h] = dlg[:T] / al[b, :, h]
            grads["dbeta"][b, :, h] = dbe[:T]
            dv_seq = dvv[:T]
            if L > 0:
                dv_seq, dWk_, dWp_, dwb_, dconv_ = refine_seq_bwd(
                    vs, x["conv"][h], x["Wk"][h], x["Wp"][h], x["wbeta"][h], u, rc,
                    dKl[:, :T], dWl[:, :T], dv_seq)
                grads["dWk"][h] += dWk_
                grads["dWp"][h] += dWp_
                grads["dwbeta"][h] += dwb_
                grads["dconv"][h] += dconv_
            grads["dv"][b, :, h] = dv_seq
    return o, ST, (grads if backward else None)
