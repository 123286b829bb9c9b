"""Seeded synthetic inputs for the PRISM layer, and the workload shapes.

This module draws random numbers and rounds them to the storage dtype.  It
holds none of the layer's arithmetic, so both the oracle-side tests and the
HIP path can take their inputs from it.

Distributions (second argument of N(., .) is the variance):
  q, k            N(0, 1), then L2-normalised per (token, head), then rounded
  v               N(0, 1)
  alpha           sigmoid(N(2, 0.5))           (forget gate, fp32)
  beta            sigmoid(N(0, 1))             (delta-rule step, fp32)
  W_k^(l), W_p^(l), w_beta^(l)   N(0, 1/d)     (per head, per step)
  conv taps       N(0, 1/4)
  S0              0 (or N(0, 1) when requested)
  dO              N(0, 1);  dST N(0, 1) when requested
Draw order is fixed: q, k, v, alpha-logits, beta-logits, Wk, Wp, wbeta,
taps, dO, dST, S0.  Values are rounded (round-to-nearest-even) to the
storage dtype and returned as float64 arrays that hold exactly those values.
"""

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str          # "f32" or "bf16": storage type of q, k, v, o, weights, taps
    B: int
    T: int
    H: int
    d: int              # d_k = d_v
    L: int
    chunk: int
    backward: bool

    @property
    def tokens(self):
        return self.B * self.T

    @property
    def token_heads(self):
        return self.B * self.T * self.H


def workloads():
    """The shapes the layer is checked and measured on.

    tiny-fp32     : B=1, H=1, T=64, d=16, L=2, chunk 16, fp32, forward.
    recsys-T200   : B=64, H=4, T=200, d=64, L=2, chunk 64, bf16, forward
                    (sequential-recommendation shape, ragged last chunk).
    lm-T2048      : B=8, H=16, T=2048, d=128, L=3, chunk 64, bf16, fwd+bwd.
    long-T{2K..16K}: B=16384/T, H=16, d=128, L=3, chunk 64, bf16, fwd+bwd.
    depth-L{0..8} : B=4, H=16, T=4096, d=128, chunk 64, bf16, fwd+bwd.
    """
    out = [
        Workload("tiny-fp32", "f32", 1, 64, 1, 16, 2, 16, True),
        Workload("recsys-T200", "bf16", 64, 200, 4, 64, 2, 64, False),
        Workload("lm-T2048", "bf16", 8, 2048, 16, 128, 3, 64, True),
    ]
    for T in (2048, 4096, 8192, 16384):
        out.append(Workload(f"long-T{T}", "bf16", 16384 // T, T, 16, 128, 3, 64, True))
    for L in (0, 1, 2, 4, 8):
        out.append(Workload(f"depth-L{L}", "bf16", 4, 4096, 16, 128, L, 64, True))
    return {w.name: w for w in out}


def round_to(x, dtype):
    """Round float64 values to the storage dtype (RNE) and back to float64."""
    f = np.asarray(x, dtype=np.float32)
    if dtype == "f32":
        return f.astype(np.float64)
    if dtype != "bf16":
        raise ValueError(dtype)
    bits = f.view(np.uint32)
    # finite inputs only (the generator draws no inf / nan): no overflow in uint32
    bits = (bits + np.uint32(0x7FFF) + ((bits >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return bits.view(np.float32).astype(np.float64)


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def make_inputs(B, T, H, d, L, dtype="bf16", seed=0, alpha_logit_mean=2.0,
                random_S0=False, with_dST=False):
    """Draw one batch.  Returns a dict of float64 arrays (exact storage values).

    Keys: q, k, v [B,T,H,d]; alpha, beta [B,T,H] (fp32-exact);
    Wk, Wp [H,L,d,d]; wbeta [H,L,d]; conv [H,d,4]; dO [B,T,H,d];
    S0 [B,H,d,d] or None; dST [B,H,d,d] or None.
    """
    rng = np.random.default_rng(seed)
    shape = (B, T, H, d)
    q = rng.standard_normal(shape)
    k = rng.standard_normal(shape)
    v = rng.standard_normal(shape)
    q /= np.sqrt(np.einsum("...i,...i->...", q, q))[..., None]
    k /= np.sqrt(np.einsum("...i,...i->...", k, k))[..., None]
    a_logit = alpha_logit_mean + np.sqrt(0.5) * rng.standard_normal((B, T, H))
    b_logit = rng.standard_normal((B, T, H))
    s = 1.0 / np.sqrt(d)
    Wk = s * rng.standard_normal((H, L, d, d))
    Wp = s * rng.standard_normal((H, L, d, d))
    wbeta = s * rng.standard_normal((H, L, d))
    conv = 0.5 * rng.standard_normal((H, d, 4))
    dO = rng.standard_normal(shape)
    dST = rng.standard_normal((B, H, d, d)) if with_dST else None
    S0 = rng.standard_normal((B, H, d, d)) if random_S0 else None
    r = lambda x: None if x is None else round_to(x, dtype)
    f32 = lambda x: None if x is None else round_to(x, "f32")
    return {
        "q": r(q), "k": r(k), "v": r(v),
        "alpha": f32(_sigmoid(a_logit)), "beta": f32(_sigmoid(b_logit)),
        "Wk": r(Wk), "Wp": r(Wp), "wbeta": r(wbeta), "conv": r(conv),
        "dO": r(dO), "dST": f32(dST), "S0": f32(S0),
    }


def make_workload_inputs(w, seed=0, **kw):
    return make_inputs(w.B, w.T, w.H, w.d, w.L, w.dtype, seed, **kw)
