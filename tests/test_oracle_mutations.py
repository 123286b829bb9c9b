"""The oracle's pins catch plausible mistakes.

Each case plants one mistake (a dropped term, a wrong sign, a transposed
operand, a wrong index, a different GELU) in a copy of the oracle's source,
loads that copy as a module, and runs every pin of test_oracle_pins.py
against it: at least one pin must fail on a value check (AssertionError).
The real oracle is never modified.  Each planted edit must match the source
exactly once, so a change to the oracle that moves an expression makes this
test fail loudly instead of silently testing nothing.
"""
import inspect
import itertools
import os
import types

import pytest

import tests.test_oracle_pins as PINS

ORACLE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                      "prism_oracle.py")

# (id, [(exact source text, replacement), ...])
MUTATIONS = [
    ("transposed-injection",
     [("S = S + w[:, :, None] * kap[:, None, :]", "S = S + kap[:, :, None] * w[:, None, :]")]),
    ("readout-on-previous-state",
     [("    Sk = np.einsum(\"nij,nj->ni\", S, k_t)\n",
       "    Sk = np.einsum(\"nij,nj->ni\", S, k_t)\n    S_prev = S\n"),
      ("o_t = np.einsum(\"nij,nj->ni\", S, q_t)", "o_t = np.einsum(\"nij,nj->ni\", S_prev, q_t)")]),
    ("residual-sign", [("    r = v - u\n", "    r = u - v\n")]),
    ("gate-sign", [("gate = sigmoid(np.einsum(\"hj,bthj->bth\", wbeta[:, l], u))",
                    "gate = sigmoid(-np.einsum(\"hj,bthj->bth\", wbeta[:, l], u))")]),
    ("transposed-Wk", [("kappa = np.einsum(\"hij,bthj->bthi\", Wk[:, l], u)",
                        "kappa = np.einsum(\"hji,bthj->bthi\", Wk[:, l], u)")]),
    ("reversed-taps", [("u[:, s:] += conv[None, None, :, :, j] * v[:, : T - s]",
                        "u[:, s:] += conv[None, None, :, :, W - 1 - j] * v[:, : T - s]")]),
    ("no-residual-update", [("        r = r - delta\n", "        r = r\n")]),
    ("no-base-write", [("    S = S + b_t[:, None, None] * v_t[:, :, None] * k_t[:, None, :]\n", "")]),
    ("misplaced-alpha",
     [("S = a_t[:, None, None] * (S - b_t[:, None, None] * Sk[:, :, None] * k_t[:, None, :])",
       "S = a_t[:, None, None] * S - b_t[:, None, None] * Sk[:, :, None] * k_t[:, None, :]")]),
    ("tanh-gelu", [("    return 0.5 * z * (1.0 + erf(z / _SQRT2))",
                    "    return 0.5 * z * (1.0 + np.tanh(0.7978845608028654 * (z + 0.044715 * z ** 3)))")]),
    ("gelu-grad-exponent", [("z * _INV_SQRT_2PI * np.exp(-0.5 * z * z)",
                             "z * _INV_SQRT_2PI * np.exp(-z * z)")]),
    ("dk-missing-term", [("dk_[t] = Gt_v - a_t * b_t * np.einsum(\"nij,ni->nj\", S_prev, y)",
                          "dk_[t] = Gt_v")]),
    ("dalpha-sign", [("da[t] = np.einsum(\"nij,nij->n\", G, S_prev) - bf[t] * xy",
                      "da[t] = np.einsum(\"nij,nij->n\", G, S_prev) + bf[t] * xy")]),
    ("dbeta-value-term", [("db[t] = -af[t] * xy + np.sum(vf[t] * y, axis=1)",
                           "db[t] = -af[t] * xy")]),
    ("conv-grad-index", [("dconv[:, :, j] += np.einsum(\"bthi,bthi->hi\", due[:, s:], ve[:, : Te - s])",
                          "dconv[:, :, j] += np.einsum(\"bthi,bthi->hi\", due[:, s:], ve[:, s:])")]),
    ("gain-grad-uses-next-residual", [("            dp = dz * ref[\"r\"][l]\n",
                                       "            dp = dz * (ref[\"r\"][l] - ref[\"delta\"][l])\n")]),
    ("state-grad-transposed", [("dq[t] = np.einsum(\"nij,ni->nj\", S_t, dOf[t])",
                                "dq[t] = np.einsum(\"nji,ni->nj\", S_t, dOf[t])")]),
]


def _mutant(edits):
    src = open(ORACLE).read()
    for old, new in edits:
        assert src.count(old) == 1, f"planted edit does not match the oracle exactly once: {old!r}"
        src = src.replace(old, new)
    mod = types.ModuleType("prism_oracle_mutant")
    mod.__file__ = ORACLE
    exec(compile(src, "prism_oracle_mutant", "exec"), mod.__dict__)
    return mod


def _pin_calls():
    """Every pin of test_oracle_pins with its parametrisations expanded."""
    calls = []
    for name, fn in inspect.getmembers(PINS, inspect.isfunction):
        if not name.startswith("test_"):
            continue
        marks = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
        grids = []
        for m in marks:
            names = m.args[0]
            names = [n.strip() for n in names.split(",")] if isinstance(names, str) else list(names)
            rows = []
            for val in m.args[1]:
                val = val.values if hasattr(val, "values") else val
                val = val if len(names) > 1 else (val,)
                rows.append(dict(zip(names, val)))
            grids.append(rows)
        for combo in itertools.product(*grids):
            kw = {}
            for part in combo:
                kw.update(part)
            calls.append((name, fn, kw))
    return calls


def test_pins_pass_on_the_oracle_itself():
    """Sanity: the unmodified source, loaded the same way, passes every pin."""
    saved = PINS.O
    PINS.O = _mutant([])
    try:
        for _, fn, kw in _pin_calls():
            fn(**kw)
    finally:
        PINS.O = saved


@pytest.mark.parametrize("edits", [m[1] for m in MUTATIONS], ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_fails_a_pin(edits):
    saved = PINS.O
    PINS.O = _mutant(edits)
    caught = []
    try:
        for name, fn, kw in _pin_calls():
            try:
                fn(**kw)
            except AssertionError:
                caught.append(name)
                break
    finally:
        PINS.O = saved
    assert caught, "no pin failed for this planted mistake"
