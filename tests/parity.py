"""Parity metrics shared by the GPU tests.

relerr(x, y) is the gate: max |x - y| / max |y| over the whole tensor (the
max-norm relative error; tolerances 1e-4 for fp32 storage, 2e-2 for bf16
storage with fp32 accumulation).  A max-norm gate can hide badly wrong
small-magnitude entries, so the value it returns also carries, as a
diagnostic, the 99.9th percentile of the elementwise relative error
|x_i - y_i| / |y_i| over the entries with y_i != 0 (attribute p999).  It is
printed next to the gate wherever the error is formatted ("2.1e-03 [p99.9
4.0e-03]") and is not itself a gate: near-zero y_i make single elementwise
ratios unbounded.
"""
import numpy as np


class RelErr(float):
    """The gate value (a float) with the elementwise 99.9th percentile."""

    def __new__(cls, value, p999):
        obj = super().__new__(cls, value)
        obj.p999 = p999
        return obj

    def __format__(self, spec):
        return f"{float(self):{spec}} [p99.9 {self.p999:.1e}]"


def p999(x, y):
    x = np.asarray(x, dtype=np.float64).ravel()
    y = np.asarray(y, dtype=np.float64).ravel()
    nz = y != 0
    if not np.any(nz):
        return 0.0
    return float(np.percentile(np.abs(x[nz] - y[nz]) / np.abs(y[nz]), 99.9))


def relerr(x, y):
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    gate = float(np.max(np.abs(x - y)) / max(np.max(np.abs(y)), 1e-30)) if y.size else 0.0
    return RelErr(gate, p999(x, y))
