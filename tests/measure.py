"""Exact-by-bisection integration of a uniform-driven decision procedure.

The oracle's sampling steps are deterministic functions of supplied uniforms.
For a function f(u) of one uniform that is piecewise constant with each output
value on one interval of [0, 1), ``pieces`` recovers every interval by
bisection on the output alone, so the probability of each outcome is
measured without looking inside f.  Resolution is ``TOL`` per boundary.
"""
from __future__ import annotations

from collections import OrderedDict

TOL = 2.0 ** -44
TOP = 1.0 - 2.0 ** -53


def pieces(f):
    """Return OrderedDict value -> (length, representative u) for a function f
    on [0, 1) that is constant on consecutive intervals."""
    out = OrderedDict()
    u = 0.0
    v = f(u)
    while True:
        if f(TOP) == v:
            hi = 1.0
        else:
            lo, hi = u, TOP
            while hi - lo > TOL:
                mid = 0.5 * (lo + hi)
                if f(mid) == v:
                    lo = mid
                else:
                    hi = mid
        length = hi - u
        if v in out:
            raise AssertionError(f"value {v!r} occurs on two separate intervals")
        out[v] = (length, u + 0.5 * length)
        if hi >= 1.0:
            break
        u = hi
        v = f(u)
    return out


def probs(pc):
    return {k: ln for k, (ln, _) in pc.items()}
