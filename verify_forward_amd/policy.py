"""Copy-as-Decode's span policy and closed-form bounds from a measured s(N)
curve (Copy-as-Decode §4.2 Table 2's bounds; appendix "Definition." and
Table 17's minimum-span policy).

s(N) = T_AR(N) / T_PP(N): the time of N one-token decode steps over the
time of one splice of N tokens, measured at a set of span lengths.  Between
measured points s is interpolated linearly in log N (the pages'
"log-linear interpolation"; beyond the ends it is held at the end values).

Host arithmetic over measured numbers, used to report the policy and the
bounds next to the kernel measurements; no part of the decode path.
"""
from __future__ import annotations

import math
from typing import Dict, Iterable, Mapping, Optional, Sequence


def s_at(curve: Mapping[int, float], n: float) -> float:
    """s(n) from measured points {N: s(N)}, linear in log N between them."""
    pts = sorted((int(k), float(v)) for k, v in curve.items())
    if not pts:
        raise ValueError("empty s(N) curve")
    if n <= pts[0][0]:
        return pts[0][1]
    if n >= pts[-1][0]:
        return pts[-1][1]
    for (n0, s0), (n1, s1) in zip(pts, pts[1:]):
        if n0 <= n <= n1:
            t = (math.log(n) - math.log(n0)) / (math.log(n1) - math.log(n0))
            return s0 + t * (s1 - s0)
    raise AssertionError("unreachable")


def min_span(curve: Mapping[int, float], c_over_tau: float = 0.0, candidates: Optional[Iterable[int]] = None,
             s_floor: Optional[float] = None) -> Optional[int]:
    """The smallest span length N for which a splice pays: N*tau > N*tau/s(N)
    + c, i.e. N * (1 - 1/s(N)) > c / tau.  With ``s_floor`` instead, the
    smallest N with s(N) > s_floor (Table 17's safe threshold is 1.5).
    Candidates default to the measured span lengths from 2 up (the sweep's
    grid, as Table 17 reads them off the measured curve; a one-token splice
    is the decode step itself, s(1) = 1).  None if no candidate pays."""
    if candidates is None:
        candidates = sorted(int(k) for k in curve if int(k) >= 2)
    for n in candidates:
        s = s_at(curve, n)
        if s_floor is not None:
            if s > s_floor:
                return n
        elif n * (1.0 - 1.0 / s) > c_over_tau:
            return n
    return None


def bound_uniform(T: float, T_gen: float, T_copy: float, s: float) -> float:
    """Wall-clock speedup bound when every copied token is charged one
    speedup s: T / (T_gen + T_copy / s) (Table 2's bnd_m8 with s = s(8),
    bnd_Nbar with s = s(mean span))."""
    return T / (T_gen + T_copy / s)


def bound_exact(T_gen: float, spans: Sequence[int], curve: Mapping[int, float]) -> float:
    """Table 2's bnd_exact: T / (T_gen + sum_k N_k / s(N_k)) over the spans'
    lengths N_k, with T = T_gen + sum_k N_k."""
    T = T_gen + sum(spans)
    return T / (T_gen + sum(n / s_at(curve, n) for n in spans))


def policy_report(curve: Mapping[int, float], c_ms: Optional[float] = None,
                  tau_ms: Optional[float] = None) -> Dict[str, object]:
    """Table 17's two thresholds (strict: s > 1, i.e. c = 0; safe: s > 1.5)
    and, given a fixed cost c per copy op and the decode step tau, the
    smallest N that clears it."""
    rep: Dict[str, object] = {"strict": min_span(curve), "safe": min_span(curve, s_floor=1.5)}
    if c_ms is not None and tau_ms:
        rep["with_fixed_cost"] = min_span(curve, c_over_tau=c_ms / tau_ms)
        rep["c_over_tau"] = round(c_ms / tau_ms, 4)
    return rep
