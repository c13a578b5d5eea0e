"""Pins for the span policy and the closed-form bounds
(``verify_forward_amd.policy``; Copy-as-Decode §4.2 Table 2, §4.1 "Two
regimes.", appendix "Definition." and Table 17).

* Table 2's conservative bound bnd_m8 = T / (T_gen + T_copy / s(8)) is
  recomputed from the table's own T, T_copy, T_gen and s(8) = 6.79 for the
  four rows and must round to the printed 6.01 / 2.72 / 3.05 / 5.00
  (fixture ``tests/golden/cad_table2.txt``).
* Table 17's thresholds (strict 2, safe 4) follow from what the pages state
  about the 7B curve -- s(1) = 1 by definition, s(2) within 1.1..1.3 (§4.1
  "Two regimes."), s(8) = 6.79 (Table 2) -- read on the sweep's grid with the
  log-linear interpolation, at both ends of the stated band.
* Closed forms: for s(N) = N a splice costs one step, so a fixed cost c
  needs N > 1 + c / tau; for s(N) = 1 nothing pays; bnd_exact over spans
  that all sit at one measured point equals the uniform bound there.
"""
import math
import os

import pytest

from verify_forward_amd import policy as P

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "cad_table2.txt")


def _rows():
    out = []
    for line in open(GOLDEN):
        if line.strip() and not line.startswith("#"):
            name, T, Tc, Tg, s, b = line.split()
            out.append((name, int(T), int(Tc), int(Tg), float(s), float(b)))
    return out


def test_table2_conservative_bound():
    rows = _rows()
    assert len(rows) == 4
    for name, T, Tc, Tg, s, printed in rows:
        assert Tc + Tg == T, name
        assert round(P.bound_uniform(T, Tg, Tc, s), 2) == printed, name


@pytest.mark.parametrize("s2", [1.1, 1.3])
def test_table17_thresholds(s2):
    curve = {1: 1.0, 2: s2, 8: 6.79}
    grid = [1, 2, 4, 8]
    assert P.min_span(curve, candidates=grid) == 2
    assert P.min_span(curve, candidates=grid, s_floor=1.5) == 4
    # s(4) comes from the log-linear interpolation: the midpoint in log N
    assert math.isclose(P.s_at(curve, 4), (s2 + 6.79) / 2)


@pytest.mark.parametrize("c", [0.0, 0.5, 1.0, 2.5, 7.0])
def test_ideal_curve_closed_form(c):
    curve = {n: float(n) for n in range(1, 65)}
    want = math.floor(1 + c) + 1          # smallest integer N with N - 1 > c
    assert P.min_span(curve, c_over_tau=c) == want


def test_nothing_pays_without_speedup():
    assert P.min_span({1: 1.0, 64: 1.0}) is None
    assert P.min_span({1: 1.0, 64: 1.0}, s_floor=1.5) is None


def test_interpolation_holds_ends_and_hits_points():
    curve = {2: 1.5, 16: 9.0}
    assert P.s_at(curve, 1) == 1.5 and P.s_at(curve, 100) == 9.0
    assert P.s_at(curve, 2) == 1.5 and P.s_at(curve, 16) == 9.0
    assert math.isclose(P.s_at(curve, 4), 1.5 + (9.0 - 1.5) / 3)


def test_exact_bound_closed_forms():
    curve = {1: 1.0, 8: 6.79, 512: 90.5}
    assert math.isclose(P.bound_exact(0, [8], curve), 6.79)
    assert math.isclose(P.bound_exact(100, [8] * 50, curve), P.bound_uniform(500, 100, 400, 6.79))
    assert math.isclose(P.bound_exact(10, [], curve), 1.0)
    rep = P.policy_report(curve, c_ms=24.0, tau_ms=24.0)
    assert rep["strict"] == 8 and rep["safe"] == 8 and rep["with_fixed_cost"] == 8
