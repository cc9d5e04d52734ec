"""Pins of the per-layer budget schedules (oracle/schedule.py) and host
parity of kvc_layer_budgets against them (no GPU needed).

Pins: hand-worked values (tests/golden/layer_budgets.json), the closed-form
endpoints of each schedule, monotonicity in the direction each page states,
and the special case r = 1 (every layer keeps the whole base).
"""
import json
import os

import pytest

import oracle
from oracle.schedule import LINEAR, QUADRATIC, layer_budgets

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "layer_budgets.json")


def test_golden_values():
    for case in json.load(open(GOLDEN))["cases"]:
        sched = LINEAR if case["schedule"] == "linear" else QUADRATIC
        got = layer_budgets(sched, case["num_layers"], case["base"], case["base_ratio"])
        if "budgets" in case:
            assert got == case["budgets"], case
        else:
            assert [got[i] for i in case["layers"]] == case["budgets_at_layers"], case


@pytest.mark.parametrize("n,base", [(1, 7), (32, 8192), (80, 131072), (7, 1000)])
def test_linear_endpoints_and_direction(n, base):
    b = layer_budgets(LINEAR, n, base)
    assert b[0] == base                              # the first layer keeps everything
    assert all(x >= y for x, y in zip(b, b[1:]))     # shallow layers keep more
    last = base * (0.2 + 0.8 / n)                    # ratio of the last layer, 1 - 0.8 (n - 1) / n
    assert abs(b[-1] - last) <= 1.0 + 1e-9 * base


@pytest.mark.parametrize("n,base,r", [(32, 8192, 0.2), (80, 131072, 0.5), (5, 100, 0.0)])
def test_quadratic_endpoints_and_direction(n, base, r):
    b = layer_budgets(QUADRATIC, n, base, r)
    assert b[0] == int(base * r)                     # the first layer keeps the base ratio
    assert all(x <= y for x, y in zip(b, b[1:]))     # deep layers keep more
    if n % 2 == 0:                                   # halfway: r + (1 - r) / 4
        assert abs(b[n // 2] - base * (r + (1 - r) / 4)) <= 1.0


def test_quadratic_full_ratio_keeps_everything():
    assert layer_budgets(QUADRATIC, 16, 4096, 1.0) == [4096] * 16


def test_min_budget_floor_and_errors():
    assert min(layer_budgets(LINEAR, 32, 1000, min_budget=600)) == 600
    with pytest.raises(ValueError):
        layer_budgets(QUADRATIC, 4, 100, 1.5)
    with pytest.raises(ValueError):
        layer_budgets(7, 4, 100)
    assert oracle.layer_budgets is layer_budgets


kvc = pytest.importorskip("compressed_kv_cache_kvc_amd")


@pytest.mark.parametrize("sched", [LINEAR, QUADRATIC])
def test_library_matches_oracle(sched):
    """kvc_layer_budgets (host C) equals the oracle integer for integer."""
    for n in (1, 2, 3, 4, 5, 7, 12, 32, 40, 61, 80, 126):
        for base in (1, 100, 512, 2457, 8192, 32768, 131072, 1 << 30):
            for r in ((0.0,) if sched == LINEAR else (0.0, 0.1, 0.2, 0.25, 0.3, 1 / 3, 0.5, 0.9, 1.0)):
                for mb in (0, 1028):
                    assert kvc.kvc_layer_budgets(sched, n, base, r, mb) == layer_budgets(sched, n, base, r, mb), \
                        (sched, n, base, r, mb)


def test_library_validation():
    with pytest.raises(kvc.KvcError):
        kvc.kvc_layer_budgets(2, 4, 100)
    with pytest.raises(kvc.KvcError):
        kvc.kvc_layer_budgets(QUADRATIC, 4, 100, 1.5)
    with pytest.raises(kvc.KvcError):
        kvc.kvc_layer_budgets(LINEAR, 0, 100)
    with pytest.raises(kvc.KvcError):
        kvc.kvc_layer_budgets(LINEAR, 4, 0)
