"""The acceptance rule itself, exercised with mistakes planted in oracle
output on the CPU."""

import math

import numpy as np

import oracle as O
from tests.parity import parity_report, QUIET_CEIL


def _ref():
    rng = np.random.default_rng(11)
    x = rng.uniform(-0.5, 0.5, 160 * 40 + 240)
    x[2000:3000] = 0.0
    L, E = O.logmel_clip(x)
    return L, E


def test_rule_accepts_oracle_in_fp32():
    L, E = _ref()
    assert parity_report(L.astype(np.float32), L, E)["ok"]


def test_rule_rejects_loud_error():
    L, E = _ref()
    bad = L.copy()
    i = np.argwhere(E >= 1e-3)[0]
    bad[tuple(i)] += 2e-3
    rep = parity_report(bad, L, E)
    assert not rep["ok"] and rep["bad_loud"] == 1


def test_rule_rejects_quiet_too_high():
    L, E = _ref()
    bad = L.copy()
    i = np.argwhere(E < 1e-7)[0]
    bad[tuple(i)] = QUIET_CEIL + 0.01
    rep = parity_report(bad, L, E)
    assert not rep["ok"] and rep["bad_quiet"] == 1


def test_rule_rejects_nan():
    L, E = _ref()
    bad = L.copy()
    bad[3, 5] = np.nan
    assert not parity_report(bad, L, E)["ok"]


def test_rule_quiet_boundary():
    assert QUIET_CEIL == math.log(1e-7) + 1
    assert math.log(1e-10) < QUIET_CEIL
