"""Oracle vs hand-derived closed forms (tests/golden/closed_form_cases.json).

Every expected number in the fixture was derived by hand from the definition
of softmax attention and its gradient; none was produced by code here.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden", "closed_form_cases.json")


def _arr(x):
    def conv(v):
        if isinstance(v, list):
            return [conv(u) for u in v]
        return -math.inf if v == "-inf" else float(v)
    return np.asarray(conv(x), dtype=np.float64)


with open(GOLD) as f:
    CASES = json.load(f)


@pytest.mark.parametrize("case", CASES["attention"], ids=lambda c: c["name"])
def test_forward_closed_form(case):
    q, k, v = _arr(case["q"]), _arr(case["k"]), _arr(case["v"])
    o, lse = oracle.forward(q, k, v, case["scale"], case["q_pos"],
                            case["k_pos"], case["causal"])
    np.testing.assert_allclose(o, _arr(case["o"]), rtol=0, atol=1e-14)
    exp = _arr(case["lse"])
    assert np.array_equal(np.isneginf(lse), np.isneginf(exp))
    fin = np.isfinite(exp)
    np.testing.assert_allclose(lse[fin], exp[fin], rtol=0, atol=1e-14)


@pytest.mark.parametrize("case", CASES["attention"], ids=lambda c: c["name"])
def test_backward_closed_form(case):
    q, k, v, do = (_arr(case[n]) for n in ("q", "k", "v", "do"))
    dq, dk, dv = oracle.backward(q, k, v, do, case["scale"], case["q_pos"],
                                 case["k_pos"], case["causal"])
    np.testing.assert_allclose(dq, _arr(case["dq"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(dk, _arr(case["dk"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(dv, _arr(case["dv"]), rtol=0, atol=1e-14)


@pytest.mark.parametrize("case", CASES["merge"], ids=lambda c: c["name"])
def test_merge_closed_form(case):
    parts = [(_arr(o)[None, :], _arr([l])) for o, l in case["parts"]]
    o, lse = oracle.merge(parts)
    np.testing.assert_allclose(o[0], _arr(case["o"]), rtol=0, atol=1e-14)
    exp = _arr([case["lse"]])
    if np.isneginf(exp[0]):
        assert np.isneginf(lse[0])
    else:
        np.testing.assert_allclose(lse, exp, rtol=0, atol=1e-14)
