"""Pass/fail criteria for GPU results against the fp64 oracle.

The accuracy bar is the one TransformerEngine PR 3527 ("cuDNN FROST
attention backend for head_dim in (256, 512]", Verification and the test
commits) applies: the error of the kernel against an fp64 reference must be
at most twice the error the reference itself incurs from reduced-precision
inputs, measured per case:

    err(gpu, true) <= 2 * err(naive, true)

where ``true`` is the oracle on the fp32 draws (promoted to fp64),
``naive`` is the oracle on the bf16-rounded inputs with its results stored
in the output dtype (a bf16 reference takes bf16 in and gives bf16 out;
for fp32 outputs nothing is rounded), and err is the maximum absolute
difference over real (non-padding, finite) elements.  Gradients must also
have relative L2 distance below 0.008 from the oracle on the kernel's own
inputs (PR 3510, "Add head-parallel FA4 backward for cuDNN CP attention",
Validation).  No absolute slack is added.  The ratio against the unrounded
naive reference is reported too ("ratio_in"), as a diagnostic.
"""
from __future__ import annotations

import os

import numpy as np

# Every passing check() of the session, for the one-line margin summary the
# test session prints at its end (tests/conftest.py): test id, output name,
# err / (2 floor), err / (2 unrounded floor), rel-L2.
RECORDS = []


def as64(x):
    import torch
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _mask(*arrs, mask=None):
    m = np.ones(arrs[0].shape, dtype=bool) if mask is None else np.asarray(mask, bool)
    for a in arrs:
        m = m & np.isfinite(a)
    return m


def max_err(a, b, mask=None):
    a, b = as64(a), as64(b)
    m = _mask(b, mask=mask)
    if not m.any():
        return 0.0
    d = np.abs(a[m] - b[m])
    return float(np.max(d)) if np.all(np.isfinite(d)) else float("inf")


def rel_l2(a, b, mask=None):
    a, b = as64(a), as64(b)
    m = _mask(b, mask=mask)
    num = np.linalg.norm((a - b)[m])
    den = np.linalg.norm(b[m])
    return float(num / den) if den > 0 else float(num)


def round_bf16(x):
    """Round to bfloat16 (nearest even) and return fp64."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(as64(x))).to(torch.bfloat16).double().numpy()


def round_fp16(x):
    """Round to IEEE half (nearest even) and return fp64."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(as64(x))).to(torch.float16).double().numpy()


def _ratio(err, floor):
    return err / (2 * floor) if floor > 0 else (0.0 if err == 0 else float("inf"))


def evaluate(gpu, true, naive, *, mask=None, grad=False, out_bf16=False):
    """Return a dict with err, floor, ratio (= err / (2*floor)), rel_l2 and
    pass flags.  ``out_bf16``: the kernel's output dtype is bf16 (True or
    "bf16") or fp16 ("fp16"), so the naive reference's results are stored
    in that type too."""
    g, t, n = as64(gpu), as64(true), as64(naive)
    n_out = round_fp16(n) if out_bf16 == "fp16" else (round_bf16(n) if out_bf16 else n)
    err = max_err(g, t, mask)
    floor = max_err(n_out, t, mask)
    res = {"err": err, "floor": floor, "ratio": _ratio(err, floor),
           "ratio_in": _ratio(err, max_err(n, t, mask)),
           "pass_floor": err <= 2 * floor}
    if grad:
        res["rel_l2"] = rel_l2(g, n, mask)
        res["pass_l2"] = res["rel_l2"] < 0.008
    return res


def passes(r):
    return r["pass_floor"] and r.get("pass_l2", True)


def _record(name, r):
    test = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0].split("::", 1)[-1]
    RECORDS.append((test, name, r["ratio"], r["ratio_in"], r.get("rel_l2")))


def check(name, gpu, true, naive, *, mask=None, grad=False, log=None, out_bf16=False):
    r = evaluate(gpu, true, naive, mask=mask, grad=grad, out_bf16=out_bf16)
    if log is not None:
        log[name] = r
    _record(name, r)
    assert r["pass_floor"], f"{name}: err {r['err']:.3e} > 2 x floor {r['floor']:.3e}"
    if grad:
        assert r["pass_l2"], f"{name}: rel L2 {r['rel_l2']:.4f} >= 0.008"
    return r


def summary():
    """Worst margins per test and output: {test: {output: [ratio, ratio_in,
    rel_l2]}} (ratio = err / (2 floor); a check passes at ratio <= 1)."""
    out = {}
    for test, name, ratio, ratio_in, l2 in RECORDS:
        cur = out.setdefault(test, {}).get(name)
        new = [round(ratio, 3), round(ratio_in, 3), None if l2 is None else round(l2, 5)]
        if cur is None:
            out[test][name] = new
        else:
            out[test][name] = [max(cur[0], new[0]), max(cur[1], new[1]),
                               None if l2 is None else max(cur[2] or 0, new[2])]
    return out


def check_lse(name, gpu, true, naive, *, mask=None, log=None):
    """LSE: -inf exactly where the oracle has -inf (keyless rows), the
    criterion on the finite entries, and |gpu - naive| <= 1e-4 (an O(1)
    error such as a wrong log base or scale is far above this)."""
    g, t, n = as64(gpu), as64(true), as64(naive)
    m = np.ones(t.shape, bool) if mask is None else np.asarray(mask, bool)
    assert np.array_equal(np.isneginf(g[m]), np.isneginf(t[m])), f"{name}: -inf rows differ"
    fin = m & np.isfinite(t)
    r = check(name, g, t, n, mask=fin, log=log)
    dev = max_err(g, n, fin)
    assert dev <= 1e-4, f"{name}: |lse - lse_naive| = {dev:.3e}"
    return r
