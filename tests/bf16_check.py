"""Parity of the chunk path in bf16 mode, split at the hidden state.

In bf16 mode the hidden state h = silu(W_g x) * (W_u x) is rounded to a bf16
code before the down projection.  That code is an integer decided by floating
point: the GPU decides it from g and u accumulated in fp32 on the matrix
cores, the oracle from the same quantities in fp64.  Where the exact h lies
within the accumulation error of the midpoint between two bf16 neighbours,
either neighbour is a correct code, and one flipped code of a large h moves
a whole output row by w * W_d[:, r] * (code spacing), which can reach the
1e-3 row bar on its own.  So, as for the routing ids, the check compares what
is unique and checks the rest for validity:

 1. every hidden code the GPU wrote is the bf16 rounding of a value within
    TAU * max_r |h_r| of the exact h (the oracle's fp64 value), that is
    |code - h| <= spacing(h) / 2 + TAU * max |h| per element: the GPU's g and u
    are fp32 sums of d/32 matrix-core partial products, whose rounding error
    is at most about gamma_{d/32} * sum |w x| (about 2^-15 of the largest h of
    a row at d_model 2048), so TAU = 2^-14; codes that differ from the
    oracle's are counted as flips (a wrong row, weight or token is off by far
    more: its h is unrelated);
 2. y equals, within the 1e-3 row bar, the oracle's down projection and
    weighted combine (fp64) of the GPU's own hidden codes;
 3. end to end, y against the oracle's y is reported with the element-wise
    statistics; it differs from 2 exactly by the flipped codes' terms.

The oracle is called only through oracle/; nothing here computes the method.
"""
from __future__ import annotations

import numpy as np

import oracle

TAU = 2.0 ** -14  # of the row's largest |h|


def _spacing(v: np.ndarray) -> np.ndarray:
    """Distance between the two bf16 values around each v (v exact in fp64)."""
    a = np.maximum(np.abs(v), 2.0 ** -126)
    e = np.floor(np.log2(a))
    return np.exp2(np.maximum(e, -126) - 7)


def check_codes(h_gpu: np.ndarray, h_exact: np.ndarray) -> tuple[int, float]:
    """Check 1 on one hidden row; returns (codes that differ from the oracle's,
    the largest excess |code - h| - spacing(h) / 2 over the row's largest |h|)."""
    ref = oracle.bf16_round(h_exact)
    hmax = max(float(np.abs(h_exact).max()), 1e-300)
    excess = (np.abs(h_gpu - h_exact) - _spacing(h_exact) / 2) / hmax
    worst = float(excess.max())
    assert worst <= TAU, (f"hidden code off by {worst:.3g} of the row's largest |h| beyond half a bf16 step "
                          f"(allowed {TAU:.3g}); gpu {h_gpu[excess.argmax()]} exact {h_exact[excess.argmax()]}")
    return int((h_gpu != ref).sum()), max(worst, 0.0)


def check_chunk(c, y: np.ndarray, tokens, h_gpu: np.ndarray, tol: float = 1e-3) -> dict:
    """Checks 1-3 for the given tokens of a bf16-mode chunk call.  c: the test's
    chunk (ids, w, x, records, shared, workload); y: the GPU output [T, d];
    h_gpu: the GPU's hidden rows [T k + T, f] as floats."""
    wl = c.wl
    E, k, d, f, qt = wl["E"], wl["k"], wl["d"], wl["f"], wl["qtype"]
    T = c.T
    _, _, _, entries = oracle.plan_union(c.ids, E)
    pos = np.empty(T * k, np.int64)
    pos[entries] = np.arange(T * k)
    x64 = oracle.x_to_f64(c.x, c.x_dtype)
    P = oracle.PREC_BF16
    flips, codes, worst_excess = 0, 0, 0.0
    given = np.zeros((len(tokens), d))
    exact = np.zeros((len(tokens), d))
    for i, t in enumerate(tokens):
        units = [(c.recs[int(c.ids[t, j])], float(c.w[t, j]), pos[t * k + j]) for j in range(k)]
        if c.shared is not None:
            units.append((c.shared, 1.0, T * k + t))
        for rec, wj, row in units:
            hx = oracle.expert_hidden(qt, P, rec, d, f, x64[t])
            hg = h_gpu[row].astype(np.float64)
            n, m = check_codes(hg, hx)
            flips += n
            codes += f
            worst_excess = max(worst_excess, m)
            given[i] += wj * oracle.expert_down(qt, P, rec, d, f, hg)
            exact[i] += wj * oracle.expert_down(qt, P, rec, d, f, oracle.bf16_round(hx))
    yt = np.asarray(y, np.float64)[tokens]
    den = np.maximum(np.abs(given).max(axis=1), 1e-30)
    given_err = float((np.abs(yt - given).max(axis=1) / den).max())
    assert given_err <= tol, f"y against the oracle's down projection of the GPU's hidden codes: {given_err}"
    from tests import harness as H
    st = H.elementwise_stats(yt, exact.astype(np.float32))
    return {"tokens": len(tokens), "hidden_codes": codes, "flipped_codes": flips,
            "worst_code_excess_over_row_max": worst_excess, "allowed": TAU, "max_rel_row_given_gpu_hidden": given_err,
            "end_to_end": st}
