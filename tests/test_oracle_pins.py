"""Pins for the CPU oracle: checks against something other than the oracle itself.

Pinned against: numpy's and torch's own float16 / bfloat16 conversions
(exhaustive), hand-worked golden blocks (tests/golden/blocks.json), brute-force
sorting and nested-loop grouping, closed forms of constant experts, linearity
in the routing weights, and a dense all-experts evaluation written with numpy
matrix products on the tiny workload.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "blocks.json")


# ---------------------------------------------------------------------------
# formats
# ---------------------------------------------------------------------------

def test_f16_decode_matches_numpy_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = oracle.f16_to_f64(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.int64), ref[~nan].view(np.int64))  # signed zeros too


def _all_scale_bits():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    return b[((b >> 10) & 0x1F) != 0x1F]  # 63,488 finite patterns


def _q8_blocks_all_codes(scale_bits):
    """8 blocks per scale covering codes -127..127 (one padding code 0)."""
    codes = np.concatenate([np.arange(-127, 128), [0]]).astype(np.int8).reshape(8, 32)
    n = scale_bits.size
    blk = np.empty((n, 8, 34), dtype=np.uint8)
    blk[:, :, 0:2] = scale_bits.view(np.uint8).reshape(n, 1, 2)
    blk[:, :, 2:] = codes.view(np.uint8)[None]
    return blk.reshape(-1), np.broadcast_to(codes.astype(np.float64), (n, 8, 32))


def test_q8_0_dequant_exact_exhaustive():
    """All finite fp16 scales x all 255 codes: d*q is exact in double and in float32."""
    sb = _all_scale_bits()
    blk, codes = _q8_blocks_all_codes(sb)
    got = oracle.dequant(oracle.Q8_0, oracle.PREC_F32, blk, sb.size * 256)
    ref = (sb.view(np.float16).astype(np.float64)[:, None, None] * codes).reshape(-1)
    assert np.array_equal(got.view(np.int64), ref.view(np.int64))
    assert np.array_equal(got.astype(np.float32).astype(np.float64), got)  # exact in fp32


def test_q4_0_dequant_exact_exhaustive():
    """All finite fp16 scales x all 16 codes in both nibble positions."""
    sb = _all_scale_bits()
    n = sb.size
    j = np.arange(16)
    byte = (((15 - j) << 4) | j).astype(np.uint8)
    blk = np.empty((n, 18), dtype=np.uint8)
    blk[:, 0:2] = sb.view(np.uint8).reshape(n, 2)
    blk[:, 2:] = byte[None]
    got = oracle.dequant(oracle.Q4_0, oracle.PREC_F32, blk.reshape(-1), n * 32).reshape(n, 32)
    d = sb.view(np.float16).astype(np.float64)[:, None]
    ref = np.concatenate([d * (j - 8.0)[None], d * ((15 - j) - 8.0)[None]], axis=1)
    assert np.array_equal(got.view(np.int64), ref.view(np.int64))
    assert np.array_equal(got.astype(np.float32).astype(np.float64), got)


def test_golden_blocks():
    g = json.load(open(GOLDEN))
    for qname, qt in (("q8_0", oracle.Q8_0), ("q4_0", oracle.Q4_0)):
        for case in g[qname]:
            got = oracle.dequant(qt, oracle.PREC_F32, np.array(case["bytes"], dtype=np.uint8), 32)
            ref = np.array(case["values"], dtype=np.float64)
            assert np.array_equal(got.view(np.int64), ref.view(np.int64)), case["note"]


def test_bf16_dequant_matches_torch_exhaustive():
    """bf16 mode rounds the exact product; torch's float32->bfloat16 conversion is the reference."""
    sb = _all_scale_bits()
    blk, codes = _q8_blocks_all_codes(sb)
    got = oracle.dequant(oracle.Q8_0, oracle.PREC_BF16, blk, sb.size * 256)
    exact = (sb.view(np.float16).astype(np.float64)[:, None, None] * codes).reshape(-1)
    ref = torch.from_numpy(exact.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(got.view(np.int64), ref.view(np.int64))


@pytest.mark.parametrize("v,expect", [
    (1.0 + 2.0 ** -8, 1.0),                          # tie -> even (down)
    (1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -6),          # tie -> even (up)
    (1.0 + 2.0 ** -8 + 2.0 ** -30, 1.0 + 2.0 ** -7),  # just above a tie: rounded once, up
    (-(1.0 + 2.0 ** -8 + 2.0 ** -30), -(1.0 + 2.0 ** -7)),
    (2.0 ** -134, 0.0),                               # half the smallest subnormal -> even (0)
    (3 * 2.0 ** -134, 2.0 ** -132),                   # 1.5 subnormal quanta -> 2
    (255.4 * 2.0 ** 120, 255.0 * 2.0 ** 120),         # largest finite
    (255.5 * 2.0 ** 120, math.inf),                   # rounds past the largest finite
    (-0.0, -0.0),
])
def test_bf16_round_closed_forms(v, expect):
    got = oracle.bf16_round([v])[0]
    assert got == expect and math.copysign(1, got) == math.copysign(1, expect)


# ---------------------------------------------------------------------------
# routing
# ---------------------------------------------------------------------------

def _brute_topk(l, k):
    return sorted(range(len(l)), key=lambda e: (-float(l[e]), e))[:k]


@pytest.mark.parametrize("seed", range(20))
def test_topk_brute_force_small(seed):
    g = np.random.default_rng(seed)
    E = int(g.integers(2, 13))
    k = int(g.integers(1, E + 1))
    T = 5
    # few distinct values so ties are frequent
    l = g.integers(-3, 4, size=(T, E)).astype(np.float32) * 0.5
    ids, w = oracle.topk(l, k)
    for t in range(T):
        assert list(ids[t]) == _brute_topk(l[t], k)
        sel = l[t, ids[t]].astype(np.float64)
        ref = np.exp(sel - sel.max()) / np.exp(sel - sel.max()).sum()
        np.testing.assert_allclose(w[t], ref, rtol=1e-6)


def test_topk_all_equal_exact_weights():
    for E, k in ((8, 2), (256, 8)):
        ids, w = oracle.topk(np.full((3, E), 0.7, np.float32), k)
        assert (ids == np.arange(k)).all()
        assert (w == np.float32(1.0 / k)).all()


def test_topk_signed_zero_tie_goes_to_lower_index():
    l = np.full((1, 8), -1.0, np.float32)
    l[0, 5] = 0.0
    l[0, 2] = -0.0
    ids, w = oracle.topk(l, 2)
    assert list(ids[0]) == [2, 5] and w[0, 0] == w[0, 1] == np.float32(0.5)


def test_topk_one_ulp_beats_lower_index():
    l = np.zeros((1, 4), np.float32)
    l[0, 3] = np.nextafter(np.float32(0), np.float32(1))
    ids, _ = oracle.topk(l, 1)
    assert ids[0, 0] == 3


def test_topk_permutation_invariance():
    g = np.random.default_rng(7)
    l = g.standard_normal((6, 64)).astype(np.float32)
    perm = g.permutation(64)
    ids, w = oracle.topk(l, 8)
    ids_p, w_p = oracle.topk(l[:, perm], 8)
    assert (perm[ids_p] == ids).all()
    assert (w_p == w).all()


def test_topk_weights_sum_and_full_softmax():
    g = np.random.default_rng(3)
    l = g.standard_normal((50, 256)).astype(np.float32)
    _, w = oracle.topk(l, 8)
    assert np.all(np.abs(w.astype(np.float64).sum(1) - 1.0) <= 8 * 2.0 ** -24)
    ids, p = oracle.topk(l, 8, norm=False)
    full = torch.softmax(torch.from_numpy(l.astype(np.float64)), dim=1).numpy()
    np.testing.assert_allclose(p, np.take_along_axis(full, ids, 1), rtol=1e-6)


def test_topk_rejects_bad_input():
    with pytest.raises(ValueError):
        oracle.topk(np.zeros((1, 4), np.float32), 5)
    bad = np.zeros((1, 4), np.float32)
    bad[0, 1] = np.nan
    with pytest.raises(ValueError):
        oracle.topk(bad, 2)


def test_router_logits_against_numpy():
    wl = synth.workload("tiny")
    x = synth.activations(wl["seed"], 4, wl["d"], "f32")
    wr = synth.router_weights(wl["seed"], wl["E"], wl["d"])
    got = oracle.router_logits(oracle.x_to_f64(x, "f32"), wr)
    ref = x.astype(np.float64) @ wr.astype(np.float64).T
    assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0 ** -24 + 1e-30)


# ---------------------------------------------------------------------------
# expert-major union
# ---------------------------------------------------------------------------

def _brute_union(ids, E):
    flat = ids.reshape(-1)
    experts, offsets, entries = [], [0], []
    for e in range(E):
        members = [i for i in range(flat.size) if flat[i] == e]
        if members:
            experts.append(e)
            entries += members
            offsets.append(len(entries))
    return experts, offsets, entries


@pytest.mark.parametrize("T,k,E,seed", [(1, 8, 256, 0), (4, 2, 8, 1), (4, 8, 256, 2),
                                        (64, 8, 16, 3), (37, 3, 5, 4), (0, 8, 256, 5), (9, 1, 1, 6)])
def test_plan_union_brute_force(T, k, E, seed):
    g = np.random.default_rng(seed)
    ids = g.integers(0, E, size=(T, k)).astype(np.int32)
    n, experts, offsets, entries = oracle.plan_union(ids, E)
    be, bo, bn = _brute_union(ids, E)
    assert n == len(be) and list(experts) == be and list(offsets) == bo and list(entries) == bn
    assert offsets[-1] == T * k and np.all(np.diff(offsets) > 0)
    assert sorted(entries) == list(range(T * k))


def test_plan_union_rejects_out_of_range():
    with pytest.raises(ValueError):
        oracle.plan_union(np.array([[0, 9]], np.int32), 8)


# ---------------------------------------------------------------------------
# expert FFN and layer
# ---------------------------------------------------------------------------

def _silu(z):
    return z / (1.0 + math.exp(-z))


def _f16(bits):
    return float(np.array([bits], np.uint16).view(np.float16)[0])


@pytest.mark.parametrize("qtype,codes", [(synth.Q8_0, (3, -2, 5)), (synth.Q4_0, (11, 6, 13))])
def test_ffn_constant_expert_closed_form(qtype, codes):
    d, f = 256, 128
    sbits = (0x2E66, 0x2A8F, 0x2C00)  # ~0.1, ~0.0451, 0.0625
    rec = synth.expert_record_fixed(qtype, d, f, sbits, codes)
    x = np.random.default_rng(1).standard_normal(d)
    y = oracle.expert_ffn(qtype, oracle.PREC_F32, rec, d, f, x)
    val = [c if qtype == synth.Q8_0 else c - 8 for c in codes]
    sg, su, sd = (_f16(b) for b in sbits)
    S = float(np.sum(x))
    expect = f * (sd * val[2]) * _silu(sg * val[0] * S) * (su * val[1] * S)
    np.testing.assert_allclose(y, expect, rtol=1e-12)


def test_ffn_zero_input_gives_zero():
    wl = synth.workload("tiny")
    rec = synth.expert_record(wl["seed"], 0, 0, synth.Q8_0, wl["d"], wl["f"])
    for prec in (oracle.PREC_F32, oracle.PREC_BF16):
        y = oracle.expert_ffn(synth.Q8_0, prec, rec, wl["d"], wl["f"], np.zeros(wl["d"]))
        assert np.all(y == 0.0)


def test_ffn_bf16_mode_closed_form():
    """bf16-exact scales, codes and inputs: only h = silu(g)*u is rounded."""
    d, f = 256, 128
    sbits = (0x2000, 0x2400, 0x2800)  # 2^-7, 2^-6, 2^-5 (exact in bf16)
    codes = (3, 5, 7)
    rec = synth.expert_record_fixed(synth.Q8_0, d, f, sbits, codes)
    x = np.full(d, 0.375)  # S = 96
    y = oracle.expert_ffn(synth.Q8_0, oracle.PREC_BF16, rec, d, f, x)
    S = 96.0
    g, u = 2.0 ** -7 * 3 * S, 2.0 ** -6 * 5 * S
    h = torch.tensor(_silu(g) * u, dtype=torch.float64).to(torch.float32).to(torch.bfloat16).item()
    expect = f * (2.0 ** -5 * 7) * h
    np.testing.assert_allclose(y, expect, rtol=1e-14)
    # and the rounding of h is really there
    assert abs(expect - f * (2.0 ** -5 * 7) * _silu(g) * u) > 0


def _bf16_nearest(v: float) -> float:
    """The bfloat16 value nearest to v, ties to an even last significand bit:
    found by comparing v with the bf16 neighbours around its float32 truncation
    in exact double arithmetic (a search, not a formula)."""
    t = torch.tensor([v], dtype=torch.float64).to(torch.float32)
    b = int(t.view(torch.int32).item()) & 0xFFFF0000  # truncate toward zero in bf16 bits
    cands = [b - 0x10000, b, b + 0x10000, b + 0x20000]
    vals = [float(torch.tensor([c], dtype=torch.int64).to(torch.int32).view(torch.float32).item()) for c in cands]
    best = None
    for c, x in zip(cands, vals):
        dist = abs(x - v)
        key = (dist, (c >> 16) & 1)  # nearer first; on a tie the even significand
        if best is None or key < best[0]:
            best = (key, x)
    return best[1]


@pytest.mark.parametrize("qtype,codes", [(synth.Q8_0, (3, -5, 7)), (synth.Q4_0, (11, 2, 14))])
def test_ffn_bf16_mode_rounds_activations_and_weights(qtype, codes):
    """BF16 mode with inputs that are NOT bf16-exact: x = 1 + 2^-8 + 2^-10 rounds
    up to 1 + 2^-7, and each d*q (fp16 scale ~0.1 times the code) rounds too.
    The closed form of the constant expert then differs from the unrounded one
    by far more than the tolerance, so dropping either rounding fails here."""
    d, f = 256, 128
    sbits = (0x2E66, 0x2A8F, 0x2C01)  # 0.0999755859375, 0.045013427734375, 0.06256103515625
    rec = synth.expert_record_fixed(qtype, d, f, sbits, codes)
    xv = 1.0 + 2.0 ** -8 + 2.0 ** -10
    x = np.full(d, xv)
    y = oracle.expert_ffn(qtype, oracle.PREC_BF16, rec, d, f, x)
    val = [c if qtype == synth.Q8_0 else c - 8 for c in codes]
    wg, wu, wd = (_bf16_nearest(_f16(b) * v) for b, v in zip(sbits, val))
    xb = _bf16_nearest(xv)
    assert xb == 1.0 + 2.0 ** -7
    S = d * xb
    h = _bf16_nearest(_silu(wg * S) * (wu * S))
    expect = f * wd * h
    np.testing.assert_allclose(y, expect, rtol=1e-14)
    # the unrounded closed form is far away: each rounding matters
    raw_w = [_f16(b) * v for b, v in zip(sbits, val)]
    unrounded = f * raw_w[2] * _silu(raw_w[0] * d * xv) * (raw_w[1] * d * xv)
    assert abs(unrounded - expect) > 1e-3 * abs(expect)
    x_only = f * wd * _bf16_nearest(_silu(wg * d * xv) * (wu * d * xv))
    assert abs(x_only - expect) > 1e-3 * abs(expect)


def test_layer_linear_in_routing_weights():
    wl = synth.workload("tiny")
    d, f = wl["d"], wl["f"]
    rec = synth.expert_record(wl["seed"], 0, 3, synth.Q8_0, d, f)
    records = [None] * 8
    records[3] = rec
    records[6] = rec.copy()
    x = synth.activations(wl["seed"], 1, d, "f32")
    x64 = oracle.x_to_f64(x, "f32")
    w = np.array([[0.625, 0.5]], np.float32)
    y = oracle.moe_layer(synth.Q8_0, oracle.PREC_F32, records, None, d, f, x64,
                         np.array([[3, 6]], np.int32), w)
    single = oracle.expert_ffn(synth.Q8_0, oracle.PREC_F32, rec, d, f, x64[0])
    np.testing.assert_allclose(y[0], (single * 1.125).astype(np.float32), rtol=1e-6, atol=1e-7)


def _np_dequant_matrix(blocks, rows, cols):
    """Independent decode with numpy float16 (Q8_0 only)."""
    b = blocks.reshape(rows * cols // 32, 34)
    d = b[:, 0:2].copy().view(np.float16).astype(np.float64)
    q = b[:, 2:].view(np.int8).astype(np.float64)
    return (d * q).reshape(rows, cols)


@pytest.mark.parametrize("with_shared", [False, True])
def test_tiny_layer_dense_brute_force(with_shared):
    """Dense evaluation of every expert for every token, masked to the top-2
    (plus an always-on shared expert of weight 1 in the second case)."""
    wl = synth.workload("tiny")
    d, f, E, k, T = wl["d"], wl["f"], wl["E"], wl["k"], wl["T"]
    recs = [synth.expert_record(wl["seed"], 0, e, synth.Q8_0, d, f) for e in range(E)]
    shared = synth.expert_record(wl["seed"], 0, 0, synth.Q8_0, d, f, shared=True) if with_shared else None
    x = synth.activations(wl["seed"], T, d, "f32").astype(np.float64)
    wr = synth.router_weights(wl["seed"], E, d)
    # oracle path
    logits = oracle.router_logits(x, wr)
    ids, w = oracle.topk(logits, k)
    y = oracle.moe_layer(synth.Q8_0, oracle.PREC_F32, recs, shared, d, f, x, ids, w)

    # dense numpy path
    def dense_ffn(m):
        n1 = f * d // 32 * 34
        Wg = _np_dequant_matrix(m[:n1], f, d)
        Wu = _np_dequant_matrix(m[n1:2 * n1], f, d)
        Wd = _np_dequant_matrix(m[2 * n1:], d, f)
        G, U = x @ Wg.T, x @ Wu.T
        return (G / (1 + np.exp(-G)) * U) @ Wd.T

    lg = (x @ wr.astype(np.float64).T).astype(np.float32).astype(np.float64)
    y_dense = dense_ffn(shared) if with_shared else np.zeros((T, d))
    for e in range(E):
        Y = dense_ffn(recs[e])
        for t in range(T):
            order = np.lexsort((np.arange(E), -lg[t]))[:k]
            if e in order:
                sel = lg[t, order]
                p = np.exp(sel - sel.max()) / np.exp(sel - sel.max()).sum()
                y_dense[t] += p[list(order).index(e)] * Y[t]
    rel = np.abs(y - y_dense).max(1) / np.abs(y_dense).max(1)
    assert rel.max() < 1e-6


@pytest.mark.parametrize("qtype,codes", [(synth.Q8_0, (3, -2, 5)), (synth.Q4_0, (11, 6, 13))])
def test_expert_halves_closed_forms(qtype, codes):
    """The hidden state and the down projection on their own: a constant
    expert gives h_r = silu(s_g c_g S) * (s_u c_u S) for every r, and
    W_d h = s_d c_d * sum(h) for any h."""
    d, f = 256, 128
    sbits = (0x2E66, 0x2A8F, 0x2C00)
    rec = synth.expert_record_fixed(qtype, d, f, sbits, codes)
    val = [c if qtype == synth.Q8_0 else c - 8 for c in codes]
    sg, su, sd = (_f16(b) for b in sbits)
    x = np.random.default_rng(3).standard_normal(d)
    S = float(np.sum(x))
    h = oracle.expert_hidden(qtype, oracle.PREC_F32, rec, d, f, x)
    np.testing.assert_allclose(h, _silu(sg * val[0] * S) * (su * val[1] * S), rtol=1e-12)
    hv = np.random.default_rng(4).standard_normal(f)
    y = oracle.expert_down(qtype, oracle.PREC_F32, rec, d, f, hv)
    np.testing.assert_allclose(y, sd * val[2] * hv.sum(), rtol=1e-12, atol=1e-12)
