"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bars: bit-exact routing ids (given the same logits), bit-exact plans and
dequantised weights; routing weights within 1e-6 relative; expert FFN outputs
within 1e-3 maximum relative error per token row (max_i |y - r| / max_i |r|);
bitwise-identical outputs under any slot assignment (cache transparency,
"Paging the Experts", §5.3) and across repeated runs.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import harness as H

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not H.gpu_available():  # pragma: no cover - the GPU suite only runs where a GPU is
    pytest.skip("no GPU", allow_module_level=True)

from routed_expert_execution_amd import moe  # noqa: E402

FFN_TOL = 1e-3


def _say(*a):
    print(*a, flush=True)


# ---------------------------------------------------------------------------
# dequantisation
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny", "decode", "mtp"])
@pytest.mark.parametrize("prec", [oracle.PREC_F32, oracle.PREC_BF16])
def test_dequant_bit_exact(name, prec):
    wl = synth.workload(name)
    _say("dequant", name, prec)
    ctx = H.make_ctx(wl, n_slots=1, max_tokens=1)
    for e in (0, 3):
        rec = synth.expert_record(wl["seed"], 0, e, wl["qtype"], wl["d"], wl["f"])
        dev = H.device_payload(ctx, rec)
        out = torch.empty(3 * wl["d"] * wl["f"], dtype=torch.float32, device="cuda")
        moe.moe_dequant(ctx, dev, out, prec=prec)
        got = out.cpu().numpy().astype(np.float64)
        ref = oracle.dequant(wl["qtype"], prec, rec, 3 * wl["d"] * wl["f"])
        assert np.array_equal(got.view(np.int64), ref.view(np.int64))


def test_dequant_exhaustive_codes_and_scales():
    """Every finite fp16 scale with every Q8_0 code, through one payload of the tiny shape."""
    wl = synth.workload("tiny")
    ctx = H.make_ctx(wl, n_slots=1, max_tokens=1)
    n_blocks = 3 * wl["d"] * wl["f"] // 32  # 3,072 blocks per expert
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    scales = b[((b >> 10) & 0x1F) != 0x1F]
    codes = np.concatenate([np.arange(-127, 128), [0]]).astype(np.int8).reshape(8, 32)
    done = 0
    out = torch.empty(3 * wl["d"] * wl["f"], dtype=torch.float32, device="cuda")
    while done < scales.size:
        sc = np.resize(scales[done:done + n_blocks // 8], n_blocks // 8)
        blk = np.empty((sc.size, 8, 34), np.uint8)
        blk[:, :, 0:2] = sc.view(np.uint8).reshape(-1, 1, 2)
        blk[:, :, 2:] = codes.view(np.uint8)[None]
        rec = blk.reshape(-1)
        moe.moe_dequant(ctx, H.device_payload(ctx, rec), out, prec=oracle.PREC_F32)
        ref = oracle.dequant(synth.Q8_0, oracle.PREC_F32, rec, out.numel())
        assert np.array_equal(out.cpu().numpy().astype(np.float64).view(np.int64), ref.view(np.int64))
        done += n_blocks // 8


# ---------------------------------------------------------------------------
# routing
# ---------------------------------------------------------------------------

def _delta_band(x64, wr):
    """Standard forward bound on the two fp32 dot products' rounding, doubled."""
    d = x64.shape[1]
    u = 2.0 ** -24
    gamma = d * u / (1 - d * u)
    return 2 * gamma * (np.abs(x64) @ np.abs(wr.astype(np.float64)).T).max(axis=1)


@pytest.mark.parametrize("name,T", [("tiny", 4), ("decode", 1), ("decode", 64), ("decode", 512)])
def test_route_from_router_weights(name, T):
    wl = synth.workload(name)
    _say("route", name, T)
    ctx = H.make_ctx(wl, n_slots=1, max_tokens=T)
    x = synth.activations(wl["seed"], T, wl["d"], wl["x_dtype"], 1000 + T)
    wr = synth.router_weights(wl["seed"], wl["E"], wl["d"])
    ids = torch.empty(T, wl["k"], dtype=torch.int32, device="cuda")
    w = torch.empty(T, wl["k"], dtype=torch.float32, device="cuda")
    lo = torch.empty(T, wl["E"], dtype=torch.float32, device="cuda")
    moe.moe_route(ctx, ids, w, x=H.torch_x(x, wl["x_dtype"]), w_router=torch.from_numpy(wr).cuda(),
                  logits_out=lo)
    g_ids, g_w, g_lo = ids.cpu().numpy(), w.cpu().numpy(), lo.cpu().numpy()
    x64 = oracle.x_to_f64(x, wl["x_dtype"])
    o_lo = oracle.router_logits(x64, wr)
    band = _delta_band(x64, wr)
    assert np.all(np.abs(g_lo - o_lo) <= band[:, None] + 1e-30)
    # (i) same logits -> bit-exact ids; weights to 1e-6
    r_ids, r_w = oracle.topk(g_lo, wl["k"])
    assert np.array_equal(g_ids, r_ids)
    np.testing.assert_allclose(g_w, r_w, rtol=1e-6, atol=1e-7)
    # (ii) end to end.  eps_t = this token's largest |gpu - oracle| logit difference
    # (itself within the rounding band above).  No perturbation of that size can
    # reorder two logits more than 2 eps_t apart, so:
    #  - where the gap between the oracle's k-th and (k+1)-th logits exceeds
    #    2 eps_t, the selected SET must be identical;
    #  - where every consecutive gap among the oracle's k + 1 largest exceeds
    #    2 eps_t, the ranked ids must be identical too.
    # Other tokens have several correct answers and are covered by (i).  The
    # logits have a spread of about 0.02 sqrt(d) (about 0.9 at d = 2048), so
    # neighbouring order statistics sit 1e-3 .. 1e-1 apart against eps_t of
    # about 1e-6: a gap inside 2 eps_t has a chance of order 1e-4 per token, and
    # at least 95 % of the tokens must be clear in both senses.
    o_ids, _ = oracle.topk(o_lo, wl["k"])
    k = wl["k"]
    eps = np.abs(g_lo.astype(np.float64) - o_lo).max(axis=1)
    srt = -np.sort(-o_lo.astype(np.float64), axis=1)[:, : k + 1]
    gaps = -np.diff(srt, axis=1)
    set_clear = gaps[:, k - 1] > 2 * eps
    ranked_clear = gaps.min(axis=1) > 2 * eps
    _say("  tokens with a forced set:", int(set_clear.sum()), "forced ranking:", int(ranked_clear.sum()),
         "of", T, "max eps", float(eps.max()))
    assert set_clear.mean() >= 0.95 and ranked_clear.mean() >= 0.95
    assert np.array_equal(np.sort(g_ids[set_clear], axis=1), np.sort(o_ids[set_clear], axis=1))
    assert np.array_equal(g_ids[ranked_clear], o_ids[ranked_clear])


@pytest.mark.parametrize("E,k", [(8, 2), (256, 8), (1024, 32), (100, 7)])
@pytest.mark.parametrize("kind", ["ties", "equal", "signed_zero", "normal", "one_ulp", "c64", "c65"])
@pytest.mark.parametrize("norm", [1, 0])
def test_route_logits_in_bit_exact(E, k, kind, norm):
    """Top-k on edge cases.  c64 / c65: 64 or 65 equal largest logits, one in
    every group of 32 keys, so that at 256 experts the candidate selection takes
    exactly 64 candidates, or falls back to the k rounds at 65."""
    T = 37  # ragged against the 4 tokens per workgroup
    g = np.random.default_rng(E * 31 + k)
    if kind in ("c64", "c65"):
        n = min(int(kind[1:]), E)
        lg = (-1.0 - g.uniform(0, 1, size=(T, E))).astype(np.float32)
        lg[:, (np.arange(n) * E) // n] = 1.0
    elif kind == "ties":
        lg = g.integers(-2, 3, size=(T, E)).astype(np.float32)
    elif kind == "equal":
        lg = np.full((T, E), 1.25, np.float32)
    elif kind == "signed_zero":
        lg = np.where(g.uniform(size=(T, E)) < 0.5, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
        lg[:, ::3] = -1.0
    elif kind == "one_ulp":
        lg = np.zeros((T, E), np.float32)
        lg[:, E - 1] = np.nextafter(np.float32(0), np.float32(1))
        lg[:, E // 2] = np.nextafter(np.float32(0), np.float32(-1))
    else:
        lg = g.standard_normal((T, E)).astype(np.float32)
    wl = dict(synth.workload("decode"), E=E, k=k)
    ctx = H.make_ctx(wl, n_slots=1, max_tokens=T, norm_topk=norm)
    ids = torch.empty(T, k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, k, dtype=torch.float32, device="cuda")
    moe.moe_route(ctx, ids, w, logits_in=torch.from_numpy(lg).cuda())
    r_ids, r_w = oracle.topk(lg, k, norm=bool(norm))
    assert np.array_equal(ids.cpu().numpy(), r_ids)
    np.testing.assert_allclose(w.cpu().numpy(), r_w, rtol=2e-6, atol=1e-7)


# ---------------------------------------------------------------------------
# expert-major union
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T,k,E,kind", [(1, 8, 256, "uniform"), (4, 8, 256, "uniform"), (4, 2, 8, "uniform"),
                                        (37, 8, 256, "uniform"), (512, 8, 256, "zipf"), (513, 8, 256, "zipf"),
                                        (300, 2, 8, "same"), (200, 32, 1024, "uniform"), (0, 8, 256, "uniform"),
                                        (4096, 8, 256, "zipf"), (1024, 8, 256, "zipf"), (1025, 8, 256, "zipf"),
                                        (2048, 32, 1024, "uniform"), (65536, 8, 256, "zipf"),
                                        (6000, 2, 8, "same")])
def test_plan_union_bit_exact(T, k, E, kind):
    """Up to 8192 assignments one workgroup sorts them (1024 x 8 is the
    last such); more run as per-segment counts, one scan and per-segment
    scatters (1025 x 8: a ragged last segment; 65536 x 8: 128 segments)."""
    _say("plan", T, k, E, kind)
    wl = dict(synth.workload("decode"), E=E, k=k)
    ctx = H.make_ctx(wl, n_slots=1, max_tokens=max(T, 1))
    g = np.random.default_rng(T + k + E)
    if kind == "zipf":
        lg = synth.zipf_gumbel_logits(T + 11, T, E, 1.1)
        ids_np = np.argsort(-lg, axis=1, kind="stable")[:, :k].astype(np.int32)
    elif kind == "same":
        ids_np = np.tile(np.arange(k, dtype=np.int32), (T, 1))
    else:
        ids_np = np.array([g.choice(E, size=k, replace=False) for _ in range(T)], dtype=np.int32).reshape(T, k)
    plan = moe.Plan(ctx, T)
    moe.moe_plan_union(ctx, torch.from_numpy(ids_np).cuda(), plan)
    n, ex, off, ent = plan.host()
    rn, rex, roff, rent = oracle.plan_union(ids_np, E)
    assert n == rn and np.array_equal(ex, rex) and np.array_equal(off, roff) and np.array_equal(ent, rent)


@pytest.mark.parametrize("T", [37, 4096])
def test_plan_union_drops_out_of_range_ids(T):
    """Out-of-range ids are dropped (the plan is the oracle's union of the
    other entries, at their own positions) and set the error word, on the
    one-workgroup path and the segmented one."""
    wl = dict(synth.workload("decode"))
    E, k = wl["E"], wl["k"]
    ctx = H.make_ctx(wl, n_slots=1, max_tokens=T)
    lg = synth.zipf_gumbel_logits(T + 5, T, E, 1.1)
    ids_np = np.argsort(-lg, axis=1, kind="stable")[:, :k].astype(np.int32)
    g = np.random.default_rng(T)
    bad = g.choice(T * k, size=max(3, T // 64), replace=False)
    flat = ids_np.reshape(-1).copy()
    flat[bad] = np.where(np.arange(bad.size) % 2 == 0, E + 3, -1)
    plan = moe.Plan(ctx, T)
    moe.moe_plan_union(ctx, torch.from_numpy(flat.reshape(T, k)).cuda(), plan)
    n, ex, off, ent = plan.host()
    valid = np.flatnonzero((flat >= 0) & (flat < E))
    rn, rex, roff, rent = oracle.plan_union(flat[valid].reshape(-1, 1), E)
    assert n == rn and np.array_equal(ex, rex) and np.array_equal(off, roff)
    assert np.array_equal(ent[: valid.size], valid[rent])
    assert moe.moe_check(ctx) == moe.MOE_EINVAL


# ---------------------------------------------------------------------------
# expert FFN
# ---------------------------------------------------------------------------

class Step:
    """One routed step on the GPU with every needed expert placed by the test."""

    def __init__(self, name, T, step=0, prec=oracle.PREC_F32, n_slots=None, **overrides):
        wl = dict(synth.workload(name), **overrides)
        self.wl, self.T, self.prec = wl, T, prec
        E, k, d, f = wl["E"], wl["k"], wl["d"], wl["f"]
        self.x = synth.activations(wl["seed"], T, d, wl["x_dtype"], step)
        if name in ("tiny", "decode"):
            wr = synth.router_weights(wl["seed"], E, d)
            lg = oracle.router_logits(oracle.x_to_f64(self.x, wl["x_dtype"]), wr)
        else:
            lg = synth.mtp_logits(wl["seed"], step, T, E, k, wl.get("p_shared_route", 0.5))
        self.ids, self.w = oracle.topk(lg, k)
        self.used = sorted(set(self.ids.reshape(-1).tolist()))
        self.recs = {e: synth.expert_record(wl["seed"], 0, e, wl["qtype"], d, f) for e in self.used}
        self.shared = synth.expert_record(wl["seed"], 0, 0, wl["qtype"], d, f, shared=True) if wl["shared"] else None
        self.ctx = H.make_ctx(wl, n_slots=n_slots or max(len(self.used), 1), max_tokens=T)
        self.sh_dev = H.device_payload(self.ctx, self.shared) if self.shared is not None else None
        self.x_dev = H.torch_x(self.x, wl["x_dtype"])
        self.ids_dev = torch.from_numpy(self.ids).cuda()
        self.w_dev = torch.from_numpy(self.w).cuda()
        self.plan = moe.Plan(self.ctx, T)
        moe.moe_plan_union(self.ctx, self.ids_dev, self.plan)

    def place(self, perm=None):
        """Put used expert i into slot perm[i] and bind the page table."""
        perm = list(range(len(self.used))) if perm is None else perm
        for i, e in enumerate(self.used):
            H.put_expert(self.ctx, perm[i], self.recs[e])
            moe.moe_slot_bind(self.ctx, 0, e, perm[i])

    def run(self):
        y = torch.full((self.T, self.wl["d"]), float("nan"), dtype=torch.float32, device="cuda")
        moe.moe_expert_ffn(self.ctx, 0, self.x_dev, self.plan, self.w_dev, y, shared_payload=self.sh_dev,
                           prec=self.prec)
        torch.cuda.synchronize()
        return y.cpu().numpy()

    def reference(self):
        wl = self.wl
        records = [self.recs.get(e) for e in range(wl["E"])]
        return oracle.moe_layer(wl["qtype"], self.prec, records, self.shared, wl["d"], wl["f"],
                                oracle.x_to_f64(self.x, wl["x_dtype"]), self.ids, self.w)


@pytest.mark.parametrize("name,T,step", [("tiny", 4, 0), ("tiny", 1, 1), ("tiny", 3, 2), ("decode", 1, 0),
                                         ("decode", 1, 7), ("decode", 2, 3), ("decode", 4, 5), ("mtp", 4, 0),
                                         ("mtp", 4, 9), ("mtp", 1, 4)])
def test_ffn_decode_parity(name, T, step):
    _say("ffn", name, T, step)
    s = Step(name, T, step)
    s.place()
    y = s.run()
    assert moe.moe_check(s.ctx) == moe.MOE_OK
    ref = s.reference()
    err = H.max_rel_row_err(y, ref)
    _say("  max rel row err", err)
    assert np.isfinite(y).all() and err <= FFN_TOL


@pytest.mark.parametrize("k,T", [(32, 4), (16, 3), (32, 1)])
def test_ffn_decode_wide_topk_parity(k, T):
    """top-16/32 of 64 experts: more plan entries than the decode kernel stages at
    once (several entry groups) and more down tiles than its registers hold."""
    _say("ffn wide", k, T)
    s = Step("decode", T, 11, E=64, k=k)
    s.place()
    y = s.run()
    assert moe.moe_check(s.ctx) == moe.MOE_OK
    err = H.max_rel_row_err(y, s.reference())
    _say("  max rel row err", err)
    assert np.isfinite(y).all() and err <= FFN_TOL


@pytest.mark.parametrize("name", ["mtp", "tiny"])
def test_decode_mixed_token_counts_share_one_workspace(name):
    """Steps of 4, 1, 3, 2, 4, 1, 3, 2 tokens on one context (one hand-off
    workspace and launch count; steps of three or four tokens split each row
    group's down work over two workgroups, the others do not): every output
    matches its reference and repeats bit for bit when its step comes again."""
    wl = synth.workload(name)
    E, k, d, f = wl["E"], wl["k"], wl["d"], wl["f"]
    Ts = [4, 1, 3, 2]
    steps = {}
    used = set()
    for T in Ts:
        x = synth.activations(wl["seed"], T, d, wl["x_dtype"], 50 + T)
        if name == "tiny":
            lg = oracle.router_logits(oracle.x_to_f64(x, wl["x_dtype"]), synth.router_weights(wl["seed"], E, d))
        else:
            lg = synth.mtp_logits(wl["seed"], 50 + T, T, E, k, wl.get("p_shared_route", 0.5))
        ids, w = oracle.topk(lg, k)
        steps[T] = (x, ids, w)
        used |= set(ids.reshape(-1).tolist())
    used = sorted(used)
    recs = {e: synth.expert_record(wl["seed"], 0, e, wl["qtype"], d, f) for e in used}
    shared = synth.expert_record(wl["seed"], 0, 0, wl["qtype"], d, f, shared=True) if wl["shared"] else None
    ctx = H.make_ctx(wl, n_slots=len(used), max_tokens=4)
    for i, e in enumerate(used):
        H.put_expert(ctx, i, recs[e])
        moe.moe_slot_bind(ctx, 0, e, i)
    sh_dev = H.device_payload(ctx, shared) if shared is not None else None
    records = [recs.get(e) for e in range(E)]
    dev, refs = {}, {}
    for T, (x, ids, w) in steps.items():
        plan = moe.Plan(ctx, T)
        ids_dev = torch.from_numpy(ids).cuda()
        moe.moe_plan_union(ctx, ids_dev, plan)
        dev[T] = (H.torch_x(x, wl["x_dtype"]), plan, torch.from_numpy(w).cuda())
        refs[T] = oracle.moe_layer(wl["qtype"], oracle.PREC_F32, records, shared, d, f,
                                   oracle.x_to_f64(x, wl["x_dtype"]), ids, w)
    first = {}
    for T in Ts + Ts:
        _say("mixed", name, T)
        xd, plan, wd = dev[T]
        y = torch.full((T, d), float("nan"), dtype=torch.float32, device="cuda")
        moe.moe_expert_ffn(ctx, 0, xd, plan, wd, y, shared_payload=sh_dev, prec=oracle.PREC_F32)
        torch.cuda.synchronize()
        y = y.cpu().numpy()
        assert moe.moe_check(ctx) == moe.MOE_OK
        assert np.isfinite(y).all() and H.max_rel_row_err(y, refs[T]) <= FFN_TOL
        if T in first:
            assert np.array_equal(y.view(np.uint32), first[T].view(np.uint32))
        else:
            first[T] = y


@pytest.mark.parametrize("T,shared", [(4, False), (3, True), (4, True)])
def test_decode_split_down_with_one_or_two_units(T, shared):
    """Every token of a three- or four-token step picks the same single expert
    (top-1): one unit, or two with the shared expert, so a row group's second
    down workgroup has no unit (or one) of its own."""
    _say("one unit", T, shared)
    wl = dict(synth.workload("tiny"), k=1, shared=shared)
    d, f = wl["d"], wl["f"]
    x = synth.activations(wl["seed"], T, d, wl["x_dtype"], 31)
    ids = np.full((T, 1), 5, dtype=np.int32)
    w = np.ones((T, 1), dtype=np.float32)
    rec = synth.expert_record(wl["seed"], 0, 5, wl["qtype"], d, f)
    sh = synth.expert_record(wl["seed"], 0, 0, wl["qtype"], d, f, shared=True) if shared else None
    ctx = H.make_ctx(wl, n_slots=1, max_tokens=4)
    H.put_expert(ctx, 0, rec)
    moe.moe_slot_bind(ctx, 0, 5, 0)
    plan = moe.Plan(ctx, T)
    moe.moe_plan_union(ctx, torch.from_numpy(ids).cuda(), plan)
    y = torch.full((T, d), float("nan"), dtype=torch.float32, device="cuda")
    moe.moe_expert_ffn(ctx, 0, H.torch_x(x, wl["x_dtype"]), plan, torch.from_numpy(w).cuda(), y,
                       shared_payload=H.device_payload(ctx, sh) if shared else None, prec=oracle.PREC_F32)
    torch.cuda.synchronize()
    assert moe.moe_check(ctx) == moe.MOE_OK
    records = [rec if e == 5 else None for e in range(wl["E"])]
    ref = oracle.moe_layer(wl["qtype"], oracle.PREC_F32, records, sh, d, f, oracle.x_to_f64(x, wl["x_dtype"]), ids, w)
    y = y.cpu().numpy()
    assert np.isfinite(y).all() and H.max_rel_row_err(y, ref) <= FFN_TOL


@pytest.mark.parametrize("name,T", [("decode", 1), ("mtp", 4)])
def test_decode_alternating_inputs_see_fresh_hidden_rows(name, T):
    """Launches alternating between two activation sets on one context (same
    experts, same hidden-row workspace): every output matches its own input's
    reference and repeats bit for bit, so no launch reads a hidden row left by
    the previous one."""
    s = Step(name, T, 4)
    s.place()
    xs = [s.x, synth.activations(s.wl["seed"], T, s.wl["d"], s.wl["x_dtype"], 777)]
    devs = [H.torch_x(x, s.wl["x_dtype"]) for x in xs]
    refs = []
    for x in xs:
        s.x = x
        refs.append(s.reference())
    first = [None, None]
    for i in range(8):
        s.x_dev = devs[i % 2]
        y = s.run()
        assert H.max_rel_row_err(y, refs[i % 2]) <= FFN_TOL
        if first[i % 2] is None:
            first[i % 2] = y
        assert np.array_equal(y.view(np.uint32), first[i % 2].view(np.uint32))
    assert moe.moe_check(s.ctx) == moe.MOE_OK


@pytest.mark.parametrize("name,T", [("decode", 1), ("mtp", 4), ("tiny", 3)])
def test_decode_wait_timeout_fails_closed_and_recovers(monkeypatch, name, T):
    """A negative wait bound (set from the host) makes every down workgroup give up
    at its first check (with three or four tokens also the wait of a row
    group's second half for the first half's sums): the launch still
    completes, rows whose wait ran out are NaN, moe_check reports MOE_ETIMEOUT
    and resets the hand-off workspace, and the next launches are exact again."""
    _say("timeout", name, T)
    s = Step(name, T, 0)
    s.place()
    ref = s.reference()
    monkeypatch.setenv("MOE_SYNC_WAIT_TICKS", "-1")
    y = s.run()
    monkeypatch.delenv("MOE_SYNC_WAIT_TICKS")
    assert np.isnan(y).any()
    assert moe.moe_check(s.ctx) == moe.MOE_ETIMEOUT
    y2 = s.run()
    assert moe.moe_check(s.ctx) == moe.MOE_OK
    assert H.max_rel_row_err(y2, ref) <= FFN_TOL
    y3 = s.run()
    assert moe.moe_check(s.ctx) == moe.MOE_OK
    assert np.array_equal(y3.view(np.uint32), y2.view(np.uint32))


@pytest.mark.parametrize("name,T", [("decode", 1), ("decode", 4), ("mtp", 4), ("tiny", 4)])
def test_ffn_decode_bf16_mode_parity(name, T):
    _say("ffn bf16", name, T)
    s = Step(name, T, 2, prec=oracle.PREC_BF16)
    s.place()
    y = s.run()
    ref = s.reference()
    err = H.max_rel_row_err(y, ref)
    _say("  max rel row err", err)
    assert np.isfinite(y).all() and err <= FFN_TOL


@pytest.mark.parametrize("name,T", [("decode", 1), ("mtp", 4), ("tiny", 4)])
def test_cache_transparency_and_determinism(name, T):
    """Identical bits under identity, reversed and random slot maps and on repeats."""
    _say("transparency", name, T)
    s = Step(name, T, 3, n_slots=None)
    n = len(s.used)
    s.ctx = H.make_ctx(s.wl, n_slots=n + 5, max_tokens=T)
    s.sh_dev = H.device_payload(s.ctx, s.shared) if s.shared is not None else None
    s.plan = moe.Plan(s.ctx, T)
    moe.moe_plan_union(s.ctx, s.ids_dev, s.plan)
    outs = []
    g = np.random.default_rng(5)
    for perm in (list(range(n)), list(range(n + 4, 4, -1)), list(g.permutation(n + 5)[:n]),
                 list(g.permutation(n + 5)[:n])):
        s.place(perm)
        outs.append(s.run())
        outs.append(s.run())
    for o in outs[1:]:
        assert np.array_equal(o.view(np.uint32), outs[0].view(np.uint32))


def test_unmapped_expert_fails_closed():
    s = Step("mtp", 4, 6)
    s.place()
    victim = s.used[len(s.used) // 2]
    moe.moe_slot_bind(s.ctx, 0, victim, -1)
    y = s.run()
    assert moe.moe_check(s.ctx) == moe.MOE_EMISS
    hit = (s.ids == victim).any(axis=1)
    assert hit.any()
    assert np.isnan(y[hit]).all(axis=1).all()
    assert np.isfinite(y[~hit]).all()
    # mapping it again recovers, and the error word was cleared by moe_check
    moe.moe_slot_bind(s.ctx, 0, victim, s.used.index(victim))
    y2 = s.run()
    assert moe.moe_check(s.ctx) == moe.MOE_OK
    assert H.max_rel_row_err(y2, s.reference()) <= FFN_TOL


def test_zero_tokens_is_a_no_op():
    s = Step("decode", 1, 0)
    y = torch.full((0, s.wl["d"]), 0.0, dtype=torch.float32, device="cuda")
    moe.moe_expert_ffn(s.ctx, 0, s.x_dev[:0], s.plan, s.w_dev[:0], y, shared_payload=s.sh_dev)
    assert moe.moe_check(s.ctx) == moe.MOE_OK


# ---------------------------------------------------------------------------
# slots filled from pinned host memory on a side stream
# ---------------------------------------------------------------------------

def test_staged_stack_matches_oracle_and_lru_model():
    """Sequential layers sharing one small LRU pool: misses are filled from pinned host
    payloads on a side stream; every layer's output matches the oracle and the
    counters match the LRU model."""
    from oracle.lru import LruModel
    wl = synth.workload("stack40")
    L, n_tok, n_slots = 3, 6, 20
    E, k, d, f = wl["E"], wl["k"], wl["d"], wl["f"]
    ctx = H.make_ctx(wl, n_slots=n_slots, max_tokens=1, n_layers=L)
    model = LruModel(n_slots, ctx.payload_bytes)
    chains = [synth.markov_route_sets(synth.rng(wl["seed"], 55, l), n_tok, E, k, wl["p_repeat"]) for l in range(L)]
    host = {}
    shared = synth.expert_record(wl["seed"], 0, 0, wl["qtype"], d, f, shared=True)
    sh_dev = H.device_payload(ctx, shared)
    side = torch.cuda.Stream()
    plan = moe.Plan(ctx, 1)
    for t in range(n_tok):
        for l in range(L):
            lg = np.full((1, E), -1.0, np.float32)
            lg[0, chains[l][t]] = 2.0 + np.arange(k, dtype=np.float32) / 16
            ids = torch.empty(1, k, dtype=torch.int32, device="cuda")
            w = torch.empty(1, k, dtype=torch.float32, device="cuda")
            moe.moe_route(ctx, ids, w, logits_in=torch.from_numpy(lg).cuda())
            moe.moe_plan_union(ctx, ids, plan)
            n, ex, _, _ = plan.host()
            slots, miss = moe.moe_slot_map(ctx, l, ex)
            ms, mm, _ = model.map(l, list(ex))
            assert list(slots) == ms and list(miss) == mm
            for e, s_, m in zip(ex, slots, miss):
                if m:
                    key = (l, int(e))
                    if key not in host:
                        rec = synth.expert_record(wl["seed"], l, int(e), wl["qtype"], d, f)
                        host[key] = (rec, torch.from_numpy(H.payload(ctx, rec)).pin_memory())
                    moe.moe_slot_fill(ctx, l, int(e), int(s_), host[key][1], stream=side)
            x = synth.activations(wl["seed"], 1, d, "bf16", t, l)
            y = torch.empty(1, d, dtype=torch.float32, device="cuda")
            moe.moe_expert_ffn(ctx, l, H.torch_x(x, "bf16"), plan, w, y, shared_payload=sh_dev)
            moe.moe_slot_release(ctx, l)
            model.release(l)
            assert moe.moe_check(ctx) == moe.MOE_OK
            records = [None] * E
            for e in ex:
                if (l, int(e)) not in host:
                    host[(l, int(e))] = (synth.expert_record(wl["seed"], l, int(e), wl["qtype"], d, f), None)
                records[int(e)] = host[(l, int(e))][0]
            ref = oracle.moe_layer(wl["qtype"], oracle.PREC_F32, records, shared, d, f,
                                   oracle.x_to_f64(x, "bf16"), ids.cpu().numpy(), w.cpu().numpy())
            assert H.max_rel_row_err(y.cpu().numpy(), ref) <= FFN_TOL
    st = moe.moe_stats(ctx)
    c = model.counters()
    assert (st["hits"], st["misses"], st["evictions"]) == (c["hits"], c["misses"], c["evictions"])
    assert st["bytes_staged"] == st["misses"] * ctx.payload_bytes and st["fills"] == st["misses"]
    assert c["evictions"] > 0
