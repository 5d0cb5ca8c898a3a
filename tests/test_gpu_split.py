"""moe_expert_ffn_split (hit/miss split of a one-token step, "Nanite for
Experts" §5.5): the resident units on a side stream while moe_route_pull's
copies of the misses run, the copied units after them, merged in plan order.
Checked against the oracle; bitwise the same whatever split of the units is
claimed (real misses, none, half of the step, every unit); refusals."""
import numpy as np
import pytest

import synth
from tests import harness as H

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not H.gpu_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import oracle  # noqa: E402
from routed_expert_execution_amd import moe  # noqa: E402

FFN_TOL = 1e-3


def _say(*a):
    print(*a, flush=True)


def _setup(n_slots=20, qtype=None):
    wl = synth.workload("stack40")
    if qtype is not None:
        wl["qtype"] = qtype
    E, k, d, f = wl["E"], wl["k"], wl["d"], wl["f"]
    ctx = H.make_ctx(wl, n_slots=n_slots, max_tokens=1, n_layers=1)
    host = {}

    def payload(e):
        if e not in host:
            rec = synth.expert_record(wl["seed"], 0, e, wl["qtype"], d, f)
            host[e] = (rec, torch.from_numpy(H.payload(ctx, rec)).pin_memory())
        return host[e][1]

    shared = synth.expert_record(wl["seed"], 0, 0, wl["qtype"], d, f, shared=True)
    return wl, ctx, host, payload, shared, H.device_payload(ctx, shared)


@pytest.mark.parametrize("qtype,prec,with_shared", [(synth.Q8_0, moe.MOE_PREC_F32, True),
                                                     (synth.Q8_0, moe.MOE_PREC_BF16, True),
                                                     (synth.Q4_0, moe.MOE_PREC_F32, True),
                                                     (synth.Q8_0, moe.MOE_PREC_F32, False)])
def test_split_matches_oracle_for_any_claimed_split(qtype, prec, with_shared):
    wl, ctx, host, payload, shared, sh_dev = _setup(qtype=qtype)
    if not with_shared:
        shared = sh_dev = None
    E, k, d, f = wl["E"], wl["k"], wl["d"], wl["f"]
    chain = synth.markov_route_sets(synth.rng(wl["seed"], 91, 0), 7, E, k, wl["p_repeat"])
    side = torch.cuda.Stream()
    plan = moe.Plan(ctx, 1)
    seen_partial = seen_none = seen_all = False
    for t in range(len(chain)):
        _say("split step", t, "qtype", qtype, "prec", prec, "shared", with_shared)
        lg = np.full((1, E), -1.0, np.float32)
        lg[0, chain[t]] = 2.0 + np.arange(k, dtype=np.float32) / 16
        ids = torch.empty(1, k, dtype=torch.int32, device="cuda")
        w = torch.empty(1, k, dtype=torch.float32, device="cuda")
        step = set(int(e) for e in chain[t])
        table = moe.payload_table(ctx, [payload(e) if e in step else None for e in range(E)])
        # the layer input is ready before the routing (the side stream waits for the routing only)
        x_np = synth.activations(wl["seed"], 1, d, "bf16", t, 5)
        x = H.torch_x(x_np, "bf16")
        ex, _, miss = moe.moe_route_pull(ctx, 0, ids, w, plan, table, logits_in=torch.from_numpy(lg).cuda())
        n_miss = int(miss.sum())
        seen_partial |= 0 < n_miss < k
        seen_none |= n_miss == 0
        seen_all |= n_miss == k
        y = torch.empty(1, d, dtype=torch.float32, device="cuda")
        moe.moe_expert_ffn_split(ctx, 0, x, plan, w, y, ex[miss], shared_payload=sh_dev, prec=prec, side=side)
        # every unit resident now: the step routed again, split as claimed
        ys = []
        for claim in ([], list(ex[:k // 2]), list(ex[1::2]), list(ex)):
            moe.moe_slot_release(ctx, 0)
            ex2, _, miss2 = moe.moe_route_pull(ctx, 0, ids, w, plan, table, logits_in=torch.from_numpy(lg).cuda())
            assert list(ex2) == list(ex) and not miss2.any()
            yc = torch.empty(1, d, dtype=torch.float32, device="cuda")
            moe.moe_expert_ffn_split(ctx, 0, x, plan, w, yc, claim, shared_payload=sh_dev, prec=prec, side=side)
            ys.append(yc)
        with pytest.raises(moe.MoeError) as ei:  # one split per moe_route_pull
            moe.moe_expert_ffn_split(ctx, 0, x, plan, w, yc, [], shared_payload=sh_dev, prec=prec, side=side)
        assert ei.value.status == moe.MOE_EINVAL
        y_ref = torch.empty(1, d, dtype=torch.float32, device="cuda")
        moe.moe_expert_ffn(ctx, 0, x, plan, w, y_ref, shared_payload=sh_dev, prec=prec)
        torch.cuda.synchronize()
        yn = y.cpu().numpy()
        for yc in ys:
            assert np.array_equal(yn.view(np.uint32), yc.cpu().numpy().view(np.uint32)), t
        records = [host[e][0] if e in host else None for e in range(E)]
        ids_n, w_n = ids.cpu().numpy(), w.cpu().numpy()
        ref = oracle.moe_layer(wl["qtype"], oracle.PREC_F32 if prec == moe.MOE_PREC_F32 else oracle.PREC_BF16,
                               records, shared, d, f, oracle.x_to_f64(x_np, "bf16"), ids_n, w_n)
        assert np.isfinite(yn).all() and H.max_rel_row_err(yn, ref) <= FFN_TOL, (t, H.elementwise_stats(yn, ref))
        # moe_expert_ffn sums in another order: close, not bitwise
        assert H.max_rel_row_err(yn, y_ref.cpu().numpy()) <= 1e-4
        moe.moe_slot_release(ctx, 0)
    assert seen_partial and seen_all
    assert moe.moe_check(ctx) == moe.MOE_OK


def test_split_is_slot_independent():
    """The same steps through two pools whose slots hold the experts in
    different places (the second pool larger and first filled with other
    experts): bitwise the same outputs."""
    outs = []
    for n_slots, warm in ((20, []), (33, [200, 201, 202, 203, 204, 205, 206])):
        wl, ctx, host, payload, shared, sh_dev = _setup(n_slots=n_slots)
        E, k, d = wl["E"], wl["k"], wl["d"]
        if warm:
            table = moe.payload_table(ctx, [payload(e) if e in warm else None for e in range(E)])
            moe.moe_slot_pull(ctx, 0, warm, table)
            moe.moe_slot_release(ctx, 0)
        chain = synth.markov_route_sets(synth.rng(wl["seed"], 93, 0), 5, E, k, wl["p_repeat"])
        side = torch.cuda.Stream()
        plan = moe.Plan(ctx, 1)
        ys, slots_seen = [], []
        for t in range(len(chain)):
            lg = np.full((1, E), -1.0, np.float32)
            lg[0, chain[t]] = 2.0 + np.arange(k, dtype=np.float32) / 16
            ids = torch.empty(1, k, dtype=torch.int32, device="cuda")
            w = torch.empty(1, k, dtype=torch.float32, device="cuda")
            step = set(int(e) for e in chain[t])
            table = moe.payload_table(ctx, [payload(e) if e in step else None for e in range(E)])
            x = H.torch_x(synth.activations(wl["seed"], 1, d, "bf16", t, 6), "bf16")
            ex, sl, miss = moe.moe_route_pull(ctx, 0, ids, w, plan, table, logits_in=torch.from_numpy(lg).cuda())
            y = torch.empty(1, d, dtype=torch.float32, device="cuda")
            moe.moe_expert_ffn_split(ctx, 0, x, plan, w, y, ex[miss], shared_payload=sh_dev, side=side)
            moe.moe_slot_release(ctx, 0)
            ys.append(y)
            slots_seen.append(list(sl))
        torch.cuda.synchronize()
        assert moe.moe_check(ctx) == moe.MOE_OK
        outs.append(([y.cpu().numpy() for y in ys], slots_seen))
    (ya, sa), (yb, sb) = outs
    assert sa != sb  # the experts did land in other slots
    for t, (a, b) in enumerate(zip(ya, yb)):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), t


def test_split_refusals():
    wl, ctx, host, payload, shared, sh_dev = _setup()
    E, k, d = wl["E"], wl["k"], wl["d"]
    x = H.torch_x(synth.activations(wl["seed"], 1, d, "bf16", 0, 5), "bf16")
    w = torch.full((1, k), 1.0 / k, dtype=torch.float32, device="cuda")
    y = torch.empty(1, d, dtype=torch.float32, device="cuda")
    plan = moe.Plan(ctx, 1)
    with pytest.raises(moe.MoeError) as ei:  # no moe_route_pull yet
        moe.moe_expert_ffn_split(ctx, 0, x, plan, w, y, [], shared_payload=sh_dev)
    assert ei.value.status == moe.MOE_EINVAL
    lg = np.full((1, E), -1.0, np.float32)
    lg[0, :k] = 2.0
    ids = torch.empty(1, k, dtype=torch.int32, device="cuda")
    table = moe.payload_table(ctx, [payload(e) if e < k else None for e in range(E)])
    moe.moe_route_pull(ctx, 0, ids, w, plan, table, logits_in=torch.from_numpy(lg).cuda())
    for bad in ([E], [-1]):
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_expert_ffn_split(ctx, 0, x, plan, w, y, bad, shared_payload=sh_dev)
        assert ei.value.status == moe.MOE_EINVAL
    lib = moe.library()
    # T = 2 and a layer out of range, straight through the C ABI
    assert lib.moe_expert_ffn_split(ctx.handle, 0, x.data_ptr(), moe.MOE_BF16, 2, moe.C.byref(plan.c), w.data_ptr(),
                                    sh_dev.data_ptr(), 0, None, 0, y.data_ptr(), None, None) == moe.MOE_EINVAL
    assert lib.moe_expert_ffn_split(ctx.handle, 3, x.data_ptr(), moe.MOE_BF16, 1, moe.C.byref(plan.c), w.data_ptr(),
                                    sh_dev.data_ptr(), 0, None, 0, y.data_ptr(), None, None) == moe.MOE_EINVAL
    torch.cuda.synchronize()
    assert moe.moe_check(ctx) == moe.MOE_OK
