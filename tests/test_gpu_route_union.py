"""moe_route_union against moe_route + moe_plan_union: the same arguments must
give bit-identical ids, weights, logits and plans (for T <= 4 the top-k and the
union run in one single-workgroup launch), and the plans must equal the
oracle's union of the ids."""
import numpy as np
import pytest

import oracle
import synth
from tests import harness as H

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not H.gpu_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

from routed_expert_execution_amd import moe  # noqa: E402


def _logits(kind, T, E, seed):
    g = np.random.default_rng(seed)
    if kind == "ties":
        return g.integers(-2, 3, size=(T, E)).astype(np.float32)
    if kind == "equal":
        return np.full((T, E), 0.5, np.float32)
    return g.standard_normal((T, E)).astype(np.float32)


def _run(ctx, T, fused, plan, **kw):
    k = ctx.top_k
    ids = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    w = torch.full((T, k), float("nan"), dtype=torch.float32, device="cuda")
    lo = torch.full((T, ctx.n_experts), float("nan"), dtype=torch.float32, device="cuda") \
        if "x" in kw else None
    if fused:
        moe.moe_route_union(ctx, ids, w, plan, logits_out=lo, **kw)
    else:
        moe.moe_route(ctx, ids, w, logits_out=lo, **kw)
        moe.moe_plan_union(ctx, ids, plan)
    torch.cuda.synchronize()
    n, experts, offsets, entries = plan.host()
    return (ids.cpu().numpy(), w.cpu().numpy().view(np.uint32), None if lo is None else lo.cpu().numpy().view(np.uint32),
            n, np.asarray(experts), np.asarray(offsets), np.asarray(entries))


def _same(a, b):
    for u, v in zip(a, b):
        if u is None:
            assert v is None
        else:
            assert np.array_equal(np.asarray(u), np.asarray(v))


@pytest.mark.parametrize("T", [0, 1, 2, 3, 4, 5, 16])
@pytest.mark.parametrize("norm", [1, 0])
def test_route_union_from_router_weights(T, norm):
    """Decode layer (256 experts, top-8, d 2048, bf16 x, fp32 router)."""
    wl = synth.workload("decode")
    ctx = H.make_ctx(wl, n_slots=1, max_tokens=max(T, 1), norm_topk=norm)
    x = H.torch_x(synth.activations(wl["seed"], T, wl["d"], "bf16", 900 + T), "bf16")
    wr = torch.from_numpy(synth.router_weights(wl["seed"], wl["E"], wl["d"])).cuda()
    plan_a, plan_b = moe.Plan(ctx, max(T, 1)), moe.Plan(ctx, max(T, 1))
    a = _run(ctx, T, False, plan_a, x=x, w_router=wr)
    for _ in range(3):  # repeated calls give the same result
        b = _run(ctx, T, True, plan_b, x=x, w_router=wr)
        _same(a, b)
    if T:
        r_n, r_exp, r_off, r_ent = oracle.plan_union(a[0], wl["E"])
        assert b[3] == r_n and np.array_equal(b[4], r_exp) and np.array_equal(b[5], r_off)
        assert np.array_equal(b[6], r_ent)
    else:
        assert b[3] == 0


@pytest.mark.parametrize("E,k", [(8, 2), (256, 8), (100, 7), (1024, 32)])
@pytest.mark.parametrize("kind", ["normal", "ties", "equal"])
@pytest.mark.parametrize("T", [1, 4])
def test_route_union_logits_in(E, k, kind, T):
    wl = dict(synth.workload("decode"), E=E, k=k)
    ctx = H.make_ctx(wl, n_slots=1, max_tokens=T)
    lg = torch.from_numpy(_logits(kind, T, E, E * 7 + k)).cuda()
    plan_a, plan_b = moe.Plan(ctx, T), moe.Plan(ctx, T)
    a = _run(ctx, T, False, plan_a, logits_in=lg)
    b = _run(ctx, T, True, plan_b, logits_in=lg)
    _same(a, b)
    r_ids, _ = oracle.topk(lg.cpu().numpy(), k)
    assert np.array_equal(b[0], r_ids)
    r_n, r_exp, r_off, r_ent = oracle.plan_union(r_ids, E)
    assert b[3] == r_n and np.array_equal(b[4], r_exp) and np.array_equal(b[5], r_off)
    assert np.array_equal(b[6], r_ent)


def test_route_union_validation():
    wl = synth.workload("decode")
    ctx = H.make_ctx(wl, n_slots=1, max_tokens=4)
    ids = torch.empty(2, wl["k"], dtype=torch.int32, device="cuda")
    w = torch.empty(2, wl["k"], dtype=torch.float32, device="cuda")
    plan = moe.Plan(ctx, 4)
    with pytest.raises(Exception):
        moe.moe_route_union(ctx, ids, w, plan)  # neither logits_in nor x / w_router
