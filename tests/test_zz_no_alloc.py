"""GPU: moe_expert_ffn_static (the chunk path's scratch in the library's fixed
device array, nothing allocated by the call) against moe_expert_ffn (the
context's workspace) through the C ABI: identical outputs bit for bit on two
calls in a row, the second with fewer tokens; a context created for at most
4 tokens (no chunk workspace of its own) runs chunks through it; a call whose
scratch would exceed the array is refused with nothing enqueued."""
import ctypes as C

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


def _say(*a):
    print(*a, flush=True)


def _setup(T_max, n_used=256):
    wl = synth.workload("prefill")
    E, k, d, f = wl["E"], wl["k"], wl["d"], wl["f"]
    cfg = moe.make_config(1, E, k, d, f, moe.MOE_Q8_0, n_used, T_max, device=-1)
    pb = moe.moe_payload_bytes(cfg)
    pool = torch.zeros(n_used * pb, dtype=torch.uint8, device="cuda")
    ctx = moe.Context(1, E, k, d, f, moe.MOE_Q8_0, n_used, T_max, device=0, slot_pool=pool)
    return wl, ctx, pool, pb


def _place(ctx, pool, pb, wl):
    for e in range(wl["E"]):
        pool[e * pb:(e + 1) * pb].copy_(torch.from_numpy(H.payload(ctx, synth.expert_record(
            wl["seed"], 0, e, wl["qtype"], wl["d"], wl["f"]))))
        moe.moe_slot_bind(ctx, 0, e, e)


def _inputs(wl, T, seed):
    lg = synth.zipf_gumbel_logits(wl["seed"] + seed, T, wl["E"], wl["zipf_s"])
    ids, w = oracle.topk(lg, wl["k"])
    x = H.torch_x(synth.activations(wl["seed"], T, wl["d"], "bf16", seed), "bf16")
    return torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda(), x


def _call(ctx, fn_static, x, plan, w, sh, prec):
    T = x.shape[0]
    y = torch.full((T, ctx.d_model), float("nan"), dtype=torch.float32, device="cuda")
    moe.moe_expert_ffn(ctx, 0, x, plan, w, y, shared_payload=sh, prec=prec, static=fn_static)
    assert moe.moe_check(ctx) == moe.MOE_OK
    return y


@pytest.mark.parametrize("prec", [moe.MOE_PREC_BF16, moe.MOE_PREC_F32])
def test_static_scratch_matches_workspace(prec):
    wl, ctx, pool, pb = _setup(512)
    _place(ctx, pool, pb, wl)
    sh = H.device_payload(ctx, synth.expert_record(wl["seed"], 0, 0, wl["qtype"], wl["d"], wl["f"], shared=True))
    for T, seed in ((512, 1), (100, 2)):  # the second call smaller than the first
        _say("static scratch", prec, T)
        ids, w, x = _inputs(wl, T, seed)
        plan = moe.Plan(ctx, T)
        moe.moe_plan_union(ctx, ids, plan)
        y_ws = _call(ctx, False, x, plan, w, sh, prec)
        y_st = _call(ctx, True, x, plan, w, sh, prec)
        assert torch.isfinite(y_st).all()
        assert torch.equal(y_st.view(torch.int32), y_ws.view(torch.int32)), f"T={T}: outputs differ"


def test_small_context_runs_chunks_through_static_scratch():
    wl, big, pool, pb = _setup(300)
    _place(big, pool, pb, wl)
    _, small, spool, _ = _setup(4)
    _place(small, spool, pb, wl)
    sh = H.device_payload(big, synth.expert_record(wl["seed"], 0, 0, wl["qtype"], wl["d"], wl["f"], shared=True))
    for T, seed in ((300, 3), (37, 4)):
        ids, w, x = _inputs(wl, T, seed)
        plan_b, plan_s = moe.Plan(big, T), moe.Plan(small, T)
        moe.moe_plan_union(big, ids, plan_b)
        # the small context takes no union of T > 4 tokens itself: the same plan
        # arrays (same n_experts, same T) from the big one's union
        plan_s._buf.copy_(plan_b._buf)
        y_ref = _call(big, False, x, plan_b, w, sh, moe.MOE_PREC_BF16)
        y_st = _call(small, True, x, plan_s, w, sh, moe.MOE_PREC_BF16)
        assert torch.equal(y_st.view(torch.int32), y_ref.view(torch.int32)), f"T={T}: outputs differ"


def test_static_scratch_refuses_oversize_call():
    wl, ctx, pool, pb = _setup(4, n_used=1)
    T = 4096  # (T k + T) rows of d_model fp32 partials alone exceed the array
    x = torch.zeros(T, wl["d"], dtype=torch.bfloat16, device="cuda")
    w = torch.zeros(T, wl["k"], dtype=torch.float32, device="cuda")
    y = torch.zeros(T, wl["d"], dtype=torch.float32, device="cuda")
    plan = moe.Plan(ctx, T)
    lib = moe.library()
    st = lib.moe_expert_ffn_static(ctx.handle, 0, x.data_ptr(), moe.MOE_BF16, T, C.byref(plan.c), w.data_ptr(),
                                   None, moe.MOE_PREC_BF16, y.data_ptr(), None)
    assert st == moe.MOE_EINVAL
    assert b"static array" in lib.moe_last_error(ctx.handle)
    torch.cuda.synchronize()
    assert moe.moe_check(ctx) == moe.MOE_OK
    assert (y == 0).all()
