"""Test harness: puts synthetic experts into slots and compares outputs.

Calls the product only through its binding (routed_expert_execution_amd.moe)
and the oracle only through oracle/; holds none of the method's arithmetic.
"""
from __future__ import annotations

import numpy as np

import synth

QT = {synth.Q8_0: 0, synth.Q4_0: 1}


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def torch_x(x: np.ndarray, dtype: str, device="cuda"):
    """synth activations (float32, or bf16 bits as uint16) -> torch tensor on device."""
    import torch
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint16).view(np.int16)).view(torch.bfloat16).to(device)


def make_ctx(wl: dict, n_slots: int | None = None, max_tokens: int | None = None, norm_topk: int = 1,
             n_layers: int | None = None):
    import torch
    from routed_expert_execution_amd import moe
    n_slots = n_slots or wl["n_slots"]
    cfg = moe.make_config(n_layers or wl["n_layers"], wl["E"], wl["k"], wl["d"], wl["f"],
                          QT[wl["qtype"]], n_slots, max_tokens or wl["T"], device=-1)
    pb = moe.moe_payload_bytes(cfg)
    pool = torch.zeros(n_slots * pb, dtype=torch.uint8, device="cuda")
    return moe.Context(n_layers or wl["n_layers"], wl["E"], wl["k"], wl["d"], wl["f"], QT[wl["qtype"]],
                       n_slots, max_tokens or wl["T"], norm_topk=norm_topk, device=0, slot_pool=pool)


def payload(ctx, rec: np.ndarray) -> np.ndarray:
    from routed_expert_execution_amd import moe
    return moe.moe_pack_expert(ctx.cfg, rec)


def put_expert(ctx, slot: int, rec: np.ndarray) -> None:
    import torch
    ctx.slot(slot).copy_(torch.from_numpy(payload(ctx, rec)))


def device_payload(ctx, rec: np.ndarray):
    import torch
    return torch.from_numpy(payload(ctx, rec)).cuda()


def max_rel_row_err(y: np.ndarray, ref: np.ndarray) -> float:
    """Per token row: max_i |y - ref| / max_i |ref|; the largest over rows."""
    y = np.asarray(y, np.float64).reshape(ref.shape[0], -1)
    ref = np.asarray(ref, np.float64).reshape(ref.shape[0], -1)
    den = np.maximum(np.abs(ref).max(axis=1), 1e-30)
    return float((np.abs(y - ref).max(axis=1) / den).max())


def elementwise_stats(y: np.ndarray, ref: np.ndarray) -> dict:
    """Element-wise error statistics beside the per-row metric: the largest
    absolute error, the largest error relative to its own element (over
    elements at least 1e-3 of their row's largest magnitude), the relative
    RMS error over all elements, and the fraction of elements whose error
    exceeds 1e-3 of their row's largest magnitude."""
    y = np.asarray(y, np.float64).reshape(ref.shape[0], -1)
    ref = np.asarray(ref, np.float64).reshape(ref.shape[0], -1)
    err = np.abs(y - ref)
    rowmax = np.maximum(np.abs(ref).max(axis=1, keepdims=True), 1e-30)
    big = np.abs(ref) >= 1e-3 * rowmax
    return {
        "max_rel_row": float((err.max(axis=1) / rowmax[:, 0]).max()),
        "max_abs": float(err.max()),
        "max_rel_elem": float((err[big] / np.abs(ref[big])).max()) if big.any() else 0.0,
        "rel_rms": float(np.sqrt((err ** 2).sum() / max((ref ** 2).sum(), 1e-300))),
        "frac_over_1e-3_of_row": float((err > 1e-3 * rowmax).mean()),
    }
