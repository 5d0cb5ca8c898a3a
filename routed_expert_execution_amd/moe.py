"""Python binding of libmoe.so (include/moe.h): argument marshalling only.

Every function has the name of the C entry point it calls.  Device buffers
are torch tensors on the context's GPU; host buffers are numpy arrays or
pinned torch tensors.  Nothing here computes any part of the routed-expert
path: each call checks types, shapes and devices, then hands raw pointers to
the library.  A missing library raises ImportError at import time; a failing
call raises MoeError with the library's own message.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

MOE_OK, MOE_EINVAL, MOE_ENOMEM, MOE_EHIP, MOE_ENOSLOT, MOE_EMISS, MOE_EBUSY, MOE_ETIMEOUT = 0, -1, -2, -3, -4, -5, -6, -7
MOE_Q8_0, MOE_Q4_0 = 0, 1
MOE_F32, MOE_BF16 = 0, 1
MOE_PREC_F32, MOE_PREC_BF16 = 0, 1
MOE_MAX_STAGE_STREAMS = 8


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


class moe_config(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("n_experts", C.c_int32), ("top_k", C.c_int32),
                ("d_model", C.c_int32), ("d_ff", C.c_int32), ("qtype", C.c_int32),
                ("n_slots", C.c_int32), ("max_tokens", C.c_int32), ("norm_topk", C.c_int32),
                ("gemm_min_tokens", C.c_int32), ("device", C.c_int32), ("reserved", C.c_int32),
                ("slot_pool", C.c_void_p)]


class moe_plan(C.Structure):
    _fields_ = [("n_active", C.c_void_p), ("experts", C.c_void_p), ("offsets", C.c_void_p),
                ("entries", C.c_void_p)]


def _load() -> C.CDLL:
    # torch ships its own HIP runtime.  Loading torch first makes libmoe's
    # libamdhip64.so.7 dependency resolve (by soname) to that same runtime;
    # the other order maps two HIP/HSA runtimes into the process.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m routed_expert_execution_amd.build`")
    lib = C.CDLL(LIB_PATH)
    P, I32, I64, S = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
    cfgp = C.POINTER(moe_config)
    planp = C.POINTER(moe_plan)
    sig = {
        "moe_payload_bytes": (S, [cfgp]),
        "moe_plan_bytes": (C.c_int, [cfgp, I64, C.POINTER(S)]),
        "moe_pack_expert": (C.c_int, [cfgp, P, P]),
        "moe_unpack_expert": (C.c_int, [cfgp, P, P]),
        "moe_create": (C.c_int, [cfgp, C.POINTER(P)]),
        "moe_destroy": (None, [P]),
        "moe_last_error": (C.c_char_p, [P]),
        "moe_status_string": (C.c_char_p, [C.c_int]),
        "moe_route": (C.c_int, [P, P, I32, P, P, I64, P, P, P, P]),
        "moe_plan_union": (C.c_int, [P, P, I64, planp, P]),
        "moe_route_union": (C.c_int, [P, P, C.c_int32, P, P, I64, P, P, P, planp, P]),
        "moe_slot_map": (C.c_int, [P, I32, P, I32, P, P]),
        "moe_slot_fill": (C.c_int, [P, I32, I32, I32, P, P]),
        "moe_slot_stage": (C.c_int, [P, I32, P, I32, P, P, P, P, I32]),
        "moe_slot_pull": (C.c_int, [P, I32, P, I32, P, P, P, P]),
        "moe_route_pull": (C.c_int, [P, I32, P, I32, P, P, I64, P, P, P, planp, P, P, P, P, P, P]),
        "moe_slot_prefetch": (C.c_int, [P, I32, P, I32, I64, P, P, P]),
        "moe_prefetch_stats": (C.c_int, [P, C.POINTER(C.c_uint64)]),
        "moe_prefetch_next": (C.c_int, [P, I32, P, I64, C.c_float, C.c_float, P, P, P, P]),
        "moe_slot_release": (C.c_int, [P, I32, P]),
        "moe_slot_bind": (C.c_int, [P, I32, I32, I32, P]),
        "moe_expert_ffn": (C.c_int, [P, I32, P, I32, I64, planp, P, P, I32, P, P]),
        "moe_expert_ffn_static": (C.c_int, [P, I32, P, I32, I64, planp, P, P, I32, P, P]),
        "moe_expert_ffn_split": (C.c_int, [P, I32, P, I32, I64, planp, P, P, I32, P, I32, P, P, P]),
        "moe_route_ffn": (C.c_int, [P, I32, P, I32, P, P, I64, P, P, planp, P, I32, P, P]),
        "moe_dequant": (C.c_int, [P, P, I32, P, P]),
        "moe_stats": (C.c_int, [P, C.POINTER(C.c_uint64)]),
        "moe_check": (C.c_int, [P, P]),
        "moe_page_table": (C.c_int, [P, C.POINTER(P)]),
        "moe_route_splits": (C.c_int, [P, C.POINTER(C.c_uint64)]),
        "moe_hidden_rows": (C.c_int, [P, C.POINTER(P), C.POINTER(I32)]),
        "moe_probe_read": (C.c_int, [P, I64, I32, P, P]),
        "moe_probe_mfma": (C.c_int, [I32, I32, I32, P, C.POINTER(I64), P]),
        "moe_probe_lds": (C.c_int, [I32, I32, P, C.POINTER(I64), P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()
EXPORTS = ("moe_payload_bytes", "moe_plan_bytes", "moe_pack_expert", "moe_unpack_expert", "moe_create",
           "moe_destroy", "moe_last_error", "moe_status_string", "moe_route", "moe_plan_union", "moe_route_union",
           "moe_slot_map", "moe_slot_prefetch", "moe_prefetch_stats", "moe_prefetch_next", "moe_slot_fill", "moe_slot_stage", "moe_slot_pull", "moe_route_pull", "moe_slot_release",
           "moe_slot_bind", "moe_expert_ffn", "moe_expert_ffn_static", "moe_expert_ffn_split",
           "moe_route_ffn", "moe_dequant", "moe_stats", "moe_check", "moe_page_table", "moe_route_splits", "moe_hidden_rows", "moe_probe_read",
           "moe_probe_mfma", "moe_probe_lds")


def library() -> C.CDLL:
    return _lib


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------

def _ptr(t) -> int | None:
    """Raw address of a torch tensor / numpy array (None stays None)."""
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        if not t.flags["C_CONTIGUOUS"]:
            raise ValueError("numpy array must be C-contiguous")
        return t.ctypes.data
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check_dev(ctx: "Context", *tensors):
    for t in tensors:
        if t is None:
            continue
        if not t.is_cuda or t.device.index != ctx.device:
            raise ValueError(f"tensor must be on cuda:{ctx.device}")


def _x_dtype(x) -> int:
    import torch
    if x.dtype == torch.float32:
        return MOE_F32
    if x.dtype == torch.bfloat16:
        return MOE_BF16
    raise ValueError("x must be float32 or bfloat16")


def _call(ctx, status: int) -> None:
    if status != MOE_OK:
        msg = _lib.moe_last_error(ctx.handle if ctx is not None else None)
        text = (msg or b"").decode() or _lib.moe_status_string(status).decode()
        raise MoeError(status, text)


def make_config(n_layers: int, n_experts: int, top_k: int, d_model: int, d_ff: int, qtype: int,
                n_slots: int, max_tokens: int, norm_topk: int = 1, gemm_min_tokens: int = 16,
                device: int = 0, slot_pool: int | None = None) -> moe_config:
    return moe_config(n_layers, n_experts, top_k, d_model, d_ff, qtype, n_slots, max_tokens, norm_topk,
                      gemm_min_tokens, device, 0, slot_pool)


def moe_payload_bytes(cfg: moe_config) -> int:
    return int(_lib.moe_payload_bytes(C.byref(cfg)))


def moe_pack_expert(cfg: moe_config, gguf_blocks: np.ndarray, out: np.ndarray | None = None) -> np.ndarray:
    n = moe_payload_bytes(cfg)
    src = np.ascontiguousarray(gguf_blocks, dtype=np.uint8).reshape(-1)
    if src.size != n:
        raise ValueError(f"expected {n} bytes of GGUF blocks, got {src.size}")
    dst = np.empty(n, dtype=np.uint8) if out is None else out
    _call(None, _lib.moe_pack_expert(C.byref(cfg), src.ctypes.data, _ptr(dst)))
    return dst


def moe_unpack_expert(cfg: moe_config, payload: np.ndarray) -> np.ndarray:
    n = moe_payload_bytes(cfg)
    src = np.ascontiguousarray(payload, dtype=np.uint8).reshape(-1)
    if src.size != n:
        raise ValueError(f"expected {n} payload bytes, got {src.size}")
    dst = np.empty(n, dtype=np.uint8)
    _call(None, _lib.moe_unpack_expert(C.byref(cfg), src.ctypes.data, dst.ctypes.data))
    return dst


class Context:
    """Owns one moe_ctx.  slot_pool: a uint8 CUDA tensor of n_slots * payload bytes
    (kept referenced here), or None together with device=-1 for a host-only context."""

    def __init__(self, n_layers, n_experts, top_k, d_model, d_ff, qtype, n_slots, max_tokens,
                 norm_topk=1, gemm_min_tokens=16, device=0, slot_pool=None):
        self.device = device
        self.slot_pool = slot_pool
        self.cfg = make_config(n_layers, n_experts, top_k, d_model, d_ff, qtype, n_slots, max_tokens,
                               norm_topk, gemm_min_tokens, device, _ptr(slot_pool))
        self.payload_bytes = moe_payload_bytes(self.cfg)
        if device >= 0:
            if slot_pool is None:
                raise ValueError("a device context needs a slot_pool tensor")
            _check_dev(self, slot_pool)
            if slot_pool.numel() * slot_pool.element_size() < n_slots * self.payload_bytes:
                raise ValueError("slot_pool is smaller than n_slots * payload bytes")
        h = C.c_void_p()
        st = _lib.moe_create(C.byref(self.cfg), C.byref(h))
        if st != MOE_OK:
            raise MoeError(st, f"moe_create: {_lib.moe_status_string(st).decode()}")
        self.handle = h.value
        self.n_experts, self.top_k, self.d_model, self.d_ff = n_experts, top_k, d_model, d_ff
        self.n_slots, self.max_tokens = n_slots, max_tokens

    def close(self):
        if getattr(self, "handle", None):
            _lib.moe_destroy(self.handle)
            self.handle = None

    def __del__(self):
        self.close()

    def slot(self, s: int):
        """View of slot s of the pool (uint8 tensor)."""
        n = self.payload_bytes
        return self.slot_pool.view(-1)[s * n:(s + 1) * n]


class Plan:
    """Device arrays of one moe_plan for up to T tokens."""

    def __init__(self, ctx: Context, T: int):
        import torch
        dev = torch.device("cuda", ctx.device)
        E = ctx.n_experts
        up = lambda n: (n + 63) // 64 * 64  # noqa: E731  (256-byte starts)
        # one allocation; n_active sits in the word just before experts, so the
        # two come back in one copy
        o_ex, o_off = 64, 64 + up(E)
        o_ent = o_off + up(E + 1)
        self._buf = torch.zeros(o_ent + max(1, T * ctx.top_k), dtype=torch.int32, device=dev)
        self.n_active = self._buf[o_ex - 1:o_ex]
        self.experts = self._buf[o_ex:o_ex + E]
        self.offsets = self._buf[o_off:o_off + E + 1]
        self.entries = self._buf[o_ent:]
        self._head = self._buf[o_ex - 1:o_ex + E]
        self._pinned = torch.empty(1 + E, dtype=torch.int32).pin_memory()
        self.c = moe_plan(_ptr(self.n_active), _ptr(self.experts), _ptr(self.offsets), _ptr(self.entries))

    def experts_host(self, stream=None, spin=False):
        """(n_active, experts[:n_active]) with one copy into pinned memory, after
        the work enqueued on `stream` (default: the current stream).  spin: poll
        an event for the copy instead of a blocking synchronise."""
        import torch
        st = stream or torch.cuda.current_stream(self._buf.device)
        with torch.cuda.stream(st):
            self._pinned.copy_(self._head, non_blocking=True)
        if spin:
            if not hasattr(self, "_ev"):
                self._ev = torch.cuda.Event()
            self._ev.record(st)
            while not self._ev.query():
                pass
        else:
            st.synchronize()
        h = self._pinned.numpy()
        n = int(h[0])
        return n, h[1:1 + n].copy()

    def host(self):
        """(n_active, experts, offsets, entries) copied to numpy (synchronises)."""
        n = int(self.n_active.item())
        off = self.offsets[:n + 1].cpu().numpy()
        return n, self.experts[:n].cpu().numpy(), off, self.entries[:int(off[-1]) if n else 0].cpu().numpy()


def moe_route(ctx: Context, topk_ids, topk_w, x=None, w_router=None, logits_in=None, logits_out=None,
              stream=None) -> None:
    T = topk_ids.shape[0]
    xd = _route_args(ctx, topk_ids, topk_w, x, w_router, logits_in, logits_out)
    _call(ctx, _lib.moe_route(ctx.handle, _ptr(x), xd, _ptr(w_router), _ptr(logits_in), T, _ptr(topk_ids),
                              _ptr(topk_w), _ptr(logits_out), _stream(stream)))


def _route_args(ctx: Context, topk_ids, topk_w, x, w_router, logits_in, logits_out) -> int:
    """Shape and dtype checks shared by moe_route and moe_route_union; returns x's dtype code."""
    import torch
    T = topk_ids.shape[0]
    if topk_ids.dtype != torch.int32 or topk_w.dtype != torch.float32:
        raise ValueError("topk_ids must be int32 and topk_w float32")
    if tuple(topk_ids.shape) != (T, ctx.top_k) or tuple(topk_w.shape) != (T, ctx.top_k):
        raise ValueError("topk_ids / topk_w must be [T, top_k]")
    _check_dev(ctx, topk_ids, topk_w, x, w_router, logits_in, logits_out)
    xd = MOE_F32
    if logits_in is not None:
        if logits_in.dtype != torch.float32 or tuple(logits_in.shape) != (T, ctx.n_experts):
            raise ValueError("logits_in must be float32 [T, n_experts]")
    else:
        xd = _x_dtype(x)
        if tuple(x.shape) != (T, ctx.d_model) or w_router.dtype != torch.float32 or \
                tuple(w_router.shape) != (ctx.n_experts, ctx.d_model):
            raise ValueError("x must be [T, d_model]; w_router float32 [n_experts, d_model]")
    if logits_out is not None and (logits_out.dtype != torch.float32 or tuple(logits_out.shape) != (T, ctx.n_experts)):
        raise ValueError("logits_out must be float32 [T, n_experts]")
    return xd


def moe_route_union(ctx: Context, topk_ids, topk_w, plan: Plan, x=None, w_router=None, logits_in=None,
                    logits_out=None, stream=None) -> None:
    T = topk_ids.shape[0]
    xd = _route_args(ctx, topk_ids, topk_w, x, w_router, logits_in, logits_out)
    if plan.entries.numel() < T * ctx.top_k:
        raise ValueError("plan is too small for T")
    _call(ctx, _lib.moe_route_union(ctx.handle, _ptr(x), xd, _ptr(w_router), _ptr(logits_in), T, _ptr(topk_ids),
                                    _ptr(topk_w), _ptr(logits_out), C.byref(plan.c), _stream(stream)))


def moe_plan_union(ctx: Context, topk_ids, plan: Plan, stream=None) -> None:
    import torch
    if topk_ids.dtype != torch.int32 or topk_ids.dim() != 2 or topk_ids.shape[1] != ctx.top_k:
        raise ValueError("topk_ids must be int32 [T, top_k]")
    if plan.entries.numel() < topk_ids.shape[0] * ctx.top_k:
        raise ValueError("plan is too small for T")
    _check_dev(ctx, topk_ids)
    _call(ctx, _lib.moe_plan_union(ctx.handle, _ptr(topk_ids), topk_ids.shape[0], C.byref(plan.c),
                                   _stream(stream)))


def moe_slot_map(ctx: Context, layer: int, experts) -> tuple:
    e = np.ascontiguousarray(experts, dtype=np.int32).reshape(-1)
    slots = np.empty(e.size, dtype=np.int32)
    miss = np.empty(e.size, dtype=np.uint8)
    _call(ctx, _lib.moe_slot_map(ctx.handle, layer, e.ctypes.data, e.size, slots.ctypes.data, miss.ctypes.data))
    return slots, miss.astype(bool)


def moe_slot_prefetch(ctx: Context, layer: int, experts, max_bytes: int) -> tuple:
    """Map predicted experts (priority order) without pinning; returns (slots,
    fill) for the ones processed (fill: the caller now calls moe_slot_fill)."""
    e = np.ascontiguousarray(experts, dtype=np.int32).reshape(-1)
    slots = np.empty(e.size, dtype=np.int32)
    fill = np.empty(e.size, dtype=np.uint8)
    done = C.c_int32()
    _call(ctx, _lib.moe_slot_prefetch(ctx.handle, layer, e.ctypes.data, e.size, int(max_bytes), slots.ctypes.data,
                                      fill.ctypes.data, C.byref(done)))
    return slots[: done.value], fill[: done.value].astype(bool)


def moe_prefetch_stats(ctx: Context) -> dict:
    out = (C.c_uint64 * 4)()
    _call(ctx, _lib.moe_prefetch_stats(ctx.handle, out))
    return dict(fills=out[0], useful=out[1], wasted=out[2], bytes=out[3])


def moe_prefetch_next(ctx: Context, layer: int, table: np.ndarray, max_bytes: int, min_weight: float = 0.20,
                      min_transition: float = 0.0, stream=None) -> tuple:
    """After moe_route_pull of `layer`: predict layer (layer + 1) % n_layers's
    experts (the previous step's at weight >= min_weight, then transition
    scores >= min_transition; 0 turns those off) and queue copies of the
    missing ones on `stream` from `table` (payload_table of that layer, pinned
    host payloads); returns (experts, filled) of the candidates processed, in
    priority order."""
    _table(ctx, table)
    n = C.c_int32()
    ex = np.empty(ctx.n_experts, dtype=np.int32)
    fill = np.empty(ctx.n_experts, dtype=np.uint8)
    _call(ctx, _lib.moe_prefetch_next(ctx.handle, layer, table.ctypes.data, int(max_bytes), float(min_weight),
                                      float(min_transition), _stream(stream), C.byref(n), ex.ctypes.data,
                                      fill.ctypes.data))
    return ex[: n.value].copy(), fill[: n.value].astype(bool)


def moe_slot_fill(ctx: Context, layer: int, expert: int, slot: int, host_payload, stream=None) -> None:
    """host_payload: pinned uint8 torch tensor (CPU) of payload bytes."""
    if host_payload.numel() * host_payload.element_size() < ctx.payload_bytes:
        raise ValueError("host payload too small")
    _call(ctx, _lib.moe_slot_fill(ctx.handle, layer, expert, slot, _ptr(host_payload), _stream(stream)))


def payload_table(ctx: Context, payloads) -> np.ndarray:
    """Addresses (int64 [n_experts]) of uint8 payload tensors indexed by expert
    id (None: never staged) for moe_slot_stage (pinned host tensors) or
    moe_slot_pull (pinned host or CUDA tensors)."""
    t = np.zeros(ctx.n_experts, dtype=np.int64)
    for e, p in enumerate(payloads):
        if p is None:
            continue
        if not (p.is_pinned() or p.is_cuda) or p.numel() * p.element_size() < ctx.payload_bytes:
            raise ValueError(f"payload of expert {e}: not pinned (or on the GPU), or too small")
        t[e] = _ptr(p)
    return t


def _table(ctx, table):
    if table.dtype != np.int64 or table.size != ctx.n_experts or not table.flags.c_contiguous:
        raise ValueError("table: int64 [n_experts] from payload_table")


def moe_slot_stage(ctx: Context, layer: int, experts, table: np.ndarray, streams) -> tuple:
    """moe_slot_map plus the fills of its misses from `table` (payload_table),
    the copies alternating over `streams`; returns (slots, miss)."""
    e = np.ascontiguousarray(experts, dtype=np.int32).reshape(-1)
    _table(ctx, table)
    slots = np.empty(e.size, dtype=np.int32)
    miss = np.empty(e.size, dtype=np.uint8)
    st = (C.c_void_p * max(1, len(streams)))(*[_stream(x) for x in streams])
    _call(ctx, _lib.moe_slot_stage(ctx.handle, layer, e.ctypes.data, e.size, table.ctypes.data, slots.ctypes.data,
                                   miss.ctypes.data, st, len(streams)))
    return slots, miss.astype(bool)


def moe_slot_pull(ctx: Context, layer: int, experts, table: np.ndarray, stream=None) -> tuple:
    """moe_slot_map, then kernels on `stream` copy the misses from `table`
    (payload_table) into their slots; returns (slots, miss)."""
    e = np.ascontiguousarray(experts, dtype=np.int32).reshape(-1)
    _table(ctx, table)
    slots = np.empty(e.size, dtype=np.int32)
    miss = np.empty(e.size, dtype=np.uint8)
    _call(ctx, _lib.moe_slot_pull(ctx.handle, layer, e.ctypes.data, e.size, table.ctypes.data, slots.ctypes.data,
                                  miss.ctypes.data, _stream(stream)))
    return slots, miss.astype(bool)


def moe_route_pull(ctx: Context, layer: int, topk_ids, topk_w, plan: "Plan", table: np.ndarray, *, x=None,
                   w_router=None, logits_in=None, logits_out=None, stream=None) -> tuple:
    """moe_route_union, then moe_slot_pull of the step's experts from `table`
    (payload_table); returns (experts, slots, miss) for the step's units."""
    _table(ctx, table)
    T = int(topk_ids.shape[0])
    xd = _route_args(ctx, topk_ids, topk_w, x, w_router, logits_in, logits_out)
    if plan.entries.numel() < T * ctx.top_k:
        raise ValueError("plan is too small for T")
    n = C.c_int32()
    ex = np.empty(ctx.n_experts, dtype=np.int32)
    slots = np.empty(ctx.n_experts, dtype=np.int32)
    miss = np.empty(ctx.n_experts, dtype=np.uint8)
    _call(ctx, _lib.moe_route_pull(ctx.handle, layer, _ptr(x), xd, _ptr(w_router), _ptr(logits_in), T,
                                   _ptr(topk_ids), _ptr(topk_w), _ptr(logits_out), C.byref(plan.c), table.ctypes.data,
                                   C.byref(n), ex.ctypes.data, slots.ctypes.data, miss.ctypes.data, _stream(stream)))
    k = n.value
    return ex[:k], slots[:k], miss[:k].astype(bool)


def moe_slot_release(ctx: Context, layer: int, stream=None) -> None:
    _call(ctx, _lib.moe_slot_release(ctx.handle, layer, _stream(stream) if ctx.device >= 0 else None))


def moe_slot_bind(ctx: Context, layer: int, expert: int, slot: int, stream=None) -> None:
    _call(ctx, _lib.moe_slot_bind(ctx.handle, layer, expert, slot, _stream(stream)))


def moe_expert_ffn(ctx: Context, layer: int, x, plan: Plan, topk_w, y, shared_payload=None,
                   prec: int = MOE_PREC_F32, stream=None, static: bool = False) -> None:
    """static: call moe_expert_ffn_static (the chunk path's scratch in the
    library's fixed device array instead of the context's workspace)."""
    import torch
    T = x.shape[0]
    if tuple(x.shape) != (T, ctx.d_model) or tuple(y.shape) != (T, ctx.d_model) or y.dtype != torch.float32:
        raise ValueError("x must be [T, d_model]; y float32 [T, d_model]")
    if topk_w.dtype != torch.float32 or tuple(topk_w.shape) != (T, ctx.top_k):
        raise ValueError("topk_w must be float32 [T, top_k]")
    if plan.entries.numel() < T * ctx.top_k:
        raise ValueError("plan is too small for T")
    if shared_payload is not None and shared_payload.numel() * shared_payload.element_size() < ctx.payload_bytes:
        raise ValueError("shared payload too small")
    _check_dev(ctx, x, topk_w, y, shared_payload)
    fn = _lib.moe_expert_ffn_static if static else _lib.moe_expert_ffn
    _call(ctx, fn(ctx.handle, layer, _ptr(x), _x_dtype(x), T, C.byref(plan.c), _ptr(topk_w),
                  _ptr(shared_payload), prec, _ptr(y), _stream(stream)))


def moe_expert_ffn_split(ctx: Context, layer: int, x, plan: Plan, topk_w, y, miss_experts, shared_payload=None,
                         prec: int = MOE_PREC_F32, side=None, stream=None) -> None:
    """Hit/miss split of a one-token step, right after moe_route_pull of the
    same layer: the resident units on `side`, the copied ones (miss_experts)
    on `stream` after their copies, merged in plan order."""
    import torch
    if tuple(x.shape) != (1, ctx.d_model) or tuple(y.shape) != (1, ctx.d_model) or y.dtype != torch.float32:
        raise ValueError("x must be [1, d_model]; y float32 [1, d_model]")
    if topk_w.dtype != torch.float32 or tuple(topk_w.shape) != (1, ctx.top_k):
        raise ValueError("topk_w must be float32 [1, top_k]")
    if plan.entries.numel() < ctx.top_k:
        raise ValueError("plan is too small for T")
    if shared_payload is not None and shared_payload.numel() * shared_payload.element_size() < ctx.payload_bytes:
        raise ValueError("shared payload too small")
    _check_dev(ctx, x, topk_w, y, shared_payload)
    m = np.ascontiguousarray(np.asarray(miss_experts, dtype=np.int32).reshape(-1))
    _call(ctx, _lib.moe_expert_ffn_split(ctx.handle, layer, _ptr(x), _x_dtype(x), 1, C.byref(plan.c), _ptr(topk_w),
                                         _ptr(shared_payload), prec, m.ctypes.data if m.size else None, m.size,
                                         _ptr(y), _stream(side), _stream(stream)))


def moe_route_ffn(ctx: Context, layer: int, x, topk_ids, topk_w, plan: Plan, y, w_router=None, logits_in=None,
                  shared_payload=None, prec: int = MOE_PREC_F32, stream=None) -> None:
    """Route (from x . w_router^T, or from logits_in), union and expert FFN of at
    most 4 tokens in one launch; topk_ids, topk_w and plan are outputs."""
    import torch
    T = x.shape[0]
    _route_args(ctx, topk_ids, topk_w, x if logits_in is None else None, w_router, logits_in, None)
    if tuple(x.shape) != (T, ctx.d_model) or tuple(y.shape) != (T, ctx.d_model) or y.dtype != torch.float32:
        raise ValueError("x must be [T, d_model]; y float32 [T, d_model]")
    if plan.entries.numel() < T * ctx.top_k:
        raise ValueError("plan is too small for T")
    if shared_payload is not None and shared_payload.numel() * shared_payload.element_size() < ctx.payload_bytes:
        raise ValueError("shared payload too small")
    _check_dev(ctx, x, y, shared_payload)
    _call(ctx, _lib.moe_route_ffn(ctx.handle, layer, _ptr(x), _x_dtype(x), _ptr(w_router), _ptr(logits_in), T,
                                  _ptr(topk_ids), _ptr(topk_w), C.byref(plan.c), _ptr(shared_payload), prec,
                                  _ptr(y), _stream(stream)))


def moe_dequant(ctx: Context, payload, out, prec: int = MOE_PREC_F32, stream=None) -> None:
    import torch
    if out.dtype != torch.float32 or out.numel() != 3 * ctx.d_ff * ctx.d_model:
        raise ValueError("out must be float32 with 3 * d_ff * d_model elements")
    _check_dev(ctx, payload, out)
    _call(ctx, _lib.moe_dequant(ctx.handle, _ptr(payload), prec, _ptr(out), _stream(stream)))


def moe_stats(ctx: Context) -> dict:
    out = (C.c_uint64 * 5)()
    _call(ctx, _lib.moe_stats(ctx.handle, out))
    return dict(hits=out[0], misses=out[1], bytes_staged=out[2], evictions=out[3], fills=out[4])


def moe_check(ctx: Context, stream=None) -> int:
    """Returns the status (MOE_OK, MOE_EMISS, MOE_ETIMEOUT, ...) without raising."""
    return int(_lib.moe_check(ctx.handle, _stream(stream)))


def moe_page_table(ctx: Context) -> np.ndarray:
    """Copy of the page table [n_layers, n_experts] (synchronises the device)."""
    import torch
    p = C.c_void_p()
    _call(ctx, _lib.moe_page_table(ctx.handle, C.byref(p)))
    out = np.empty((ctx.cfg.n_layers, ctx.n_experts), dtype=np.int32)
    torch.cuda.synchronize(ctx.device)
    hip = C.CDLL("libamdhip64.so")
    hip.hipMemcpy.restype = C.c_int
    hip.hipMemcpy.argtypes = [C.c_void_p, C.c_void_p, C.c_size_t, C.c_int]
    st = hip.hipMemcpy(out.ctypes.data, p.value, out.nbytes, 2)  # hipMemcpyDeviceToHost
    if st != 0:
        raise MoeError(MOE_EHIP, f"hipMemcpy of the page table failed ({st})")
    return out


def moe_route_splits(ctx: Context) -> int:
    """moe_route_ffn calls (with router weights) that took the two-launch path."""
    v = C.c_uint64()
    _call(ctx, _lib.moe_route_splits(ctx.handle, C.byref(v)))
    return int(v.value)


def moe_hidden_rows(ctx: Context, rows: int):
    """Copy of the first `rows` hidden rows the last chunk call (more than 4
    tokens) left in the workspace, as float32 [rows, d_ff] (bf16 codes widened
    exactly); synchronises the device."""
    import torch
    p = C.c_void_p()
    eb = C.c_int32()
    _call(ctx, _lib.moe_hidden_rows(ctx.handle, C.byref(p), C.byref(eb)))
    f = ctx.cfg.d_ff
    raw = np.empty(rows * f * eb.value, dtype=np.uint8)
    torch.cuda.synchronize(ctx.device)
    hip = C.CDLL("libamdhip64.so")
    hip.hipMemcpy.restype = C.c_int
    hip.hipMemcpy.argtypes = [C.c_void_p, C.c_void_p, C.c_size_t, C.c_int]
    st = hip.hipMemcpy(raw.ctypes.data, p.value, raw.nbytes, 2)  # hipMemcpyDeviceToHost
    if st != 0:
        raise MoeError(MOE_EHIP, f"hipMemcpy of the hidden rows failed ({st})")
    if eb.value == 4:
        return raw.view(np.float32).reshape(rows, f).copy()
    return (raw.view(np.uint16).astype(np.uint32) << 16).view(np.float32).reshape(rows, f)


def moe_probe_read(src, sink, workgroups: int = 0, stream=None) -> None:
    """One streaming-read launch over every byte of the device tensor src."""
    n = src.numel() * src.element_size()
    if _lib.moe_probe_read(_ptr(src), n, workgroups, _ptr(sink), _stream(stream)) != MOE_OK:
        raise ValueError("moe_probe_read: bad arguments (bytes must be a positive multiple of 16)")


def moe_probe_lds(iters: int, grid: int, sink, stream=None) -> int:
    """LDS read loop; returns the bytes it reads."""
    b = C.c_int64()
    if _lib.moe_probe_lds(iters, grid, _ptr(sink), C.byref(b), _stream(stream)) != MOE_OK:
        raise ValueError("moe_probe_lds: bad arguments")
    return int(b.value)


def moe_probe_mfma(iters: int, grid: int, sink, shape: int = 0, stream=None) -> int:
    """bf16 matrix-core loop (shape 0: 16x16x32, 1: 32x32x16); returns the
    floating-point operations it performs."""
    fl = C.c_int64()
    if _lib.moe_probe_mfma(iters, grid, shape, _ptr(sink), C.byref(fl), _stream(stream)) != MOE_OK:
        raise ValueError("moe_probe_mfma: bad arguments")
    return int(fl.value)
