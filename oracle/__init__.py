"""CPU oracle for routed mixture-of-experts FFN execution (ctypes wrapper).

TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check and the benchmark's
CPU-baseline leg may import this package.  It imports nothing from the
product package and the product never imports it.

The arithmetic lives in oracle.c (plain C, double precision); this module only
marshals numpy arrays.  The slot-cache model is in oracle/lru.py.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

Q8_0, Q4_0 = 0, 1
PREC_F32, PREC_BF16 = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")


def build() -> str:
    """Compile oracle.c with gcc into oracle/liboracle.so (IEEE double, no contraction)."""
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", os.path.join(_HERE, "oracle.c"), "-o", _SO + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_SO + ".tmp", _SO)
    return _SO


def _load() -> C.CDLL:
    if not os.path.exists(_SO):
        build()
    lib = C.CDLL(_SO)
    if not hasattr(lib, "orc_bf16_round_array"):  # built from an older oracle.c
        build()
        lib = C.CDLL(_SO)
    P = C.c_void_p
    sig = {
        "orc_set_threads": (C.c_int, [C.c_int]),
        "orc_f16_to_f64": (C.c_double, [C.c_uint16]),
        "orc_bf16_round": (C.c_double, [C.c_double]),
        "orc_block_bytes": (C.c_size_t, [C.c_int]),
        "orc_dequant": (None, [C.c_int, C.c_int, P, C.c_int64, P]),
        "orc_router_logits": (None, [P, P, C.c_int64, C.c_int, C.c_int, P]),
        "orc_topk": (C.c_int, [P, C.c_int64, C.c_int, C.c_int, C.c_int, P, P]),
        "orc_plan_union": (C.c_int, [P, C.c_int64, C.c_int, C.c_int, P, P, P, P]),
        "orc_expert_ffn": (None, [C.c_int, C.c_int, P, C.c_int, C.c_int, P, P]),
        "orc_expert_hidden": (None, [C.c_int, C.c_int, P, C.c_int, C.c_int, P, P]),
        "orc_expert_down": (None, [C.c_int, C.c_int, P, C.c_int, C.c_int, P, P]),
        "orc_bf16_round_array": (None, [P, C.c_int64, P]),
        "orc_moe_layer": (C.c_int, [C.c_int, C.c_int, P, C.c_int, P, C.c_int, C.c_int,
                                    C.c_int64, C.c_int, P, P, P, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def _p(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


def set_threads(n: int) -> int:
    return _lib.orc_set_threads(int(n))


def block_bytes(qtype: int) -> int:
    return int(_lib.orc_block_bytes(qtype))


def f16_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).reshape(-1)
    return np.array([_lib.orc_f16_to_f64(int(v)) for v in b], dtype=np.float64)


def bf16_round(v) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(v, dtype=np.float64).reshape(-1))
    out = np.empty_like(a)
    _lib.orc_bf16_round_array(_p(a), a.size, _p(out))
    return out


def x_to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Activations as exact doubles: float32 values, or bf16 bit patterns (uint16)."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32).astype(np.float64)
    bits = np.ascontiguousarray(x, dtype=np.uint16).astype(np.uint32) << 16
    return bits.view(np.float32).astype(np.float64)


def dequant(qtype: int, prec: int, blocks: np.ndarray, n_elems: int) -> np.ndarray:
    blocks = np.ascontiguousarray(blocks, dtype=np.uint8)
    assert n_elems % 32 == 0 and blocks.size >= n_elems // 32 * block_bytes(qtype)
    out = np.empty(n_elems, dtype=np.float64)
    _lib.orc_dequant(qtype, prec, _p(blocks), n_elems, _p(out))
    return out


def router_logits(x64: np.ndarray, w_r: np.ndarray) -> np.ndarray:
    x64 = np.ascontiguousarray(x64, dtype=np.float64)
    w_r = np.ascontiguousarray(w_r, dtype=np.float32)
    T, d = x64.shape
    E = w_r.shape[0]
    out = np.empty((T, E), dtype=np.float32)
    _lib.orc_router_logits(_p(x64), _p(w_r), T, E, d, _p(out))
    return out


def topk(logits: np.ndarray, k: int, norm: bool = True):
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    if _lib.orc_topk(_p(logits), T, E, k, int(norm), _p(ids), _p(w)) != 0:
        raise ValueError("topk: k outside [1, E] or non-finite logit")
    return ids, w


def plan_union(ids: np.ndarray, E: int):
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, k = ids.shape
    n_active = np.zeros(1, dtype=np.int32)
    experts = np.full(E, -1, dtype=np.int32)
    offsets = np.full(E + 1, -1, dtype=np.int32)
    entries = np.full(max(T * k, 1), -1, dtype=np.int32)
    if _lib.orc_plan_union(_p(ids), T, k, E, _p(n_active), _p(experts), _p(offsets), _p(entries)) != 0:
        raise ValueError("plan_union: expert id out of range")
    n = int(n_active[0])
    return n, experts[:n].copy(), offsets[:n + 1].copy(), entries[:T * k].copy()


def expert_ffn(qtype: int, prec: int, rec: np.ndarray, d: int, f: int, x64: np.ndarray) -> np.ndarray:
    rec = np.ascontiguousarray(rec, dtype=np.uint8)
    x64 = np.ascontiguousarray(x64, dtype=np.float64).reshape(d)
    y = np.empty(d, dtype=np.float64)
    _lib.orc_expert_ffn(qtype, prec, _p(rec), d, f, _p(x64), _p(y))
    return y


def expert_hidden(qtype: int, prec: int, rec: np.ndarray, d: int, f: int, x64: np.ndarray) -> np.ndarray:
    """h = silu(W_g x) * (W_u x) before any rounding of h (f values)."""
    rec = np.ascontiguousarray(rec, dtype=np.uint8)
    x64 = np.ascontiguousarray(x64, dtype=np.float64).reshape(d)
    h = np.empty(f, dtype=np.float64)
    _lib.orc_expert_hidden(qtype, prec, _p(rec), d, f, _p(x64), _p(h))
    return h


def expert_down(qtype: int, prec: int, rec: np.ndarray, d: int, f: int, h: np.ndarray) -> np.ndarray:
    """y = W_d h for a given hidden state h (f values)."""
    rec = np.ascontiguousarray(rec, dtype=np.uint8)
    h = np.ascontiguousarray(h, dtype=np.float64).reshape(f)
    y = np.empty(d, dtype=np.float64)
    _lib.orc_expert_down(qtype, prec, _p(rec), d, f, _p(h), _p(y))
    return y


def moe_layer(qtype: int, prec: int, records, shared, d: int, f: int,
              x64: np.ndarray, ids: np.ndarray, w: np.ndarray) -> np.ndarray:
    """records: sequence of length E (uint8 arrays or None); shared: uint8 array or None."""
    E = len(records)
    recs = [None if r is None else np.ascontiguousarray(r, dtype=np.uint8) for r in records]
    ptrs = (C.c_void_p * E)(*[None if r is None else r.ctypes.data for r in recs])
    sh = None if shared is None else np.ascontiguousarray(shared, dtype=np.uint8)
    x64 = np.ascontiguousarray(x64, dtype=np.float64)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    T, k = ids.shape
    y = np.empty((T, d), dtype=np.float32)
    rc = _lib.orc_moe_layer(qtype, prec, ptrs, E, None if sh is None else _p(sh), d, f, T, k,
                            _p(x64), _p(ids), _p(w), _p(y))
    if rc != 0:
        raise ValueError("moe_layer: invalid or missing expert id")
    return y
