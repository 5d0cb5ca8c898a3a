"""Seeded synthetic inputs for the routed-expert FFN path.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark.  It only draws random inputs (quant codes, fp16 scales, activations,
router weights, route logits) and lays them out in the GGUF block format that
the pages name as the expert storage format ("Nanite for Experts" §1 and
"MawForge" §V-B name GGUF Q8_0 models; block layout: 32 codes + one fp16
scale).  It holds none of the method's arithmetic: no dequantisation, no
routing, no matrix products.

Workloads (sizes of the pages' Qwen3.6-35B-A3B-style layer: 256 routed experts,
top-8 plus one shared expert, 40 routed layers — "Nanite for Experts" §1,
"Paging the Experts" §3.1):

  tiny      E=8   k=2 no shared d=256  f=128 Q8_0 T=4   fp32 activations
  decode    E=256 k=8 + shared  d=2048 f=512 Q8_0 T=1   bf16 activations, 38 slots
  mtp       E=256 k=8 + shared  d=2048 f=512 Q4_0 T=4   bf16, overlapping routes, 89 slots
  prefill   E=256 k=8 + shared  d=2048 f=512 Q8_0 T=512 bf16, Zipf(1.1) routes, 256 slots
  stack40   40 layers of the decode shape, Markov routes (p_repeat 0.6), 1536 slots

Every stream is keyed by (workload seed, layer, expert or token, purpose), so
any single expert can be regenerated without drawing the others.
"""
from __future__ import annotations

import numpy as np

Q8_0 = 0
Q4_0 = 1
QK = 32  # elements per quant block
BLOCK_BYTES = {Q8_0: 2 + QK, Q4_0: 2 + QK // 2}

# purpose tags for independent random streams
_P_EXPERT, _P_SHARED, _P_ROUTER, _P_X, _P_ROUTE = 0, 1, 2, 3, 4

WORKLOADS = {
    "tiny": dict(seed=1, n_layers=1, E=8, k=2, shared=False, d=256, f=128,
                 qtype=Q8_0, T=4, x_dtype="f32", n_slots=8, prec="f32"),
    "decode": dict(seed=2, n_layers=1, E=256, k=8, shared=True, d=2048, f=512,
                   qtype=Q8_0, T=1, x_dtype="bf16", n_slots=38, steps=1000,
                   prec="f32"),
    "mtp": dict(seed=3, n_layers=1, E=256, k=8, shared=True, d=2048, f=512,
                qtype=Q4_0, T=4, x_dtype="bf16", n_slots=89, steps=1000,
                p_shared_route=0.5, prec="f32"),
    "prefill": dict(seed=4, n_layers=1, E=256, k=8, shared=True, d=2048, f=512,
                    qtype=Q8_0, T=512, x_dtype="bf16", n_slots=256,
                    zipf_s=1.1, prec="bf16"),
    "stack40": dict(seed=5, n_layers=40, E=256, k=8, shared=True, d=2048, f=512,
                    qtype=Q8_0, T=1, x_dtype="bf16", n_slots=1536, tokens=256,
                    p_repeat=0.6, prec="f32"),
}


def workload(name: str) -> dict:
    return dict(WORKLOADS[name])


def rng(*key: int) -> np.random.Generator:
    """Independent generator for a tuple of non-negative integer keys."""
    return np.random.default_rng(np.random.SeedSequence([int(k) for k in key]))


# ---------------------------------------------------------------------------
# quantised expert weights in GGUF block layout
# ---------------------------------------------------------------------------

def fp16_scales(g: np.random.Generator, n: int, lo=0.001, hi=0.01) -> np.ndarray:
    """fp16 scales, numpy's round-to-nearest-even of U(lo, hi)."""
    return g.uniform(lo, hi, size=n).astype(np.float16)


def q8_0_blocks(g: np.random.Generator, n_blocks: int) -> np.ndarray:
    """[n_blocks, 34] uint8: fp16 scale (little endian) then 32 int8 codes in [-127, 127]."""
    out = np.empty((n_blocks, BLOCK_BYTES[Q8_0]), dtype=np.uint8)
    out[:, 0:2] = fp16_scales(g, n_blocks).view(np.uint8).reshape(n_blocks, 2)
    codes = g.integers(-127, 128, size=(n_blocks, QK), dtype=np.int16).astype(np.int8)
    out[:, 2:] = codes.view(np.uint8)
    return out


def q4_0_blocks(g: np.random.Generator, n_blocks: int) -> np.ndarray:
    """[n_blocks, 18] uint8: fp16 scale then 16 bytes holding 32 uniform 4-bit codes."""
    out = np.empty((n_blocks, BLOCK_BYTES[Q4_0]), dtype=np.uint8)
    out[:, 0:2] = fp16_scales(g, n_blocks).view(np.uint8).reshape(n_blocks, 2)
    out[:, 2:] = g.integers(0, 256, size=(n_blocks, QK // 2), dtype=np.int16).astype(np.uint8)
    return out


def blocks(g: np.random.Generator, qtype: int, n_blocks: int) -> np.ndarray:
    return q8_0_blocks(g, n_blocks) if qtype == Q8_0 else q4_0_blocks(g, n_blocks)


def expert_record_bytes(qtype: int, d: int, f: int) -> int:
    """Bytes of one expert in GGUF blocks: gate [f x d], up [f x d], down [d x f]."""
    return 3 * f * d // QK * BLOCK_BYTES[qtype]


def expert_record(seed: int, layer: int, expert: int, qtype: int, d: int, f: int,
                  shared: bool = False) -> np.ndarray:
    """One expert as GGUF blocks, flat uint8: gate rows, then up rows, then down rows.

    gate and up have f rows of d inputs; down has d rows of f inputs; blocks
    run along each row's input dimension.
    """
    g = rng(seed, layer, expert, _P_SHARED if shared else _P_EXPERT)
    return blocks(g, qtype, 3 * f * d // QK).reshape(-1)


def expert_record_fixed(qtype: int, d: int, f: int, scale_bits: tuple, codes: tuple) -> np.ndarray:
    """Expert whose gate, up and down blocks all carry one scale and one code each.

    scale_bits: fp16 bit patterns (gate, up, down); codes: raw code per matrix
    (int8 for Q8_0, 0..15 for Q4_0).  Used for closed-form tests.
    """
    mats = []
    for rows, cols, sb, c in ((f, d, scale_bits[0], codes[0]), (f, d, scale_bits[1], codes[1]),
                              (d, f, scale_bits[2], codes[2])):
        nb = rows * cols // QK
        b = np.empty((nb, BLOCK_BYTES[qtype]), dtype=np.uint8)
        b[:, 0] = sb & 0xFF
        b[:, 1] = (sb >> 8) & 0xFF
        if qtype == Q8_0:
            b[:, 2:] = np.uint8(np.int8(c).view(np.uint8))
        else:
            b[:, 2:] = np.uint8((c & 0xF) | ((c & 0xF) << 4))
        mats.append(b.reshape(-1))
    return np.concatenate(mats)


# ---------------------------------------------------------------------------
# activations and router
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 with torch's conversion; returns uint16 bits."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def activations(seed: int, T: int, d: int, dtype: str, *key: int) -> np.ndarray:
    """x ~ N(0, 1): float32 array, or uint16 bf16 bits when dtype == 'bf16'."""
    x = rng(seed, _P_X, *key).standard_normal((T, d)).astype(np.float32)
    return x if dtype == "f32" else f32_to_bf16_bits(x)


def router_weights(seed: int, E: int, d: int, layer: int = 0) -> np.ndarray:
    """W_r [E, d] float32 ~ N(0, 0.02) (0.02 is the standard deviation)."""
    return rng(seed, layer, 0, _P_ROUTER).normal(0.0, 0.02, size=(E, d)).astype(np.float32)


# ---------------------------------------------------------------------------
# route models, realised as router logits [T, E] float32
# ---------------------------------------------------------------------------

def _realise(g: np.random.Generator, chosen: list, E: int) -> np.ndarray:
    """Logits whose top-k is exactly the chosen sets: chosen 3 + 2 U(0,1), others min(N(0,1), 2.5)."""
    T = len(chosen)
    lg = np.minimum(g.standard_normal((T, E)), 2.5)
    for t, s in enumerate(chosen):
        s = np.fromiter(s, dtype=np.int64)
        lg[t, s] = 3.0 + 2.0 * g.uniform(size=s.size)
    return lg.astype(np.float32)


def mtp_route_sets(g: np.random.Generator, T: int, E: int, k: int, p: float) -> list:
    """Overlapping top-k sets of a multi-token window.

    Token 0 takes k distinct uniform experts.  Each pick of a later token comes,
    with probability p, from the union of the window so far (experts not yet in
    this token), otherwise uniformly from experts not yet in this token.
    """
    union: list = []
    sets = []
    for t in range(T):
        cur: list = []
        for _ in range(k):
            pool_u = [e for e in union if e not in cur]
            if t > 0 and pool_u and g.uniform() < p:
                e = pool_u[g.integers(len(pool_u))]
            else:
                free = np.setdiff1d(np.arange(E), np.array(cur, dtype=np.int64))
                e = int(free[g.integers(free.size)])
            cur.append(int(e))
        for e in cur:
            if e not in union:
                union.append(e)
        sets.append(sorted(cur))
    return sets


def mtp_logits(seed: int, step: int, T: int, E: int, k: int, p: float) -> np.ndarray:
    g = rng(seed, _P_ROUTE, step)
    return _realise(g, mtp_route_sets(g, T, E, k, p), E)


def zipf_gumbel_logits(seed: int, T: int, E: int, s: float) -> np.ndarray:
    """log Zipf_s(rank(e)) + Gumbel(0, 1): top-k of these is k draws without
    replacement proportional to Zipf weights (Gumbel-top-k)."""
    g = rng(seed, _P_ROUTE, 0)
    rank = g.permutation(E) + 1
    base = -s * np.log(rank.astype(np.float64))
    return (base[None, :] + g.gumbel(size=(T, E))).astype(np.float32)


def markov_route_sets(g: np.random.Generator, n_tokens: int, E: int, k: int, p_repeat: float) -> list:
    """Per-layer route chain: each expert of the previous token's set is kept with
    probability p_repeat; the rest are drawn uniformly from non-members."""
    sets = []
    prev: list = []
    for _ in range(n_tokens):
        cur = [e for e in prev if g.uniform() < p_repeat]
        while len(cur) < k:
            free = np.setdiff1d(np.arange(E), np.array(cur, dtype=np.int64))
            cur.append(int(free[g.integers(free.size)]))
        cur = sorted(cur)
        sets.append(cur)
        prev = cur
    return sets


def markov_logits(seed: int, layer: int, n_tokens: int, E: int, k: int, p_repeat: float) -> np.ndarray:
    """[n_tokens, E] logits of one layer's Markov route chain."""
    g = rng(seed, _P_ROUTE, layer)
    return _realise(g, markov_route_sets(g, n_tokens, E, k, p_repeat), E)


def follow_stack_logits(seed: int, n_layers: int, n_tokens: int, E: int, k: int, p_repeat: float,
                        p_follow: float) -> np.ndarray:
    """[n_layers, n_tokens, E] logits of Markov route chains that also follow
    the layer below: a token keeps each expert of its previous set at a layer
    with probability p_repeat (as markov_route_sets); each other pick is, with
    probability p_follow, the image under a fixed map of a random expert the
    same token selected one layer down (e -> (37 e + 11 l) mod E at layer l),
    else uniform.  Not a workload of the pages: routes whose new experts a
    layer-to-layer table can predict."""
    g = rng(seed, _P_ROUTE, 1000)
    sets = [[None] * n_tokens for _ in range(n_layers)]
    for t in range(n_tokens):
        for l in range(n_layers):
            prev = sets[l][t - 1] if t > 0 else []
            cur = [e for e in prev if g.uniform() < p_repeat]
            below = sets[l - 1][t] if l > 0 else []
            while len(cur) < k:
                e = -1
                if below and g.uniform() < p_follow:
                    e = (37 * below[g.integers(len(below))] + 11 * l) % E
                if e < 0 or e in cur:
                    free = np.setdiff1d(np.arange(E), np.array(cur, dtype=np.int64))
                    e = int(free[g.integers(free.size)])
                cur.append(int(e))
            sets[l][t] = sorted(cur)
    return np.stack([_realise(g, sets[l], E) for l in range(n_layers)])


def markov_trace(seed: int, n_layers: int, n_tokens: int, n_experts: int, k: int, p_repeat: float) -> list:
    """Replay trace: steps (layer, experts) for n_tokens tokens through n_layers
    layers, token-major, each layer's route a Markov chain over tokens (the
    stack workload's routes)."""
    chains = [markov_route_sets(rng(seed, 55, l), n_tokens, n_experts, k, p_repeat) for l in range(n_layers)]
    return [(l, sorted(int(e) for e in chains[l][t])) for t in range(n_tokens) for l in range(n_layers)]
