"""GPU parity of the chunk (T > 4) path: bucket tile products on the matrix
cores: 64-token tiles for buckets of at least gemm_min tokens (bf16 mode), 16-token
tiles for the rest and for fp32 mode, against the CPU oracle.

Bars: fp32 mode, 1e-3 maximum relative error per token row.  bf16 mode, split
at the hidden state (tests/bf16_check.py): hidden codes bit-exact except at a
rounding midpoint, and y within 1e-3 per row of the oracle's down projection
and combine of the GPU's own hidden codes; end-to-end statistics reported.
Bitwise-identical outputs under any slot assignment.
"""
import os

import numpy as np
import pytest

import oracle
import synth
from tests import bf16_check
from tests import harness as H

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not H.gpu_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

from routed_expert_execution_amd import moe  # noqa: E402

FFN_TOL = 1e-3


def _say(*a):
    print(*a, flush=True)


class Chunk:
    def __init__(self, wl, T, logits, prec, gemm_min=16, perm_seed=None, x_dtype=None, wide_min=None):
        self.wl, self.T, self.prec = wl, T, prec
        E, k, d, f = wl["E"], wl["k"], wl["d"], wl["f"]
        self.x_dtype = x_dtype or wl["x_dtype"]
        self.x = synth.activations(wl["seed"], T, d, self.x_dtype, 777)
        self.ids, self.w = oracle.topk(logits, k)
        self.used = sorted(set(self.ids.reshape(-1).tolist()))
        self.recs = {e: synth.expert_record(wl["seed"], 0, e, wl["qtype"], d, f) for e in self.used}
        self.shared = synth.expert_record(wl["seed"], 0, 0, wl["qtype"], d, f, shared=True) if wl["shared"] else None
        n = len(self.used)
        from routed_expert_execution_amd import moe as m
        cfg = m.make_config(1, E, k, d, f, H.QT[wl["qtype"]], n, T, device=-1)
        pb = m.moe_payload_bytes(cfg)
        self.pool = torch.zeros(n * pb, dtype=torch.uint8, device="cuda")
        # wide_min: the bucket size from which bf16 calls use 128-token tiles
        # (a context reads it when it is created)
        old_env = os.environ.get("MOE_WIDE_MIN_TOKENS")
        if wide_min is not None:
            os.environ["MOE_WIDE_MIN_TOKENS"] = str(wide_min)
        try:
            self.ctx = m.Context(1, E, k, d, f, H.QT[wl["qtype"]], n, T, gemm_min_tokens=gemm_min, device=0,
                                 slot_pool=self.pool)
        finally:
            if wide_min is not None:
                if old_env is None:
                    del os.environ["MOE_WIDE_MIN_TOKENS"]
                else:
                    os.environ["MOE_WIDE_MIN_TOKENS"] = old_env
        self.payloads = {e: torch.from_numpy(H.payload(self.ctx, r)).cuda() for e, r in self.recs.items()}
        self.sh_dev = H.device_payload(self.ctx, self.shared) if self.shared is not None else None
        self.x_dev = H.torch_x(self.x, self.x_dtype)
        self.w_dev = torch.from_numpy(self.w).cuda()
        self.plan = moe.Plan(self.ctx, T)
        moe.moe_plan_union(self.ctx, torch.from_numpy(self.ids).cuda(), self.plan)

    def place(self, perm):
        for i, e in enumerate(self.used):
            self.ctx.slot(int(perm[i])).copy_(self.payloads[e])
            moe.moe_slot_bind(self.ctx, 0, e, int(perm[i]))

    def run(self):
        y = torch.full((self.T, self.wl["d"]), float("nan"), dtype=torch.float32, device="cuda")
        moe.moe_expert_ffn(self.ctx, 0, self.x_dev, self.plan, self.w_dev, y, shared_payload=self.sh_dev,
                           prec=self.prec)
        torch.cuda.synchronize()
        assert moe.moe_check(self.ctx) == moe.MOE_OK
        # the hidden rows this call left (bf16 codes in bf16 mode), for verify()
        self.h = moe.moe_hidden_rows(self.ctx, self.T * self.wl["k"] + self.T)
        return y.cpu().numpy()

    def verify(self, y, tokens):
        """The bar for these tokens (see the module docstring); returns the statistics."""
        tokens = np.asarray(tokens)
        if self.prec == oracle.PREC_BF16:
            st = bf16_check.check_chunk(self, y, tokens, self.h, FFN_TOL)
        else:
            st = H.elementwise_stats(y[tokens], self.reference(tokens))
            assert st["max_rel_row"] <= FFN_TOL, st
        assert np.isfinite(y[tokens]).all()
        return st

    def reference(self, tokens):
        wl = self.wl
        records = [self.recs.get(e) for e in range(wl["E"])]
        x64 = oracle.x_to_f64(self.x, self.x_dtype)[tokens]
        return oracle.moe_layer(wl["qtype"], self.prec, records, self.shared, wl["d"], wl["f"], x64,
                                self.ids[tokens], self.w[tokens])

    def bucket_sizes(self):
        return np.bincount(self.ids.reshape(-1), minlength=self.wl["E"])


@pytest.mark.parametrize("T,prec,gemm_min,wide_min", [
    (37, oracle.PREC_BF16, 16, None), (37, oracle.PREC_F32, 16, None), (100, oracle.PREC_BF16, 16, None),
    (100, oracle.PREC_BF16, 1000, None), (5, oracle.PREC_BF16, 2, None), (200, oracle.PREC_F32, 16, None),
    (100, oracle.PREC_BF16, 16, 8), (300, oracle.PREC_BF16, 16, 60), (37, oracle.PREC_BF16, 2, 1)])
def test_prefill_tiny_shape(T, prec, gemm_min, wide_min):
    """Tiny layer (8 experts, top-2, d 256, d_ff 128): buckets of ~9-50 tokens cover
    every tile size (16, 64 and, with wide_min lowered, 128 tokens), ragged tiles
    and fp32 mode."""
    wl = dict(synth.workload("tiny"), shared=True)
    lg = synth.zipf_gumbel_logits(wl["seed"] + T, T, wl["E"], 1.1)
    _say("prefill tiny", T, prec, gemm_min, wide_min)
    c = Chunk(wl, T, lg, prec, gemm_min, wide_min=wide_min)
    c.place(list(range(len(c.used))))
    y = c.run()
    st = c.verify(y, np.arange(T))
    _say("  buckets", sorted(c.bucket_sizes()[c.used].tolist()), st)


@pytest.mark.parametrize("T,wide_min", [(24, 40), (48, 40)])
def test_prefill_bucket_larger_than_chunk(T, wide_min):
    """Both ranks of every token name the same expert (a plan the C ABI accepts),
    so its bucket holds 2 T entries, at least wide_min.  A call of fewer than
    wide_min tokens launches no 128-token tiles, and its schedule must not
    make any (the bucket goes to 64-token tiles); a call of at least wide_min
    tokens takes them.  Both match the oracle on every row."""
    wl = dict(synth.workload("tiny"), shared=True)
    lg = synth.zipf_gumbel_logits(wl["seed"] + T, T, wl["E"], 1.1)
    _say("prefill duplicate ranks", T, wide_min)
    c = Chunk(wl, T, lg, oracle.PREC_BF16, 16, wide_min=wide_min)
    c.place(list(range(len(c.used))))
    e = c.used[0]
    c.ids = np.full((T, wl["k"]), e, dtype=np.int32)
    c.w = np.full((T, wl["k"]), 1.0 / wl["k"], dtype=np.float32)
    c.w_dev = torch.from_numpy(c.w).cuda()
    c.plan = moe.Plan(c.ctx, T)
    moe.moe_plan_union(c.ctx, torch.from_numpy(c.ids).cuda(), c.plan)
    y = c.run()
    st = c.verify(y, np.arange(T))
    _say("  ", st)


@pytest.mark.parametrize("T,prec,wide_min", [(24, oracle.PREC_BF16, None), (24, oracle.PREC_F32, None),
                                             (24, oracle.PREC_BF16, 2)])
def test_prefill_mtp_q4(T, prec, wide_min):
    """Q4_0 experts through the chunk path (with wide_min 2: on 128-token tiles)."""
    wl = synth.workload("mtp")
    lg = synth.zipf_gumbel_logits(wl["seed"], T, wl["E"], 1.1)
    _say("prefill q4", T, prec, wide_min)
    c = Chunk(wl, T, lg, prec, gemm_min=4, wide_min=wide_min)
    c.place(list(range(len(c.used))))
    y = c.run()
    _say("  ", c.verify(y, np.arange(T)))


def test_prefill_workload_all_rows():
    """The prefill workload at full size: 512 tokens, Zipf(1.1) routes over 256
    experts, Q8_0, bf16 mode; every row against the oracle (the busiest
    expert's bucket spans several 64-token tiles, most buckets are under 16)."""
    wl = synth.workload("prefill")
    lg = synth.zipf_gumbel_logits(wl["seed"], wl["T"], wl["E"], wl["zipf_s"])
    c = Chunk(wl, wl["T"], lg, oracle.PREC_BF16)
    sizes = c.bucket_sizes()
    _say("prefill full: experts used", len(c.used), "largest buckets", sorted(sizes)[-3:],
         ">=16:", int((sizes >= 16).sum()))
    c.place(list(range(len(c.used))))
    y = c.run()
    assert np.isfinite(y).all()
    st = c.verify(y, np.arange(wl["T"]))
    _say("  all 512 rows:", st)


def _tile_edge_tokens(c, gemm_min=16, big=64, small=16):
    """Tokens at the first and last row of the first and last tile of every
    bucket (tiles of 64 positions for buckets of at least gemm_min, else 16),
    and of the shared expert's tiles over all tokens, by plan position."""
    n, experts, offsets, entries = oracle.plan_union(c.ids, c.wl["E"])
    k = c.wl["k"]
    pos = set()
    for u in range(n):
        p0, p1 = int(offsets[u]), int(offsets[u + 1])
        M = p1 - p0
        B = big if M >= gemm_min else small
        last = p0 + (M - 1) // B * B
        pos.update({p0, min(p0 + B, p1) - 1, last, p1 - 1})
    toks = {int(entries[p]) // k for p in pos}
    T = c.T
    toks.update({0, min(big, T) - 1, (T - 1) // big * big, T - 1})
    return np.array(sorted(toks))

@pytest.mark.parametrize("wide_min", [None, 8])
def test_prefill_cache_transparency(wide_min):
    wl = dict(synth.workload("tiny"), shared=True)
    T = 150
    lg = synth.zipf_gumbel_logits(wl["seed"] + 5, T, wl["E"], 1.1)
    c = Chunk(wl, T, lg, oracle.PREC_BF16, wide_min=wide_min)
    n = len(c.used)
    c.place(list(range(n)))
    y0 = c.run()
    c.place(list(range(n))[::-1])
    y1 = c.run()
    c.place(list(np.random.default_rng(2).permutation(n)))
    y2 = c.run()
    assert np.array_equal(y0.view(np.uint32), y1.view(np.uint32))
    assert np.array_equal(y0.view(np.uint32), y2.view(np.uint32))


@pytest.mark.parametrize("wide_min", [None, 4])
def test_prefill_unmapped_expert_fails_closed(wide_min):
    wl = dict(synth.workload("tiny"), shared=True)
    T = 60
    lg = synth.zipf_gumbel_logits(wl["seed"] + 9, T, wl["E"], 1.1)
    c = Chunk(wl, T, lg, oracle.PREC_BF16, wide_min=wide_min)
    c.place(list(range(len(c.used))))
    victim = c.used[-1]
    moe.moe_slot_bind(c.ctx, 0, victim, -1)
    y = torch.empty((T, wl["d"]), dtype=torch.float32, device="cuda")
    moe.moe_expert_ffn(c.ctx, 0, c.x_dev, c.plan, c.w_dev, y, shared_payload=c.sh_dev, prec=oracle.PREC_BF16)
    assert moe.moe_check(c.ctx) == moe.MOE_EMISS
    y = y.cpu().numpy()
    hit = (c.ids == victim).any(axis=1)
    assert hit.any() and np.isnan(y[hit]).all(axis=1).all() and np.isfinite(y[~hit]).all()


def test_prefill_large_chunk_tile_edges():
    """A 4096-token chunk of the prefill layer (Zipf(1.1) routes, Q8_0, bf16
    mode): more tiles than one launch's workgroups, so every tile kernel loops;
    oracle on the tokens at the first and last row of the first and last tile
    of every bucket, by plan position, plus 32 drawn at random."""
    wl = dict(synth.workload("prefill"), T=4096)
    T = wl["T"]
    lg = synth.zipf_gumbel_logits(wl["seed"] + 21, T, wl["E"], wl["zipf_s"])
    c = Chunk(wl, T, lg, oracle.PREC_BF16)
    sizes = c.bucket_sizes()
    _say("prefill 4096: experts used", len(c.used), "largest buckets", sorted(sizes)[-3:])
    c.place(list(range(len(c.used))))
    y = c.run()
    assert np.isfinite(y).all()
    g = np.random.default_rng(8)
    tokens = np.unique(np.concatenate([_tile_edge_tokens(c), g.choice(T, size=32, replace=False)]))
    st = c.verify(y, tokens)
    _say("  tokens checked", tokens.size, st)


def test_prefill_max_tokens_tile_edges():
    """The largest chunk a context takes (max_tokens 65536) on the prefill layer:
    buckets of tens of thousands of tokens, about 590K hidden rows; oracle on
    the tokens at the first and last row of the first and last tile of every
    bucket, by plan position, plus 16 drawn at random."""
    wl = dict(synth.workload("prefill"), T=65536)
    T = wl["T"]
    lg = synth.zipf_gumbel_logits(wl["seed"] + 31, T, wl["E"], wl["zipf_s"])
    c = Chunk(wl, T, lg, oracle.PREC_BF16)
    _say("prefill 65536: largest buckets", sorted(c.bucket_sizes())[-2:])
    c.place(list(range(len(c.used))))
    y = c.run()
    assert np.isfinite(y).all()
    g = np.random.default_rng(9)
    tokens = np.unique(np.concatenate([_tile_edge_tokens(c), g.choice(T, size=16, replace=False)]))
    st = c.verify(y, tokens)
    _say("  tokens checked", tokens.size, st)
