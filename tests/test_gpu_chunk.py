"""GPU parity of chunked prefill over the packed cache (rq_chunk_attention)
against the fp64 oracle's chunk_attention, on the oracle's packed bytes.

Cases: an Ouro-like layer (D128, G128, INT2 residuals) with a ragged context
and shuffled table, and a Huginn-like one (D96, G96, INT4 and INT2 residual
loops); chunks of 1..256 queries (256 is the largest chunk), with and without
the chunk's own K/V, split sizes chosen by the library, forced small and the
largest (1024 pages: one split); empty caches; C = 1 against decode attention;
queries with one channel x100 / x1000 and all-zero queries (the scores use a
fixed-point copy of each query, one power of two per row); the
supported-layout check.
"""
import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_util import SmallCase, check_attention, dev, to_dev, torch

pytestmark = pytest.mark.gpu

CASES = {
    "ouro_small": lambda: SmallCase(W.get(1).replace(batch=3, heads=3, context=203), shuffled=True,
                                    seq_lens=[203, 17, 160]),
    "huginn_small": lambda: SmallCase(W.get(3).replace(batch=2, heads=3, context=95), shuffled=True,
                                      seq_lens=[95, 0]),
    # layouts whose K code areas land in LDS transposed: D64 with INT4 and INT2
    # residuals, and D128 with INT4 residuals
    "d64_mixed": lambda: SmallCase(W.get(1).replace(batch=2, heads=2, context=70, head_dim=64, group_size=64,
                                                    res_bits=(4, 2, 2)), shuffled=True, seq_lens=[70, 33]),
    "d128_int4_res": lambda: SmallCase(W.get(1).replace(batch=2, heads=2, context=90, res_bits=(4, 4, 2)),
                                       shuffled=True, seq_lens=[90, 41]),
}
_cache = {}


def case(name):
    if name not in _cache:
        print(f"[chunk case] building {name}", flush=True)
        _cache[name] = CASES[name]()
    return _cache[name]


def chunk_inputs(c, C, seed):
    """Seeded queries and chunk K/V [B][C][H][D], rounded to bf16."""
    w = c.w
    rng = np.random.default_rng(seed)
    shp = (w.batch, C, w.heads, w.head_dim)
    q = W.bf16_round(rng.normal(size=shp) / np.sqrt(w.head_dim))
    ck = W.bf16_round(rng.normal(size=shp))
    cv = W.bf16_round(rng.normal(size=shp))
    return q, ck, cv


def run_chunk(c, pool, loop, q, ck, cv, split_pages=0):
    import looped_transformer_decode_rq_amd as R
    T = torch()
    w = c.w
    B, C = q.shape[:2]
    out = T.full((B, C, w.heads, w.head_dim), float("nan"), device=dev())
    ws = T.empty(R.chunk_workspace_bytes(c.lay, C, B, c.table.shape[1], split_pages), dtype=T.uint8, device=dev())
    ws.fill_(0xFF)     # stale workspace contents must never reach the output
    R.chunk_attention(c.lay, pool, loop, to_dev(q, "bf16"), c.d_rot, c.d_table, c.d_seq,
                      None if ck is None else to_dev(ck, "bf16"), None if cv is None else to_dev(cv, "bf16"),
                      c.tau, out, ws, split_pages=split_pages)
    T.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("C,split_pages", [(1, 0), (16, 0), (37, 3), (64, 1), (100, 0), (256, 1024)])
def test_chunk_matches_oracle(name, C, split_pages):
    c = case(name)
    pool = c.device_pool_from_oracle()
    q, ck, cv = chunk_inputs(c, C, seed=C)
    for l in range(c.w.loops):
        got = run_chunk(c, pool, l, q, ck, cv, split_pages)
        want = O.chunk_attention(c.pool_o, c.olay, l, q, c.st["rot32"], c.table, c.seq, c.tau, ck, cv)
        e, r = check_attention(f"chunk {name} C{C} sp{split_pages} loop {l}", got, want)
        print(f"[chunk {name} C={C} sp={split_pages} loop {l}] max-abs {e:.2e} rel-L2 {r:.2e}", flush=True)


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("mult", [100.0, 1000.0])
def test_chunk_outlier_query_channel(name, mult):
    """One seeded channel of every query scaled by mult (it sets the row's
    fixed-point scale); the first queries of sequence 0 all zero."""
    c = case(name)
    pool = c.device_pool_from_oracle()
    q, ck, cv = chunk_inputs(c, 24, seed=11)
    rng = np.random.default_rng([int(mult), 5])
    B, C, H, D = q.shape
    ch = rng.integers(0, D, size=(B, C, H))
    bi, ci, hi = np.meshgrid(np.arange(B), np.arange(C), np.arange(H), indexing="ij")
    q = q.copy()
    q[bi, ci, hi, ch] *= mult
    q = W.bf16_round(q)
    q[0, :5] = 0.0
    for l in range(c.w.loops):
        got = run_chunk(c, pool, l, q, ck, cv)
        want = O.chunk_attention(c.pool_o, c.olay, l, q, c.st["rot32"], c.table, c.seq, c.tau, ck, cv)
        e, r = check_attention(f"chunk {name} x{mult:g} loop {l}", got, want)
        print(f"[chunk {name} x{mult:g} loop {l}] max-abs {e:.2e} rel-L2 {r:.2e}", flush=True)


@pytest.mark.parametrize("name", list(CASES))
def test_chunk_without_chunk_kv(name):
    c = case(name)
    pool = c.device_pool_from_oracle()
    q, _, _ = chunk_inputs(c, 20, seed=7)
    for l in (0, c.w.loops - 1):
        got = run_chunk(c, pool, l, q, None, None)
        want = O.chunk_attention(c.pool_o, c.olay, l, q, c.st["rot32"], c.table, c.seq, c.tau)
        # a sequence with nothing cached and no chunk K/V attends nothing: zero rows
        empty = np.asarray(c.seq) == 0
        want[empty] = 0.0
        check_attention(f"chunk {name} no chunk K/V loop {l}", got, want)


def test_chunk_of_one_equals_decode():
    """C = 1 with the chunk token as the current token is decode attention."""
    c = case("ouro_small")
    pool = c.device_pool_from_oracle()
    for l in range(c.w.loops):
        q = c.q[l][:, None]
        got = run_chunk(c, pool, l, q, c.tail_k[l][:, None], c.tail_v[l][:, None])[:, 0]
        dec = c.run_decode(pool, [l], tail=True)[0]
        np.testing.assert_allclose(got, dec, rtol=0, atol=2e-5)


def test_chunk_split_count_changes_only_rounding():
    c = case("ouro_small")
    pool = c.device_pool_from_oracle()
    q, ck, cv = chunk_inputs(c, 40, seed=3)
    outs = [run_chunk(c, pool, 0, q, ck, cv, sp) for sp in (1, 4, 64)]
    for o in outs[1:]:
        np.testing.assert_allclose(o, outs[0], rtol=0, atol=2e-5)


def test_chunk_unsupported_layouts_are_refused():
    import looped_transformer_decode_rq_amd as R
    T = torch()
    for w in (W.get(0), W.get(1).replace(group_size=32)):       # fp32 K/V; groups smaller than the head
        lay = R.make_layout(w.heads, w.head_dim, w.group_size, w.loops, w.res_bits, 4, w.meta_dtype, w.kv_dtype)
        assert R.chunk_workspace_bytes(lay, 8, 1, 4) == 0
