"""GPU parity of decode attention when the query has one large channel.

The split kernels score tokens with exact integer dot products of the packed
codes against a fixed-point copy of the query (one power-of-two scale per lane
slice of channels). A channel ×100 or ×1000 larger than the others sets its
slice's scale; these cases check that the other channels keep enough precision
for the attention tolerance, per-loop and multi-loop, at head dims 64, 96 and
128, with an all-zero query row (scores all zero: the mean of the values).
Attention over the packed cache must equal attention over the restored states
(ResidualQuant, rit.work summary, section on how each pass's KV cache is
restored), whatever the query.
"""
import numpy as np
import pytest

import workloads as W
from gpu_util import SmallCase, check_attention

pytestmark = pytest.mark.gpu

CASES = {
    "d128": lambda: SmallCase(W.get(1).replace(batch=3, heads=2, context=203), shuffled=True,
                              seq_lens=[203, 150, 97]),
    "d96": lambda: SmallCase(W.get(3).replace(batch=3, heads=3, context=95), shuffled=True,
                             seq_lens=[95, 80, 33]),
    "d64": lambda: SmallCase(W.get(1).replace(batch=3, heads=2, context=150, head_dim=64, group_size=64,
                                              res_bits=(4, 2, 2)), seq_lens=[150, 120, 64]),
    "d64_f32": lambda: SmallCase(W.get(0).replace(batch=3, heads=2, context=120), seq_lens=[120, 77, 16]),
}
_cache = {}


def case(name):
    if name not in _cache:
        print(f"[case] building {name}", flush=True)
        _cache[name] = CASES[name]()
    return _cache[name]


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("mult", [100.0, 1000.0])
def test_outlier_query_channel(name, mult):
    c = case(name)
    q0 = c.q.copy()
    try:
        # sequence 1: all-zero query; the others: one channel x mult
        c.q = W.outlier_queries(c.w, q0, mult, zero_rows=(1,), seed=int(mult))
        pool = c.device_pool_from_oracle()
        L = c.w.loops
        multi = c.run_decode(pool, list(range(L)))
        worst = 0.0
        for l in range(L):
            want = c.oracle_out(l)
            for sp in (0, 1):
                got = c.run_decode(pool, [l], split_pages=sp)[0]
                e, r = check_attention(f"{name} x{mult:g} loop {l} sp {sp}", got, want)
                worst = max(worst, e)
            e, r = check_attention(f"{name} x{mult:g} multi-loop loop {l}", multi[l], want)
            worst = max(worst, e)
        print(f"[query range {name} x{mult:g}] worst max-abs {worst:.2e}", flush=True)
    finally:
        c.q = q0


@pytest.mark.parametrize("name", ["d128", "d96"])
def test_zero_query_gives_mean_of_values(name):
    """q = 0 (no current token): every score is 0, so the output is the mean
    of the reconstructed values of the cached tokens."""
    import oracle as O
    c = case(name)
    q0 = c.q.copy()
    try:
        c.q = np.zeros_like(q0)
        pool = c.device_pool_from_oracle()
        for l in (0, c.w.loops - 1):
            got = c.run_decode(pool, [l], tail=False)[0]
            for b in range(c.w.batch):
                for h in range(c.w.heads):
                    K, V = O.reconstruct_sequence(c.pool_o, c.olay, c.table[b], int(c.seq[b]), h, l,
                                                  c.st["rot32"][h])
                    check_attention(f"{name} q=0 loop {l} seq {b} head {h}", got[b, h], V.mean(axis=0))
    finally:
        c.q = q0
