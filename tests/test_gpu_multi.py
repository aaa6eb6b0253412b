"""GPU parity of the multi-loop decode mode (several loops' queries in one
call, each reference page read once for all of them) against the fp64 oracle,
and against the same loops decoded one call at a time.

As in test_gpu_parity, the HIP kernels run on the oracle's packed bytes."""
import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_util import SmallCase, check_attention, dev, torch

pytestmark = pytest.mark.gpu

CASES = {
    "tiny": lambda: SmallCase(W.get(0)),
    "ouro_small": lambda: SmallCase(W.get(1).replace(batch=3, heads=3, context=203), shuffled=True,
                                    seq_lens=[203, 17, 160]),
    "huginn_small": lambda: SmallCase(W.get(3).replace(batch=2, heads=4, context=95), shuffled=True,
                                      seq_lens=[95, 33]),
    "g32_f32meta": lambda: SmallCase(W.get(1).replace(batch=2, heads=2, context=70, group_size=32,
                                                      meta_dtype="f32", res_bits=(4, 2, 2)), seq_lens=[70, 49]),
    # D64 with groups of 16, INT4 and INT2 residual loops
    "d64_g16": lambda: SmallCase(W.get(0).replace(batch=3, heads=2, context=120, group_size=16, loops=3,
                                                  res_bits=(4, 2), sigma=(0.2, 0.1), meta_dtype="f16",
                                                  kv_dtype="bf16"),
                                 shuffled=True, seq_lens=[120, 64, 1]),
}

_cache = {}


def case(name):
    if name not in _cache:
        print(f"[case] building {name}", flush=True)
        _cache[name] = CASES[name]()
    return _cache[name]


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("split_pages", [0, 1, 3])
def test_multi_loop_matches_oracle(name, split_pages):
    c = case(name)
    pool = c.device_pool_from_oracle()
    loops = list(range(c.w.loops))[::-1]
    got = c.run_decode(pool, loops, tail=True, split_pages=split_pages)
    for i, l in enumerate(loops):
        e, r = check_attention(f"{name} multi loop {l} sp {split_pages}", got[i], c.oracle_out(l, tail=True))
        print(f"[multi {name} loop {l} sp {split_pages}] max-abs {e:.2e} rel-L2 {r:.2e}", flush=True)


@pytest.mark.parametrize("name", ["ouro_small", "huginn_small", "d64_g16"])
def test_multi_loop_equals_single_calls(name):
    """Decoding loops together changes only the order in which split partials
    are merged."""
    c = case(name)
    pool = c.device_pool_from_oracle()
    loops = list(range(c.w.loops))
    multi = c.run_decode(pool, loops, split_pages=2)
    for i, l in enumerate(loops):
        single = c.run_decode(pool, [l], split_pages=2)[0]
        np.testing.assert_allclose(multi[i], single, rtol=0, atol=5e-5)


def test_multi_loop_subsets_duplicates_and_groups():
    """Any list of loops: residual loops only, repeats, and more calls than one
    workgroup holds (several groups, each reading the reference once)."""
    c = case("huginn_small")
    pool = c.device_pool_from_oracle()
    L = c.w.loops
    for loops in ([0, 2], [1, 1, L - 1, 0], list(range(L)) + [0, L - 1, 3], [L - 1, L - 1]):
        got = c.run_decode(pool, loops, tail=True)
        for i, l in enumerate(loops):
            check_attention(f"subset {loops} loop {l}", got[i], c.oracle_out(l, tail=True))
        # a repeated loop (same query) gives the same bits
        for i, l in enumerate(loops):
            j = loops.index(l)
            np.testing.assert_array_equal(got[i], got[j])


def test_multi_loop_edge_sequences():
    w = W.get(1).replace(batch=4, heads=2, context=40)
    c = SmallCase(w, seq_lens=[0, 0, 1, 40])
    pool = c.device_pool_from_oracle()
    loops = list(range(w.loops))
    got_nt = c.run_decode(pool, loops, tail=False)
    got = c.run_decode(pool, loops, tail=True)
    for i, l in enumerate(loops):
        assert not got_nt[i, 0].any() and not got_nt[i, 1].any()
        K, V = O.reconstruct_sequence(c.pool_o, c.olay, c.table[2], 1, 1, l, c.st["rot32"][1])
        np.testing.assert_allclose(got_nt[i, 2, 1], V[0], rtol=0, atol=2e-5)
        check_attention(f"multi edge nt loop {l}", got_nt[i], c.oracle_out(l, tail=False))
        np.testing.assert_allclose(got[i, 0], c.tail_v[l, 0], rtol=0, atol=1e-6)
        check_attention(f"multi edge tail loop {l}", got[i], c.oracle_out(l, tail=True))


def test_multi_loop_identical_loop_equals_reference_bitwise():
    import looped_transformer_decode_rq_amd as R
    from gpu_util import to_dev
    w = W.get(1).replace(batch=2, heads=2, context=50)
    c = SmallCase(w)
    kv = c.kv_tok.copy()
    kv[1] = kv[-1]
    T = torch()
    pool = T.zeros(c.olay.pool_bytes, dtype=T.uint8, device=dev())
    R.encode_pack(c.lay, pool, to_dev(kv, w.kv_dtype), c.d_rot, c.d_slots)
    ref = w.loops - 1
    c.q[1] = c.q[ref]
    c.tail_k[1], c.tail_v[1] = c.tail_k[ref], c.tail_v[ref]
    out = c.run_decode(pool, [0, 1, 2, ref])
    np.testing.assert_array_equal(out[1], out[3])


def test_multi_loop_shuffled_table_is_bitwise_invariant():
    w = W.get(1).replace(batch=2, heads=2, context=90)
    a = SmallCase(w, shuffled=False)
    b = SmallCase(w, shuffled=True)
    loops = list(range(w.loops))
    np.testing.assert_array_equal(a.run_decode(a.device_pool_from_oracle(), loops),
                                  b.run_decode(b.device_pool_from_oracle(), loops))
