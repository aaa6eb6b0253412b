"""rq_decode_attention_encode: decode attention with the current tokens'
compression in the same launches must equal rq_decode_attention followed by
rq_encode_pack, bit for bit (outputs and every pool byte), in per-loop and
multi-loop mode and when no reference-loop call carries the encode."""
import numpy as np
import pytest

import workloads as W
from gpu_util import SmallCase, dev, to_dev, torch

pytestmark = pytest.mark.gpu

CASES = {
    "ouro_small": lambda: SmallCase(W.get(1).replace(batch=3, heads=3, context=203), shuffled=True,
                                    seq_lens=[203, 17, 160]),
    "huginn_small": lambda: SmallCase(W.get(3).replace(batch=2, heads=4, context=95), shuffled=True,
                                      seq_lens=[95, 33]),
    "tiny": lambda: SmallCase(W.get(0)),
    "d64_g16": lambda: SmallCase(W.get(0).replace(batch=3, heads=2, context=120, group_size=16, loops=3,
                                                  res_bits=(4, 2), sigma=(0.2, 0.1), meta_dtype="f16",
                                                  kv_dtype="bf16"), shuffled=True, seq_lens=[120, 64, 1]),
}
_cache = {}


def case(name):
    if name not in _cache:
        print(f"[case] building {name}", flush=True)
        _cache[name] = CASES[name]()
    return _cache[name]


def _current_tokens(c):
    """The current token of every sequence: all loops' K/V [L][2][B][H][D] and
    its slot (position seq_len of the sequence)."""
    T = torch()
    B, N = c.w.batch, c.w.context
    kv = np.ascontiguousarray(c.kv[:, :, :, N])                     # [L][2][B][H][D]
    slots = np.array([c.table[b, int(c.seq[b]) // 16] * 16 + int(c.seq[b]) % 16 for b in range(B)], np.int64)
    return to_dev(kv, c.w.kv_dtype), T.from_numpy(slots).to(dev())


def _run(c, pool, loops, fused, kv, slots, split_pages=0):
    import looped_transformer_decode_rq_amd as R
    T = torch()
    w = c.w
    q = to_dev(c.q[loops], w.kv_dtype)
    tk = to_dev(c.tail_k[loops], w.kv_dtype)
    tv = to_dev(c.tail_v[loops], w.kv_dtype)
    out = T.full((len(loops), w.batch, w.heads, w.head_dim), float("nan"), device=dev())
    ws = T.empty(R.decode_workspace_bytes(c.lay, len(loops), w.batch, c.table.shape[1], split_pages),
                 dtype=T.uint8, device=dev())
    ws.fill_(0xFF)
    if fused:
        R.decode_attention(c.lay, pool, loops, q, c.d_rot, c.d_table, c.d_seq, tk, tv, c.tau, out, ws,
                           split_pages=split_pages, kv_new=kv, slot_mapping=slots)
    else:
        R.decode_attention(c.lay, pool, loops, q, c.d_rot, c.d_table, c.d_seq, tk, tv, c.tau, out, ws,
                           split_pages=split_pages)
    return out


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("mode", ["per_loop", "multi_loop", "no_reference_call"])
def test_fused_encode_equals_decode_then_encode(name, mode):
    import looped_transformer_decode_rq_amd as R
    T = torch()
    c = case(name)
    kv, slots = _current_tokens(c)
    L = c.w.loops
    pool_a = c.device_pool_from_oracle()     # fused
    pool_b = c.device_pool_from_oracle()     # separate launches
    if mode == "per_loop":
        calls = [[l] for l in range(L)]
    elif mode == "multi_loop":
        calls = [list(range(L))[::-1]]
    else:
        calls = [[0]]
    outs_a, outs_b = [], []
    for loops in calls:
        carries = L - 1 in loops or mode == "no_reference_call"
        outs_a.append(_run(c, pool_a, loops, carries, kv, slots))
        outs_b.append(_run(c, pool_b, loops, False, kv, slots))
    R.encode_pack(c.lay, pool_b, kv, c.d_rot, slots)
    T.cuda.synchronize()
    for a, b in zip(outs_a, outs_b):
        np.testing.assert_array_equal(a.cpu().numpy(), b.cpu().numpy())
    ga, gb = pool_a.cpu().numpy(), pool_b.cpu().numpy()
    assert np.array_equal(ga, gb), f"{int((ga != gb).sum())} pool bytes differ"
    # the encode did write the current tokens (the pool changed)
    assert not np.array_equal(ga, c.pool_o)
