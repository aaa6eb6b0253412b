"""The allocation-free decode entry point (rq_decode_attention_noalloc, for
callers that cannot allocate device memory) against rq_decode_attention_ex
with a caller workspace: the same kernels on the same inputs, so the outputs
must agree (they are compared bit for bit, and against the parity tolerance),
on two calls in a row of which the second is smaller, and in both per-loop and
multi-loop mode. A request beyond the fixed scratch is refused."""
import numpy as np
import pytest

import workloads as W
from gpu_util import SmallCase, check_attention, dev, to_dev, torch

pytestmark = pytest.mark.gpu


def _run_noalloc(c, pool, loops, split_pages=0):
    import looped_transformer_decode_rq_amd as R
    T = torch()
    w = c.w
    q = to_dev(c.q[loops], w.kv_dtype)
    tk = to_dev(c.tail_k[loops], w.kv_dtype)
    tv = to_dev(c.tail_v[loops], w.kv_dtype)
    out = T.full((len(loops), w.batch, w.heads, w.head_dim), float("nan"), device=dev())
    R.decode_attention_noalloc(c.lay, pool, loops, q, c.d_rot, c.d_table, c.d_seq, tk, tv, c.tau, out,
                               split_pages=split_pages)
    T.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def test_noalloc_matches_workspace_entry_point_twice():
    big = SmallCase(W.get(1).replace(batch=4, heads=3, context=300), shuffled=True, seq_lens=[300, 211, 17, 160])
    small = SmallCase(W.get(3).replace(batch=2, heads=2, context=90), seq_lens=[90, 41])
    for c in (big, small):                   # the second call is smaller (and another layout)
        pool = c.device_pool_from_oracle()
        L = c.w.loops
        for loops in ([0], [L - 1], list(range(L))):
            for sp in (0, 1):
                want = c.run_decode(pool, loops, split_pages=sp)
                got = _run_noalloc(c, pool, loops, split_pages=sp)
                np.testing.assert_array_equal(got, want)
                for i, l in enumerate(loops):
                    check_attention(f"noalloc loop {l} sp {sp}", got[i], c.oracle_out(l))


def test_noalloc_refuses_requests_beyond_its_scratch():
    import looped_transformer_decode_rq_amd as R
    T = torch()
    w = W.get(1).replace(batch=64, heads=16, context=32768)
    lay = R.make_layout(w.heads, w.head_dim, w.group_size, w.loops, w.res_bits, 8, w.meta_dtype, w.kv_dtype)
    mb = 2049
    need = R.decode_workspace_bytes(lay, 4, w.batch, mb, 8)
    assert need > R.RQ_NOALLOC_SCRATCH_BYTES
    pool = T.zeros(R.pool_bytes(lay), dtype=T.uint8, device=dev())
    q = T.zeros((4, w.batch, w.heads, w.head_dim), dtype=T.bfloat16, device=dev())
    out = T.full((4, w.batch, w.heads, w.head_dim), 7.0, device=dev())
    table = T.zeros((w.batch, mb), dtype=T.int32, device=dev())
    seq = T.zeros((w.batch,), dtype=T.int32, device=dev())
    rot = T.zeros((w.heads, 2, w.head_dim, w.head_dim), dtype=T.float32, device=dev())
    with pytest.raises(R.RqError) as e:
        R.decode_attention_noalloc(lay, pool, [0, 1, 2, 3], q, rot, table, seq, None, None, 0.1, out, split_pages=8)
    assert e.value.status == -6
    T.cuda.synchronize()
    assert bool((out == 7.0).all())          # refused before touching memory
