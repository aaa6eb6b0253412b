"""A multi-layer decode step captured in one HIP graph (torch.cuda.CUDAGraph
over the library's stream-ordered launches) replays to the eager results bit
for bit. Per layer: every loop's decode call in order, the current tokens'
compression riding in the reference-loop call, then one multi-loop call.
Every replay follows eager work of the program itself and a synchronization,
and every replay is checked: outputs and every pool byte."""
import numpy as np
import pytest

import workloads as W
from gpu_util import SmallCase, dev, to_dev, torch

pytestmark = pytest.mark.gpu


def test_graph_replay_equals_eager():
    import looped_transformer_decode_rq_amd as R
    T = torch()
    c = SmallCase(W.get(1).replace(batch=3, heads=3, context=203), shuffled=True, seq_lens=[203, 17, 160])
    w = c.w
    L, B, H, D, N = w.loops, w.batch, w.heads, w.head_dim, w.context
    layers = 2
    pools = [c.device_pool_from_oracle() for _ in range(layers)]
    q = to_dev(c.q, w.kv_dtype)
    tk, tv = to_dev(c.tail_k, w.kv_dtype), to_dev(c.tail_v, w.kv_dtype)
    # the current token of every sequence (all loops) and its slot, position seq_len
    kv_new = to_dev(np.ascontiguousarray(c.kv[:, :, :, N]), w.kv_dtype)          # [L][2][B][H][D]
    slots = np.array([c.table[b, int(c.seq[b]) // 16] * 16 + int(c.seq[b]) % 16 for b in range(B)], np.int64)
    slots_new = T.from_numpy(slots).to(dev())
    ws1 = T.empty(R.decode_workspace_bytes(c.lay, 1, B, c.table.shape[1]), dtype=T.uint8, device=dev())
    wsm = T.empty(R.decode_workspace_bytes(c.lay, L, B, c.table.shape[1]), dtype=T.uint8, device=dev())
    outs = T.empty((layers, L, B, H, D), device=dev())
    multi = T.empty((layers, L, B, H, D), device=dev())

    def step():
        for i in range(layers):
            for l in range(L):
                enc = dict(kv_new=kv_new, slot_mapping=slots_new) if l == L - 1 else {}
                R.decode_attention(c.lay, pools[i], [l], q[l:l + 1], c.d_rot, c.d_table, c.d_seq, tk[l:l + 1],
                                   tv[l:l + 1], c.tau, outs[i, l:l + 1], ws1, **enc)
            R.decode_attention(c.lay, pools[i], list(range(L)), q, c.d_rot, c.d_table, c.d_seq, tk, tv, c.tau,
                               multi[i], wsm)

    step()
    T.cuda.synchronize()
    want_o, want_m = outs.clone(), multi.clone()
    want_p = [p.clone() for p in pools]
    assert T.isfinite(want_o).all() and T.isfinite(want_m).all()

    side = T.cuda.Stream()
    side.wait_stream(T.cuda.current_stream())
    with T.cuda.stream(side):
        step()
    T.cuda.current_stream().wait_stream(side)
    T.cuda.synchronize()
    g = T.cuda.CUDAGraph()
    with T.cuda.graph(g):
        step()
    T.cuda.synchronize()

    scratch = T.empty((1, B, H, D), device=dev())
    for rep in range(3):
        outs.fill_(float("nan"))
        multi.fill_(float("nan"))
        # the program's own eager work between replays
        R.decode_attention(c.lay, pools[0], [0], q[0:1], c.d_rot, c.d_table, c.d_seq, tk[0:1], tv[0:1], c.tau,
                           scratch, ws1)
        T.cuda.synchronize()
        g.replay()
        T.cuda.synchronize()
        print(f"[graph] replay {rep}", flush=True)
        assert T.equal(outs, want_o), f"replay {rep}: per-loop outputs differ"
        assert T.equal(multi, want_m), f"replay {rep}: multi-loop outputs differ"
        for i in range(layers):
            assert T.equal(pools[i], want_p[i]), f"replay {rep}: pool of layer {i} differs"


def test_chunk_graph_replay_equals_eager():
    """Chunked prefill of every loop (a ragged 37-query chunk: partial query
    tiles) captured in one graph replays to the eager outputs bit for bit."""
    import looped_transformer_decode_rq_amd as R
    T = torch()
    c = SmallCase(W.get(1).replace(batch=2, heads=3, context=150), shuffled=True, seq_lens=[150, 33])
    w = c.w
    L, B, H, D, C = w.loops, w.batch, w.heads, w.head_dim, 37
    rng = np.random.default_rng(7)
    shp = (L, B, C, H, D)
    q = to_dev(W.bf16_round(rng.normal(size=shp) / np.sqrt(D)), "bf16")
    ck = to_dev(W.bf16_round(rng.normal(size=shp)), "bf16")
    cv = to_dev(W.bf16_round(rng.normal(size=shp)), "bf16")
    pool = c.device_pool_from_oracle()
    ws = T.empty(R.chunk_workspace_bytes(c.lay, C, B, c.table.shape[1]), dtype=T.uint8, device=dev())
    out = T.empty((L, B, C, H, D), device=dev())

    def step():
        for l in range(L):
            R.chunk_attention(c.lay, pool, l, q[l], c.d_rot, c.d_table, c.d_seq, ck[l], cv[l], c.tau, out[l], ws)

    step()
    T.cuda.synchronize()
    want = out.clone()
    assert T.isfinite(want).all()
    side = T.cuda.Stream()
    side.wait_stream(T.cuda.current_stream())
    with T.cuda.stream(side):
        step()
    T.cuda.current_stream().wait_stream(side)
    T.cuda.synchronize()
    g = T.cuda.CUDAGraph()
    with T.cuda.graph(g):
        step()
    T.cuda.synchronize()
    scratch = T.empty((B, C, H, D), device=dev())
    for rep in range(3):
        out.fill_(float("nan"))
        # the program's own eager work between replays
        R.chunk_attention(c.lay, pool, 0, q[1], c.d_rot, c.d_table, c.d_seq, ck[1], cv[1], c.tau, scratch, ws)
        T.cuda.synchronize()
        g.replay()
        T.cuda.synchronize()
        print(f"[chunk graph] replay {rep}", flush=True)
        assert T.equal(out, want), f"replay {rep}: chunk outputs differ"
