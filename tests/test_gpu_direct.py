"""GPU parity of the direct per-loop baseline (layout mode RQ_MODE_DIRECT:
every loop quantized on its own, no reference, alpha or rotation) against the
fp64 oracle: the HIP encoder's records (exemption rule of gpu_util) and decode
attention of every loop on the oracle's packed bytes."""
import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_util import check_attention, check_caps, compare_quantized, dev, to_dev, torch

pytestmark = pytest.mark.gpu


class DirectCase:
    def __init__(self, w, bits, seq_lens=None, shuffled=True):
        import looped_transformer_decode_rq_amd as R
        T = torch()
        self.w, self.bits = w, tuple(bits)
        B, N, H, D, L = w.batch, w.context, w.heads, w.head_dim, w.loops
        self.kv = W.kv_numpy(w)                                   # [L][2][B][N+1][H][D]
        self.q = W.queries_numpy(w)
        self.table, self.nblk = W.block_table(w, spare_blocks=3, shuffled=shuffled)
        self.seq = np.full(B, N, np.int32) if seq_lens is None else np.asarray(seq_lens, np.int32)
        self.olay = O.PoolLayout(H, D, w.group_size, L, (), w.meta_dtype, self.nblk, direct_bits=self.bits)
        self.lay = R.make_layout(H, D, w.group_size, L, self.bits, self.nblk, w.meta_dtype, w.kv_dtype,
                                 mode=R.RQ_MODE_DIRECT)
        pos = [np.arange(int(self.seq[b])) for b in range(B)]
        tb = np.concatenate([np.full(len(p), b) for b, p in enumerate(pos)]).astype(np.int64)
        tp = np.concatenate(pos).astype(np.int64)
        self.slots = self.table[tb, tp // 16].astype(np.int64) * 16 + tp % 16
        self.kv_tok = self.kv[:, :, tb, tp]                           # [L][2][T][H][D]
        self.enc = O.encode_direct(self.kv_tok, self.bits, w.group_size, w.meta_dtype)
        self.pool_o = np.zeros(self.olay.pool_bytes, np.uint8)
        O.write_tokens(self.pool_o, self.olay, self.enc, self.slots)
        self.tail_k, self.tail_v = self.kv[:, 0, :, N], self.kv[:, 1, :, N]
        self.tau = 1.0 / np.sqrt(D)
        self.d_table = T.from_numpy(self.table).to(dev())
        self.d_seq = T.from_numpy(self.seq).to(dev())

    def oracle_out(self, l, tail=True):
        return O.decode_attention(self.pool_o, self.olay, l, self.q[l], None, self.table, self.seq, self.tau,
                                  self.tail_k[l] if tail else None, self.tail_v[l] if tail else None)

    def run(self, pool, loops, tail=True, split_pages=0):
        import looped_transformer_decode_rq_amd as R
        T = torch()
        w = self.w
        out = T.full((len(loops), w.batch, w.heads, w.head_dim), float("nan"), device=dev())
        ws = T.empty(R.decode_workspace_bytes(self.lay, len(loops), w.batch, self.table.shape[1], split_pages),
                     dtype=T.uint8, device=dev())
        ws.fill_(0xFF)
        R.decode_attention(self.lay, pool, list(loops), to_dev(self.q[loops], w.kv_dtype), None, self.d_table,
                           self.d_seq, to_dev(self.tail_k[loops], w.kv_dtype) if tail else None,
                           to_dev(self.tail_v[loops], w.kv_dtype) if tail else None, self.tau, out, ws,
                           split_pages=split_pages)
        T.cuda.synchronize()
        return out.cpu().numpy().astype(np.float64)


CASES = {
    "ouro_int2": lambda: DirectCase(W.get(1).replace(batch=3, heads=3, context=203), (2, 2, 2, 2),
                                    seq_lens=[203, 17, 160]),
    "ouro_mixed": lambda: DirectCase(W.get(1).replace(batch=2, heads=2, context=90, group_size=32,
                                                      meta_dtype="f32"), (4, 2, 4, 2)),
    "huginn_int2": lambda: DirectCase(W.get(3).replace(batch=2, heads=3, context=95), (2,) * 8, seq_lens=[95, 33]),
    "tiny_int4": lambda: DirectCase(W.get(0), (4, 4)),
}
_cache = {}


def case(name):
    if name not in _cache:
        print(f"[case] building {name}", flush=True)
        _cache[name] = CASES[name]()
    return _cache[name]


@pytest.mark.parametrize("name", list(CASES))
def test_direct_encode_matches_oracle(name):
    import looped_transformer_decode_rq_amd as R
    T = torch()
    c = case(name)
    pool = T.zeros(c.olay.pool_bytes, dtype=T.uint8, device=dev())
    R.encode_pack(c.lay, pool, to_dev(c.kv_tok, c.w.kv_dtype), None, T.from_numpy(c.slots).to(dev()))
    g = pool.cpu().numpy()
    pages, offs = c.slots // 16, c.slots % 16
    ar = np.arange(len(c.slots))
    stats = {}
    for l in range(c.w.loops):
        q = c.enc.q[l]
        for kv in range(2):
            for h in range(c.w.heads):
                cg, sg, zg, a = O.read_pages(g, c.olay, pages, h, l, kv)
                assert a is None
                sub = O.Quantized(codes=q.codes[kv, :, h], scale=q.scale[kv, :, h], zero=q.zero[kv, :, h],
                                  u=q.u[kv, :, h], bits=q.bits, step64=q.step64[kv, :, h], lo64=q.lo64[kv, :, h])
                compare_quantized(f"{name} loop {l} kv {kv} h {h}", cg[ar, offs], sg[ar, offs], zg[ar, offs], sub,
                                  c.w.meta_dtype, c.w.group_size, stats)
    check_caps(stats)
    print(f"[direct encode {name}] {stats}", flush=True)


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("split_pages", [0, 1, 3])
def test_direct_decode_matches_oracle(name, split_pages):
    c = case(name)
    pool = torch().from_numpy(c.pool_o.copy()).to(dev())
    L = c.w.loops
    for l in range(L):
        e, r = check_attention(f"{name} loop {l}", c.run(pool, [l], split_pages=split_pages)[0], c.oracle_out(l))
        print(f"[direct {name} loop {l} sp {split_pages}] max-abs {e:.2e} rel-L2 {r:.2e}", flush=True)
    # several loops in one call (one kernel per loop in this mode), without tails
    loops = list(range(L))[::-1]
    got = c.run(pool, loops, tail=False, split_pages=split_pages)
    for i, l in enumerate(loops):
        check_attention(f"{name} multi loop {l}", got[i], c.oracle_out(l, tail=False))


def test_direct_decode_encode_equals_separate():
    import looped_transformer_decode_rq_amd as R
    T = torch()
    c = case("ouro_int2")
    w = c.w
    B, N, L = w.batch, w.context, w.loops
    kv = to_dev(np.ascontiguousarray(c.kv[:, :, :, N]), w.kv_dtype)
    slots = T.from_numpy(np.array([c.table[b, int(c.seq[b]) // 16] * 16 + int(c.seq[b]) % 16 for b in range(B)],
                                  np.int64)).to(dev())
    outs = []
    pools = []
    for fused in (True, False):
        pool = T.from_numpy(c.pool_o.copy()).to(dev())
        out = T.empty((L, B, w.heads, w.head_dim), device=dev())
        ws = T.empty(R.decode_workspace_bytes(c.lay, L, B, c.table.shape[1]), dtype=T.uint8, device=dev())
        args = (c.lay, pool, list(range(L)), to_dev(c.q, w.kv_dtype), None, c.d_table, c.d_seq,
                to_dev(c.tail_k, w.kv_dtype), to_dev(c.tail_v, w.kv_dtype), c.tau, out, ws)
        if fused:
            R.decode_attention(*args, kv_new=kv, slot_mapping=slots)
        else:
            R.decode_attention(*args)
            R.encode_pack(c.lay, pool, kv, None, slots)
        T.cuda.synchronize()
        outs.append(out.cpu().numpy())
        pools.append(pool.cpu().numpy())
    np.testing.assert_array_equal(outs[0], outs[1])
    assert np.array_equal(pools[0], pools[1])
    assert not np.array_equal(pools[0], c.pool_o)
