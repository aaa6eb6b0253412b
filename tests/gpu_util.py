"""Shared helpers of the GPU parity tests: device upload of generator data,
oracle references, and the comparison rules.

Comparison rules:
* packed codes are bit-exact, except elements whose pre-rounding value
  (y - zero)/step, as the oracle computes it, lies within 1e-6 of a rounding
  boundary (a half-integer); such elements are counted and capped at 1e-5 of
  all elements;
* scale, zero and alpha are bit-exact, except where the oracle's value before
  rounding lies within 1e-6*step (alpha: 1e-6 relative) of a rounding boundary
  of the metadata dtype; such groups are counted (cap 1e-4 of groups), and
  their codes are checked against the codes the oracle's values give under the
  GPU's stored scale and zero, by the same rule and toward the same cap;
* attention outputs: max-abs error <= 2e-3 and rel-L2 error <= 1e-3 against
  the oracle run on the same packed inputs.
"""
from __future__ import annotations

import numpy as np

import oracle as O
import workloads as W

ATOL = 2e-3
REL_L2 = 1e-3
CODE_BAND = 1e-6
CODE_CAP = 1e-5
META_CAP = 1e-4


def torch():
    import torch as T
    return T


def dev():
    return torch().device("cuda:0")


def to_dev(x: np.ndarray, dtype: str):
    """float64 array holding bf16/fp32 values -> device tensor of that dtype."""
    T = torch()
    if dtype == "bf16":
        bits = W.bf16_bits(x).view(np.int16)
        return T.from_numpy(np.ascontiguousarray(bits)).view(T.bfloat16).to(dev())
    return T.from_numpy(np.ascontiguousarray(x.astype(np.float32))).to(dev())


def to_host64(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def oracle_layout(w: W.Workload, nblk: int) -> O.PoolLayout:
    return O.PoolLayout(w.heads, w.head_dim, w.group_size, w.loops, w.res_bits, w.meta_dtype, nblk)


def lib_layout(w: W.Workload, nblk: int):
    import looped_transformer_decode_rq_amd as R
    return R.make_layout(w.heads, w.head_dim, w.group_size, w.loops, w.res_bits, nblk, w.meta_dtype, w.kv_dtype)


# ------------------------------------------------------------ comparisons
def _near_half(u):
    return np.abs(u - (np.floor(u) + 0.5)) < CODE_BAND


def _near_boundary(v64, meta, band):
    """True where v64 lies within band of a rounding boundary of the meta dtype."""
    v64 = np.asarray(v64, dtype=np.float64)
    dt = np.float16 if meta == "f16" else np.float32
    r = v64.astype(dt)
    up = np.nextafter(r, dt(np.inf)).astype(np.float64)
    dn = np.nextafter(r, dt(-np.inf)).astype(np.float64)
    rf = r.astype(np.float64)
    mid = np.where(v64 >= rf, (rf + up) / 2, (rf + dn) / 2)
    return np.abs(v64 - mid) <= band


def compare_quantized(tag, codes_g, scale_g, zero_g, q: O.Quantized, meta: str, G: int, stats: dict,
                      alpha_g=None, alpha_o=None, alpha64=None):
    """Compare GPU codes/metadata of some token-heads against the oracle's.

    codes_g [..., D], scale_g/zero_g [..., D/G], q the oracle's Quantized of the
    same token-heads. Updates stats counters; raises AssertionError on a
    mismatch that the rules do not exempt.
    """
    D = codes_g.shape[-1]
    ng = D // G
    meta_bad = (scale_g != q.scale) | (zero_g != q.zero)
    if meta_bad.any():
        ok = (_near_boundary(q.step64, meta, CODE_BAND * np.abs(q.scale) + 1e-300) |
              _near_boundary(q.lo64, meta, CODE_BAND * np.abs(q.scale) + 1e-300))
        assert np.all(ok[meta_bad]), f"{tag}: scale/zero differ off a rounding boundary"
    stats["groups"] = stats.get("groups", 0) + meta_bad.size
    stats["meta_exempt"] = stats.get("meta_exempt", 0) + int(meta_bad.sum())
    if alpha_g is not None:
        abad = alpha_g != alpha_o
        if abad.any():
            ok = _near_boundary(alpha64, meta, CODE_BAND * np.abs(alpha64) + 1e-300)
            assert np.all(ok[abad]), f"{tag}: alpha differs off a rounding boundary"
        stats["meta_exempt"] = stats.get("meta_exempt", 0) + int(abad.sum())
    # codes: where the group metadata agree, against the oracle's codes; in a
    # metadata-exempt group, against the codes the oracle's pre-rounding
    # values give under the GPU's stored scale and zero (same rounding rule)
    u = np.array(q.u, dtype=np.float64)
    want = np.array(q.codes)
    if meta_bad.any():
        s_o, z_o = np.repeat(q.scale, G, axis=-1), np.repeat(q.zero, G, axis=-1)
        s_g, z_g = np.repeat(scale_g, G, axis=-1).astype(np.float64), np.repeat(zero_g, G, axis=-1).astype(np.float64)
        bad = np.repeat(meta_bad, G, axis=-1)
        y = np.where(np.isnan(u), z_o, u * s_o + z_o)   # a degenerate oracle group: every value ~ zero
        with np.errstate(divide="ignore", invalid="ignore"):
            u2 = np.where(s_g != 0, (y - z_g) / np.where(s_g != 0, s_g, 1.0), 0.0)
        c2 = np.where(s_g != 0, np.clip(np.rint(u2), 0, 2 ** q.bits - 1), 0).astype(want.dtype)
        u = np.where(bad, u2, u)
        want = np.where(bad, c2, want)
    diff = codes_g != want
    if diff.any():
        assert np.all(_near_half(u[diff])), f"{tag}: {int(diff.sum())} codes differ off a rounding boundary"
    stats["codes"] = stats.get("codes", 0) + codes_g.size
    stats["code_exempt"] = stats.get("code_exempt", 0) + int(diff.sum())


def check_caps(stats):
    if stats.get("codes"):
        assert stats["code_exempt"] <= CODE_CAP * stats["codes"], stats
    if stats.get("groups"):
        assert stats["meta_exempt"] <= META_CAP * stats["groups"], stats


def compare_pool_tokens(tag, pool_g: np.ndarray, lay: O.PoolLayout, enc: O.Encoded, slots: np.ndarray,
                        stats: dict):
    """Check every encoded token of `enc` (written at `slots`) in the GPU pool."""
    slots = np.asarray(slots, dtype=np.int64)
    pages, offs = slots // lay.bs, slots % lay.bs
    for l in range(lay.L):
        q = enc.ref if l == lay.L - 1 else enc.res[l]
        for kv in range(2):
            for h in range(lay.H):
                c, s, z, a = O.read_pages(pool_g, lay, pages, h, l, kv)
                ar = np.arange(len(slots))
                cg, sg, zg = c[ar, offs], s[ar, offs], z[ar, offs]
                sub = O.Quantized(codes=q.codes[kv, :, h], scale=q.scale[kv, :, h], zero=q.zero[kv, :, h],
                                  u=q.u[kv, :, h], bits=q.bits, step64=q.step64[kv, :, h], lo64=q.lo64[kv, :, h])
                if l < lay.L - 1:
                    compare_quantized(f"{tag} loop {l} kv {kv} head {h}", cg, sg, zg, sub, lay.meta, lay.G, stats,
                                      a[ar, offs], enc.alpha[l][kv, :, h], enc.alpha64[l][kv, :, h])
                else:
                    compare_quantized(f"{tag} ref kv {kv} head {h}", cg, sg, zg, sub, lay.meta, lay.G, stats)


def check_attention(tag, got: np.ndarray, want: np.ndarray):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{tag}: non-finite output"
    err = np.abs(got - want)
    rel = np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30)
    assert err.max() <= ATOL and rel <= REL_L2, f"{tag}: max-abs {err.max():.3e} rel-L2 {rel:.3e}"
    return float(err.max()), float(rel)


# --------------------------------------------------------------- builders
class SmallCase:
    """A workload small enough for the oracle end to end, with its inputs on
    both sides: generator arrays (host), oracle-packed pool, device tensors."""

    def __init__(self, w: W.Workload, shuffled=None, seq_lens=None, spare=3):
        self.w = w
        T = torch()
        B, N, H, D, L = w.batch, w.context, w.heads, w.head_dim, w.loops
        self.st = W.structure(w)
        self.kv = W.kv_numpy(w, st=self.st)                    # [L][2][B][N+1][H][D]
        self.q = W.queries_numpy(w)                              # [L][B][H][D]
        self.table, self.nblk = W.block_table(w, spare_blocks=spare, shuffled=shuffled)
        self.seq = np.full(B, N, dtype=np.int32) if seq_lens is None else np.asarray(seq_lens, np.int32)
        self.olay = oracle_layout(w, self.nblk)
        self.lay = lib_layout(w, self.nblk)
        # tokens 0..seq_b-1 of every sequence go to the cache; token N is the current one
        pos = [np.arange(int(self.seq[b])) for b in range(B)]
        self.tok_b = np.concatenate([np.full(len(p), b) for b, p in enumerate(pos)]).astype(np.int64)
        self.tok_p = np.concatenate(pos).astype(np.int64)
        self.slots = (self.table[self.tok_b, self.tok_p // 16].astype(np.int64) * 16 + self.tok_p % 16)
        self.kv_tok = self.kv[:, :, self.tok_b, self.tok_p]           # [L][2][T][H][D]
        self.enc = O.encode(self.kv_tok, self.st["rot32"], w.res_bits, w.group_size, w.meta_dtype)
        self.pool_o = np.zeros(self.olay.pool_bytes, np.uint8)
        O.write_tokens(self.pool_o, self.olay, self.enc, self.slots)
        self.tail_k = self.kv[:, 0, :, N]                            # [L][B][H][D]
        self.tail_v = self.kv[:, 1, :, N]
        self.tau = 1.0 / np.sqrt(D)
        # device copies
        self.d_rot = T.from_numpy(self.st["rot32"]).to(dev())
        self.d_table = T.from_numpy(self.table).to(dev())
        self.d_seq = T.from_numpy(self.seq).to(dev())
        self.d_slots = T.from_numpy(self.slots).to(dev())
        self.d_kv_tok = to_dev(self.kv_tok, w.kv_dtype)

    def device_pool_from_oracle(self):
        T = torch()
        return T.from_numpy(self.pool_o.copy()).to(dev())

    def oracle_out(self, l, tail=True, pairs=None):
        return O.decode_attention(self.pool_o, self.olay, l, self.q[l], self.st["rot32"], self.table, self.seq,
                                  self.tau, self.tail_k[l] if tail else None, self.tail_v[l] if tail else None,
                                  pairs=pairs)

    def run_decode(self, pool, loops, tail=True, split_pages=0):
        import looped_transformer_decode_rq_amd as R
        T = torch()
        w = self.w
        loops = list(loops)
        q = to_dev(self.q[loops], w.kv_dtype)
        tk = to_dev(self.tail_k[loops], w.kv_dtype) if tail else None
        tv = to_dev(self.tail_v[loops], w.kv_dtype) if tail else None
        out = T.full((len(loops), w.batch, w.heads, w.head_dim), float("nan"), device=dev())
        ws = T.empty(R.decode_workspace_bytes(self.lay, len(loops), w.batch, self.table.shape[1], split_pages),
                     dtype=T.uint8, device=dev())
        ws.fill_(0xFF)   # poison: stale workspace contents must never reach the output
        R.decode_attention(self.lay, pool, loops, q, self.d_rot, self.d_table, self.d_seq, tk, tv, self.tau, out,
                           ws, split_pages=split_pages)
        T.cuda.synchronize()
        return out.cpu().numpy().astype(np.float64)
