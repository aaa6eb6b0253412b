"""fp64 reference implementation (test infrastructure only -- see package docstring).

Readings taken where the pages leave a step open (each is listed with its
reason in the design notes of the repository):

R1  alpha granularity: one least-squares scale per (layer, loop, token, head,
    K|V), taken over the D channels of that token-head.
R2  the residual is taken against the exact (unquantized) reference.
R3  the residual uses the stored (rounded) alpha, so that reconstruction is
    consistent with what is stored.
R4  only the residual is rotated; the reference is stored unrotated.
R5  one rotation per (layer, head, K|V), shared by every loop and token.
R6  groups of G contiguous channels inside one head.
R7  asymmetric quantizer: step s = (max-min)/(2^b-1), offset z = min, both
    rounded to the metadata dtype; code = clamp(rint((y-z)/s), 0, 2^b-1);
    dequantized value c*s + z.
R8  a group whose rounded step is 0 stores all-zero codes and decodes to z.
R9  round-to-nearest-even for codes and for every dtype cast.
R10 fp16 step, zero and alpha (fp32 in the tiny fp32 case).
R11 little-endian packing: element i sits in the low bits first.
R12 softmax scale 1/sqrt(D) by default, attention over every cached token plus
    the current (uncompressed) token.
R13 reconstruction of loop l: alpha * xref_hat + R^T dequant(residual).
R18 rotation fitting (a stand-in for calibration; the pages fix no fitting
    rule): alternate (1) quantize the rotated residual samples with the
    quantizer above and (2) the orthogonal Procrustes step, the orthogonal R
    closest to mapping the samples onto their quantized values, R = U V^T for
    M = Yhat D^T = U S V^T; keep the R with the lowest mean squared
    quantization error seen (the starting R included).
R19 storage order of V codes inside a page record (the pages fix no storage
    layout; this is the library's format): tokens in quads, channels in
    column groups of J = min(16, D), one "lane" per (quad, column) holding
    that column's codes of the quad's four tokens for every column group,
    split into 32-bit words and stored word-plane by word-plane (see
    v_code_bits). K codes stay token-major (pack_codes per token).
R20 chunked prefill over the packed cache (the serving setting the pages
    describe; they give no kernel-level definition): a chunk of C new tokens
    per sequence, for one loop, attends all cached (packed) tokens of that
    loop plus the chunk's own uncompressed K/V causally (query i sees chunk
    tokens 0..i); softmax scale as in R12.
R17 the direct per-loop baseline (the "quantize every loop on its own"
    approach the pages compare against): loop l's K/V quantized with the
    quantizer of R6-R10 at its own bit width, no reference, no alpha, no
    rotation; stored in the same paged record format without the alpha field.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

__all__ = [
    "meta_round", "ls_alpha", "Quantized", "quantize", "dequantize",
    "Encoded", "encode", "reconstruct", "pack_codes", "unpack_codes",
    "v_code_bits", "PoolLayout", "write_tokens", "read_pages", "gather_sequence",
    "reconstruct_sequence", "attention", "decode_attention", "chunk_attention",
    "bf16_pool_write", "bf16_decode_attention", "DirectEncoded", "encode_direct",
    "rotation_quant_error", "procrustes", "fit_rotation",
]


# --------------------------------------------------------------------- casts
def meta_round(x, meta: str) -> np.ndarray:
    """Round float64 values to the metadata dtype (nearest even), back as float64.

    Reading R9/R10. numpy converts float64 -> float16 directly from the double
    (no intermediate float32), which is the single rounding wanted here; a test
    pins this against exact rational rounding.
    """
    x = np.asarray(x, dtype=np.float64)
    if meta == "f16":
        return x.astype(np.float16).astype(np.float64)
    if meta == "f32":
        return x.astype(np.float32).astype(np.float64)
    raise ValueError(meta)


def _meta_np(meta: str):
    return np.dtype("<f2") if meta == "f16" else np.dtype("<f4")


# ------------------------------------------------------------ least squares
def ls_alpha(x: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Least-squares scale of the reference for each difference.

    rit.work summary, "how each pass is restored": the coefficient is the one
    that makes the state and the scaled reference differ least in the squared
    sense, i.e. argmin_a ||x - a*ref||^2 = <x, ref> / <ref, ref> (0 when the
    reference is all zeros). Reduction over the last axis (reading R1).
    """
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.sum(x * ref, axis=-1)
    den = np.sum(ref * ref, axis=-1)
    with np.errstate(invalid="ignore", divide="ignore"):
        a = np.where(den == 0, 0.0, num / np.where(den == 0, 1.0, den))
    return a


# ---------------------------------------------------------------- quantizer
@dataclass
class Quantized:
    codes: np.ndarray   # uint8 [..., D]
    scale: np.ndarray   # float64 [..., D/G]  (values exactly in the meta dtype)
    zero: np.ndarray    # float64 [..., D/G]
    u: np.ndarray       # float64 [..., D]  pre-rounding code values (NaN where scale == 0)
    bits: int
    step64: np.ndarray = None   # float64 [..., D/G] (max-min)/(2^b-1) before rounding
    lo64: np.ndarray = None     # float64 [..., D/G] group minimum before rounding


def quantize(y: np.ndarray, bits: int, G: int, meta: str) -> Quantized:
    """Asymmetric uniform group quantizer (readings R6-R9).

    rit.work summary: the quantizer has a tunable step and offset so that all
    levels of the low-bit code are in use instead of spending one on symmetry
    about zero. TaSQ page section 2.1 gives the generic form: the range
    [min, max] cut into 2^b bins, dequantized as index * step + offset.
    """
    y = np.asarray(y, dtype=np.float64)
    D = y.shape[-1]
    assert D % G == 0
    yg = y.reshape(y.shape[:-1] + (D // G, G))
    lo = yg.min(axis=-1)
    hi = yg.max(axis=-1)
    qmax = (1 << bits) - 1
    step64 = (hi - lo) / qmax
    s = meta_round(step64, meta)
    z = meta_round(lo, meta)
    degenerate = s == 0
    with np.errstate(invalid="ignore", divide="ignore"):
        u = (yg - z[..., None]) / np.where(degenerate, 1.0, s)[..., None]
    c = np.clip(np.rint(u), 0, qmax)
    c = np.where(degenerate[..., None], 0, c).astype(np.uint8)
    u = np.where(degenerate[..., None], np.nan, u)
    return Quantized(codes=c.reshape(y.shape), scale=s, zero=z, u=u.reshape(y.shape), bits=bits,
                     step64=step64, lo64=lo)


def dequantize(codes: np.ndarray, scale: np.ndarray, zero: np.ndarray, G: int) -> np.ndarray:
    """code * step + offset, per group of G channels (reading R7)."""
    c = np.asarray(codes, dtype=np.float64)
    D = c.shape[-1]
    cg = c.reshape(c.shape[:-1] + (D // G, G))
    return (cg * np.asarray(scale)[..., None] + np.asarray(zero)[..., None]).reshape(c.shape)


# ------------------------------------------------------------------- encode
@dataclass
class Encoded:
    ref: Quantized            # [2][T][H][D]: INT4 reference (final loop)
    res: list                 # per loop l < L-1: Quantized of the rotated residual
    alpha: list               # per loop l < L-1: stored alpha [2][T][H] (meta dtype)
    alpha64: list             # per loop l < L-1: unrounded least-squares alpha
    G: int
    meta: str


def encode(kv: np.ndarray, rot32: np.ndarray, res_bits, G: int, meta: str) -> Encoded:
    """Compress the K/V of every loop of T tokens, once the final loop has run.

    kv     [L][2][T][H][D]  values of all loops (float64 holding bf16/fp32 values)
    rot32  [H][2][D][D]     rotation per (head, K|V) as fp32, r = R @ d

    Steps (arXiv 2610.10381 abstract; rit.work summary, "how each pass is
    restored"): the final-loop K/V is the reference and is stored in INT4; for
    every other loop the least-squares scale of the reference is found, the
    scaled reference is subtracted, the difference is rotated in channel space
    and stored in low precision (INT2, or INT4 under loop-wise mixed
    precision). Readings R1-R5, R10.
    """
    kv = np.asarray(kv, dtype=np.float64)
    L = kv.shape[0]
    R = np.asarray(rot32, dtype=np.float32).astype(np.float64)  # [H][2][D][D]
    ref = kv[L - 1]                                  # [2][T][H][D]
    ref_q = quantize(ref, 4, G, meta)
    res, alpha, alpha64 = [], [], []
    for l in range(L - 1):
        a64 = ls_alpha(kv[l], ref)                   # [2][T][H]
        a = meta_round(a64, meta)
        d = kv[l] - a[..., None] * ref               # exact in float64 for these inputs
        # r[kv, t, h, :] = R[h, kv] @ d[kv, t, h, :]
        r = np.einsum("hkij,kthj->kthi", R, d, optimize=True)
        res.append(quantize(r, int(res_bits[l]), G, meta))
        alpha.append(a)
        alpha64.append(a64)
    return Encoded(ref=ref_q, res=res, alpha=alpha, alpha64=alpha64, G=G, meta=meta)


def reconstruct(enc: Encoded, rot32: np.ndarray) -> np.ndarray:
    """x_hat of every loop, [L][2][T][H][D] (reading R13).

    Reference: c*s + z. Loop l: alpha * x_ref_hat + R^T (c_r*s_r + z_r); the
    inverse rotation is the transpose of the stored fp32 rotation.
    """
    R = np.asarray(rot32, dtype=np.float32).astype(np.float64)
    G = enc.G
    xr = dequantize(enc.ref.codes, enc.ref.scale, enc.ref.zero, G)
    out = [None] * (len(enc.res) + 1)
    out[-1] = xr
    for l, q in enumerate(enc.res):
        dq = dequantize(q.codes, q.scale, q.zero, G)
        back = np.einsum("hkji,kthj->kthi", R, dq, optimize=True)   # R^T @ dq
        out[l] = enc.alpha[l][..., None] * xr + back
    return np.stack(out)


@dataclass
class DirectEncoded:
    q: list                   # per loop l: Quantized of x_l itself [2][T][H][D]
    G: int
    meta: str


def encode_direct(kv: np.ndarray, bits, G: int, meta: str) -> DirectEncoded:
    """The direct per-loop baseline (reading R17): every loop's K/V quantized
    on its own, with loop l at bits[l] (2 or 4)."""
    kv = np.asarray(kv, dtype=np.float64)
    return DirectEncoded(q=[quantize(kv[l], int(bits[l]), G, meta) for l in range(kv.shape[0])], G=G, meta=meta)


# ------------------------------------------------------------------ packing
def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """Pack codes along the last axis, little-endian inside each byte (R11).

    INT4: element 2j in bits 0-3 of byte j, element 2j+1 in bits 4-7.
    INT2: element 4j+k in bits 2k..2k+1 of byte j.
    """
    c = np.asarray(codes, dtype=np.uint8)
    per = 8 // bits
    D = c.shape[-1]
    assert D % per == 0
    cg = c.reshape(c.shape[:-1] + (D // per, per)).astype(np.uint32)
    out = np.zeros(cg.shape[:-1], dtype=np.uint32)
    for k in range(per):
        out |= (cg[..., k] & ((1 << bits) - 1)) << (bits * k)
    return out.astype(np.uint8)


def unpack_codes(packed: np.ndarray, bits: int) -> np.ndarray:
    """Inverse of pack_codes."""
    p = np.asarray(packed, dtype=np.uint8)
    per = 8 // bits
    parts = [(p >> (bits * k)) & ((1 << bits) - 1) for k in range(per)]
    return np.stack(parts, axis=-1).reshape(p.shape[:-1] + (p.shape[-1] * per,)).astype(np.uint8)


# ------------------------------------------------------------------- layout
def v_code_bits(bs: int, D: int, bits: int) -> np.ndarray:
    """Bit offset of the code of (token t, channel c) inside the V code block
    of one page record, [bs][D] int64 (reading R19).

    Tokens: quad u = t // 4, position v = t % 4 (bs a multiple of 4).
    Channels: column group m = c // J, column j = c % J, J = min(16, D),
    M = D / J groups. Lane lam = J*u + j holds, for m = 0..M-1, the codes of
    (token 4u+v, channel J*m+j), v = 0..3. With W = 8 // bits groups per
    32-bit word, word p of a lane holds groups W*p .. W*p + W_p - 1 where
    W_p = min(W, M - W*p) (the last word may be partial), and inside word p
    the code (group W*p + i, position v) is field
        f = 2*W_p*(v % 2) + W_p*(v // 2) + i,
    i.e. bits [f*bits, (f+1)*bits) of the word, little-endian. Word p of every
    lane forms plane p (lanes in order, W_p*bits/2 bytes each); the planes
    follow one another from plane 0.
    """
    assert bs % 4 == 0 and bits in (2, 4)
    J = min(16, D)
    assert D % J == 0
    M = D // J
    W = 8 // bits
    nlanes = (bs // 4) * J
    wp = [min(W, M - W * p) for p in range(-(-M // W))]
    plane_start = [0]
    for w in wp:
        plane_start.append(plane_start[-1] + nlanes * w * bits // 2)
    pos = np.zeros((bs, D), dtype=np.int64)
    for t in range(bs):
        u, v = divmod(t, 4)
        for c in range(D):
            m, j = divmod(c, J)
            lam = J * u + j
            p, i = divmod(m, W)
            f = 2 * wp[p] * (v % 2) + wp[p] * (v // 2) + i
            byte0 = plane_start[p] + lam * wp[p] * bits // 2
            pos[t, c] = 8 * byte0 + f * bits
    return pos


class PoolLayout:
    """Byte layout of one layer's packed, paged cache (the library's format).

    The pool is [num_blocks][H] slabs; a slab holds, for loops l = 0..L-1 and
    then K (kv=0) before V (kv=1), one page record of ``block_size`` tokens:

        codes  block_size * D*b_l/8 bytes: K token-major (pack_codes per
               token), V in the order of v_code_bits (reading R19)
        meta   block_size * (D/G) pairs (scale, zero), token-major, meta dtype
        alpha  block_size values, meta dtype          (residual loops only)
        pad    to a multiple of 16 bytes

    b_l = res_bits[l] for l < L-1 and 4 for the reference loop L-1. The paged
    cache management itself (block table, slots) is the usual one; the pages
    only change what is stored per token (rit.work summary: scheduler and paged
    management stay as they are).

    Direct mode (``direct_bits`` given, reading R17): every loop's record holds
    its own codes at ``direct_bits[l]`` bits and the (scale, zero) pairs, with
    no alpha field; ``res_bits`` is then unused.
    """

    def __init__(self, H, D, G, L, res_bits, meta, num_blocks, block_size=16, direct_bits=None):
        self.H, self.D, self.G, self.L = int(H), int(D), int(G), int(L)
        self.direct = direct_bits is not None
        if self.direct:
            self.dbits = tuple(int(b) for b in direct_bits)
            assert len(self.dbits) == self.L
            self.res_bits = ()
        else:
            self.res_bits = tuple(int(b) for b in res_bits)
            assert len(self.res_bits) == self.L - 1
        self.meta = meta
        self.msz = 2 if meta == "f16" else 4
        self.num_blocks = int(num_blocks)
        self.bs = int(block_size)

    def bits(self, l):
        if self.direct:
            return self.dbits[l]
        return 4 if l == self.L - 1 else self.res_bits[l]

    def code_bytes(self, l):
        return self.bs * self.D * self.bits(l) // 8

    def meta_bytes(self):
        return self.bs * 2 * (self.D // self.G) * self.msz

    def alpha_bytes(self, l):
        return self.bs * self.msz if (l < self.L - 1 and not self.direct) else 0

    def rec_bytes(self, l):
        n = self.code_bytes(l) + self.meta_bytes() + self.alpha_bytes(l)
        return (n + 15) // 16 * 16

    def loop_offset(self, l):
        return sum(2 * self.rec_bytes(j) for j in range(l))

    @property
    def slab_bytes(self):
        return self.loop_offset(self.L)

    @property
    def pool_bytes(self):
        return self.num_blocks * self.H * self.slab_bytes

    def record_offset(self, block, head, l, kv):
        block = np.asarray(block, dtype=np.int64)
        return (block * self.H + head) * self.slab_bytes + self.loop_offset(l) + kv * self.rec_bytes(l)


def write_tokens(pool: np.ndarray, lay: PoolLayout, enc: Encoded, slots: np.ndarray) -> None:
    """Scatter encoded tokens into their page records (slot = page*block + offset).

    The write happens once per token, after its final loop (rit.work summary:
    the current token's intermediate KV stay uncompressed until the final pass
    and the compressed write is deferred until then).
    """
    slots = np.asarray(slots, dtype=np.int64)
    page, off = slots // lay.bs, slots % lay.bs
    mdt = _meta_np(lay.meta)
    ng = lay.D // lay.G
    direct = isinstance(enc, DirectEncoded)
    assert direct == lay.direct
    for l in range(lay.L):
        q = enc.q[l] if direct else (enc.ref if l == lay.L - 1 else enc.res[l])
        b = lay.bits(l)
        tb = lay.D * b // 8
        packed = pack_codes(q.codes, b)                     # [2][T][H][tb]
        vpos = v_code_bits(lay.bs, lay.D, b)[off]           # [T][D] bit offsets of V codes
        vmask = (1 << b) - 1
        for kv in range(2):
            for h in range(lay.H):
                base = lay.record_offset(page, h, l, kv)    # [T]
                if kv == 0:
                    cidx = (base + off * tb)[:, None] + np.arange(tb)
                    pool[cidx] = packed[kv, :, h, :]
                else:
                    # codes of several tokens can share a byte: clear then set
                    # each code's bits with unbuffered (repeat-safe) updates
                    byte = base[:, None] + vpos // 8
                    sh = (vpos % 8).astype(np.uint8)
                    code = q.codes[kv, :, h, :].astype(np.uint8)
                    np.bitwise_and.at(pool, byte.ravel(), (~(np.uint8(vmask) << sh)).ravel().astype(np.uint8))
                    np.bitwise_or.at(pool, byte.ravel(), (code << sh).ravel().astype(np.uint8))
                meta = np.stack([q.scale[kv, :, h, :], q.zero[kv, :, h, :]], axis=-1)
                mb = np.ascontiguousarray(meta.astype(mdt)).view(np.uint8).reshape(len(slots), -1)
                midx = (base + lay.code_bytes(l) + off * (2 * ng * lay.msz))[:, None] + np.arange(mb.shape[1])
                pool[midx] = mb
                if lay.alpha_bytes(l):
                    ab = np.ascontiguousarray(enc.alpha[l][kv, :, h].astype(mdt)).view(np.uint8).reshape(len(slots), -1)
                    aidx = (base + lay.code_bytes(l) + lay.meta_bytes() + off * lay.msz)[:, None] + np.arange(lay.msz)
                    pool[aidx] = ab


def read_pages(pool: np.ndarray, lay: PoolLayout, pages, head: int, l: int, kv: int):
    """Decode the records of ``pages`` for (head, loop, kv).

    Returns codes [P][bs][D] uint8, scale/zero [P][bs][D/G] float64, alpha
    [P][bs] float64 (None for the reference loop).
    """
    pages = np.asarray(pages, dtype=np.int64)
    rec = lay.rec_bytes(l)
    idx = lay.record_offset(pages, head, l, kv)[:, None] + np.arange(rec)
    raw = pool[idx]                                          # [P][rec]
    b = lay.bits(l)
    tb = lay.D * b // 8
    if kv == 0:
        codes = unpack_codes(raw[:, : lay.bs * tb].reshape(len(pages), lay.bs, tb), b)
    else:
        vpos = v_code_bits(lay.bs, lay.D, b)                 # [bs][D]
        codes = ((raw[:, vpos // 8] >> (vpos % 8).astype(np.uint8)) & ((1 << b) - 1)).astype(np.uint8)
    mdt = _meta_np(lay.meta)
    mbytes = raw[:, lay.code_bytes(l): lay.code_bytes(l) + lay.meta_bytes()]
    meta = np.ascontiguousarray(mbytes).view(mdt).astype(np.float64).reshape(len(pages), lay.bs, lay.D // lay.G, 2)
    alpha = None
    if lay.alpha_bytes(l):
        a0 = lay.code_bytes(l) + lay.meta_bytes()
        alpha = np.ascontiguousarray(raw[:, a0: a0 + lay.alpha_bytes(l)]).view(mdt).astype(np.float64).reshape(len(pages), lay.bs)
    return codes, meta[..., 0], meta[..., 1], alpha


def gather_sequence(pool, lay: PoolLayout, table_row, n_tokens: int, head: int, l: int, kv: int):
    """Tokens 0..n-1 of one sequence for (head, loop, kv), following its block table."""
    n_pages = -(-n_tokens // lay.bs)
    codes, s, z, a = read_pages(pool, lay, np.asarray(table_row)[:n_pages], head, l, kv)
    flat = lambda x: None if x is None else x.reshape((-1,) + x.shape[2:])[:n_tokens]
    return flat(codes), flat(s), flat(z), flat(a)


def reconstruct_sequence(pool, lay: PoolLayout, table_row, n_tokens: int, head: int, l: int,
                         rot32_h: np.ndarray):
    """Reconstructed K_hat, V_hat [N][D] of loop l for one (sequence, head).

    rit.work summary: attention rebuilds the reference and the loop's own
    difference from the compressed cache (each loop reads only the reference
    and its own residual). rot32_h is [2][D][D] for this head.
    """
    out = []
    if lay.direct:
        # direct baseline (R17): loop l's own record, nothing else
        for kv in range(2):
            c, s, z, _ = gather_sequence(pool, lay, table_row, n_tokens, head, l, kv)
            out.append(dequantize(c, s, z, lay.G))
        return out[0], out[1]
    R = np.asarray(rot32_h, dtype=np.float32).astype(np.float64)
    for kv in range(2):
        c, s, z, _ = gather_sequence(pool, lay, table_row, n_tokens, head, lay.L - 1, kv)
        xr = dequantize(c, s, z, lay.G)
        if l == lay.L - 1:
            out.append(xr)
            continue
        c2, s2, z2, a2 = gather_sequence(pool, lay, table_row, n_tokens, head, l, kv)
        dq = dequantize(c2, s2, z2, lay.G)
        out.append(a2[:, None] * xr + dq @ R[kv])          # rows: (R^T dq)^T = dq^T R
    return out[0], out[1]


# ---------------------------------------------------------------- attention
def attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, tau: float,
              tail_k=None, tail_v=None) -> np.ndarray:
    """Single-query softmax attention, brute force in float64.

    s_t = tau * q.k_t over every key (cached tokens plus the optional current
    token); p = exp(s - max s) / sum; o = sum_t p_t v_t. An empty key set gives
    a zero vector.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64).reshape(-1, q.shape[-1])
    V = np.asarray(V, dtype=np.float64).reshape(-1, q.shape[-1])
    if tail_k is not None:
        K = np.concatenate([K, np.asarray(tail_k, dtype=np.float64)[None]], axis=0)
        V = np.concatenate([V, np.asarray(tail_v, dtype=np.float64)[None]], axis=0)
    if K.shape[0] == 0:
        return np.zeros_like(q)
    s = tau * (K @ q)
    p = np.exp(s - s.max())
    return (p @ V) / p.sum()


def decode_attention(pool, lay: PoolLayout, l: int, q, rot32, table, seq_lens, tau,
                     tail_k=None, tail_v=None, pairs=None) -> np.ndarray:
    """Decode attention of loop l over the packed cache, [B][H][D] float64.

    q [B][H][D]; tail_k/tail_v [B][H][D] or None (current token, uncompressed).
    ``pairs``: optional list of (b, h) to compute; other rows are left NaN.
    """
    q = np.asarray(q, dtype=np.float64)
    B, H, D = q.shape
    out = np.full((B, H, D), np.nan)
    todo = pairs if pairs is not None else [(b, h) for b in range(B) for h in range(H)]
    for b, h in todo:
        n = int(seq_lens[b])
        K, V = reconstruct_sequence(pool, lay, table[b], n, h, l, None if rot32 is None else rot32[h])
        tk = None if tail_k is None else tail_k[b, h]
        tv = None if tail_v is None else tail_v[b, h]
        out[b, h] = attention(q[b, h], K, V, tau, tk, tv)
    return out


def chunk_attention(pool, lay: PoolLayout, l: int, q, rot32, table, seq_lens, tau,
                    chunk_k=None, chunk_v=None, pairs=None) -> np.ndarray:
    """Attention of a chunk of C queries per sequence over loop l's packed
    cache and, causally, over the chunk itself; [B][C][H][D] float64 (reading
    R20).

    q [B][C][H][D]; chunk_k/chunk_v [B][C][H][D] (the chunk's own K/V of loop
    l, uncompressed) or None. Query i of sequence b attends the seq_lens[b]
    reconstructed cached tokens and chunk tokens 0..i, each key once, with
    plain softmax (same brute force as ``attention``). The serving context of
    the rit.work summary (a prefill chunk reading the compressed cache) gives
    the setting; with C = 1 this is decode attention with the chunk token as
    the uncompressed current token.
    """
    q = np.asarray(q, dtype=np.float64)
    B, C, H, D = q.shape
    out = np.full((B, C, H, D), np.nan)
    todo = pairs if pairs is not None else [(b, h) for b in range(B) for h in range(H)]
    for b, h in todo:
        n = int(seq_lens[b])
        K, V = reconstruct_sequence(pool, lay, table[b], n, h, l, None if rot32 is None else rot32[h])
        for i in range(C):
            if chunk_k is not None:
                Kc = np.concatenate([K, np.asarray(chunk_k[b, : i + 1, h], dtype=np.float64)], axis=0)
                Vc = np.concatenate([V, np.asarray(chunk_v[b, : i + 1, h], dtype=np.float64)], axis=0)
            else:
                Kc, Vc = K, V
            out[b, i, h] = attention(q[b, i, h], Kc, Vc, tau)
    return out


# ----------------------------------------------------------- BF16 baseline
def bf16_pool_write(kcache: np.ndarray, vcache: np.ndarray, kv_loop: np.ndarray, slots) -> None:
    """Uncompressed paged cache [num_blocks][H][bs][D] of one loop (baseline).

    kv_loop [2][T][H][D]: values already in bf16; written at their slots.
    """
    slots = np.asarray(slots, dtype=np.int64)
    bs = kcache.shape[2]
    page, off = slots // bs, slots % bs
    kcache[page, :, off, :] = kv_loop[0]
    vcache[page, :, off, :] = kv_loop[1]


def bf16_decode_attention(kcache, vcache, q, table, seq_lens, tau, tail_k=None, tail_v=None,
                          pairs=None) -> np.ndarray:
    """Baseline decode attention over an uncompressed paged cache, [B][H][D]."""
    q = np.asarray(q, dtype=np.float64)
    B, H, D = q.shape
    bs = kcache.shape[2]
    out = np.full((B, H, D), np.nan)
    todo = pairs if pairs is not None else [(b, h) for b in range(B) for h in range(H)]
    for b, h in todo:
        n = int(seq_lens[b])
        pages = np.asarray(table[b])[: -(-n // bs)]
        K = np.asarray(kcache[pages, h], dtype=np.float64).reshape(-1, D)[:n]
        V = np.asarray(vcache[pages, h], dtype=np.float64).reshape(-1, D)[:n]
        tk = None if tail_k is None else tail_k[b, h]
        tv = None if tail_v is None else tail_v[b, h]
        out[b, h] = attention(q[b, h], K, V, tau, tk, tv)
    return out


# ---------------------------------------------------------- rotation fitting
def rotation_quant_error(samples: np.ndarray, R: np.ndarray, bits: int, G: int, meta: str) -> float:
    """Mean over samples of ||Q(R d) - R d||^2 (reading R18); samples [n][D]."""
    Y = np.asarray(samples, dtype=np.float64) @ np.asarray(R, dtype=np.float64).T      # rows: (R d)^T
    q = quantize(Y, bits, G, meta)
    Yh = dequantize(q.codes, q.scale, q.zero, G)
    return float(((Yh - Y) ** 2).sum() / Y.shape[0])


def procrustes(M: np.ndarray) -> np.ndarray:
    """argmax_R trace(R^T M) over orthogonal R (= argmin ||R D - Yhat|| for
    M = Yhat D^T): R = U V^T from the SVD M = U S V^T."""
    U, _, Vt = np.linalg.svd(np.asarray(M, dtype=np.float64))
    return U @ Vt


def fit_rotation(samples: np.ndarray, R0: np.ndarray, bits: int, G: int, meta: str, iters: int):
    """Reading R18. Returns (best R, objective of R0 and of every iterate)."""
    Dm = np.asarray(samples, dtype=np.float64)                 # [n][D]
    R = np.asarray(R0, dtype=np.float32).astype(np.float64)
    best, best_err = R.copy(), rotation_quant_error(Dm, R, bits, G, meta)
    hist = [best_err]
    for _ in range(iters):
        Y = Dm @ R.T
        q = quantize(Y, bits, G, meta)
        Yh = dequantize(q.codes, q.scale, q.zero, G)           # [n][D]
        R = procrustes(Yh.T @ Dm)                              # sum_i yhat_i d_i^T
        err = rotation_quant_error(Dm, R, bits, G, meta)
        hist.append(err)
        if err < best_err:
            best, best_err = R.copy(), err
    return best, hist
