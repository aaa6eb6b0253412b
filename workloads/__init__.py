"""Seeded synthetic workloads for ResidualQuant decode attention.

This module is shared by the tests, the benchmark and the smoke check. It only
draws random numbers, rounds the drawn values to their storage dtype and builds
page tables. It holds no step of the method itself (no least-squares scale, no
quantizer, no packing): those live in ``oracle/`` (CPU reference) and in the HIP
library, which share no code.

Data model (what the looped-Transformer pages describe as the observation that
makes the method work: KV states of different loops are highly similar, and the
final loop serves as reference -- arXiv 2610.10381 abstract; rit.work summary,
section on why a shared block still makes a large cache):

* per (layer, kv, head) a channel scale sigma_c = exp(0.5 * N(0,1)); round(0.02*D)
  channels, picked by a seeded permutation, are multiplied by 10 (outliers);
* reference (final loop) ref[t, c] = sigma_c * N(0, 1);
* loop l < L-1: x_l = a_l * ref + N(0, sigma_l^2), one a_l ~ U(lo, hi) per
  (layer, loop, kv, head);
* queries q ~ N(0, 1/D);
* rotations R_{h,kv}: Q factor of a seeded Gaussian D x D, columns sign-fixed
  so that diag(R_qr) > 0, handed to the library as fp32;
* values are rounded to bf16 (round-to-nearest-even) except the fp32 tiny case.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "get", "bf16_round", "bf16_bits",
    "structure", "kv_numpy", "queries_numpy", "block_table", "slot_mapping",
    "kv_torch", "queries_torch", "outlier_queries",
]


@dataclass(frozen=True)
class Workload:
    name: str
    layers: int
    heads: int
    head_dim: int
    loops: int
    batch: int
    context: int
    group_size: int
    res_bits: tuple          # bits of residual loops 0..L-2 (the reference loop is INT4)
    kv_dtype: str            # 'bf16' or 'f32': dtype of K/V, queries and tails
    meta_dtype: str          # 'f16' or 'f32': dtype of scale, zero and alpha
    alpha_range: tuple
    sigma: tuple             # noise std of each residual loop
    shuffled_table: bool
    seed: int
    block_size: int = 16

    @property
    def ref_loop(self) -> int:
        return self.loops - 1

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _lin(a, b, n):
    if n == 1:
        return (float(a),)
    return tuple(float(v) for v in np.linspace(a, b, n))


# The five looped-model workloads: a tiny fp32 case, an Ouro-1.4B-like layer,
# the same layer at long context (split-K, paged), a Huginn-3.5B-like layer with
# loop-wise mixed precision, and a 24-layer peak-batch step with a shuffled table.
WORKLOADS = {
    "tiny_d64_l2_n256": Workload(
        name="tiny_d64_l2_n256", layers=1, heads=1, head_dim=64, loops=2, batch=1,
        context=256, group_size=32, res_bits=(2,), kv_dtype="f32", meta_dtype="f32",
        alpha_range=(0.8, 1.2), sigma=(0.1,), shuffled_table=False, seed=0),
    "ouro_h16_d128_l4_b32_n4096": Workload(
        name="ouro_h16_d128_l4_b32_n4096", layers=1, heads=16, head_dim=128, loops=4,
        batch=32, context=4096, group_size=128, res_bits=(2, 2, 2), kv_dtype="bf16",
        meta_dtype="f16", alpha_range=(0.8, 1.2), sigma=_lin(0.2, 0.05, 3),
        shuffled_table=False, seed=1),
    "ouro_h16_d128_l4_b16_n32768": Workload(
        name="ouro_h16_d128_l4_b16_n32768", layers=1, heads=16, head_dim=128, loops=4,
        batch=16, context=32768, group_size=128, res_bits=(2, 2, 2), kv_dtype="bf16",
        meta_dtype="f16", alpha_range=(0.8, 1.2), sigma=_lin(0.2, 0.05, 3),
        shuffled_table=False, seed=2),
    "huginn_h55_d96_l8_b8_n8192_mixed": Workload(
        name="huginn_h55_d96_l8_b8_n8192_mixed", layers=1, heads=55, head_dim=96, loops=8,
        batch=8, context=8192, group_size=96, res_bits=(4, 4, 2, 2, 2, 2, 2),
        kv_dtype="bf16", meta_dtype="f16", alpha_range=(0.6, 1.4),
        sigma=tuple(0.05 * (8 - l) for l in range(7)), shuffled_table=False, seed=3),
    "ouro_24layer_h16_d128_l4_b128_n8192": Workload(
        name="ouro_24layer_h16_d128_l4_b128_n8192", layers=24, heads=16, head_dim=128,
        loops=4, batch=128, context=8192, group_size=128, res_bits=(2, 2, 2),
        kv_dtype="bf16", meta_dtype="f16", alpha_range=(0.8, 1.2),
        sigma=_lin(0.2, 0.05, 3), shuffled_table=True, seed=4),
}
ORDER = list(WORKLOADS)


def get(key) -> Workload:
    """Workload by name or by its index in the order above (0 = tiny case)."""
    if isinstance(key, int):
        return WORKLOADS[ORDER[key]]
    return WORKLOADS[key]


# ----------------------------------------------------------------- dtype rounding
def bf16_bits(x) -> np.ndarray:
    """uint16 bf16 bit patterns of x, rounded to nearest even (finite inputs)."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_round(x) -> np.ndarray:
    """x rounded to bf16 (nearest even), returned as float64."""
    b = bf16_bits(x).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def _store_round(w: Workload, x) -> np.ndarray:
    if w.kv_dtype == "bf16":
        return bf16_round(x)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


# ------------------------------------------------------------- structure draws
def _rng(w: Workload, layer: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([w.seed, layer, stream])


def structure(w: Workload, layer: int = 0) -> dict:
    """Per-layer structure: channel scales, drawn loop scales, noise levels, rotations.

    Returns float64 arrays; ``rot32`` is the rotation rounded to fp32 exactly as
    it is handed to the library (layout [H][2][D][D], r = R @ d).
    """
    H, D, L = w.heads, w.head_dim, w.loops
    g = _rng(w, layer, 0)
    scale = np.exp(0.5 * g.standard_normal((2, H, D)))
    n_out = int(round(0.02 * D))
    for kv in range(2):
        for h in range(H):
            idx = g.permutation(D)[:n_out]
            scale[kv, h, idx] *= 10.0
    lo, hi = w.alpha_range
    alpha = g.uniform(lo, hi, size=(max(L - 1, 0), 2, H))
    rot = np.empty((H, 2, D, D))
    for h in range(H):
        for kv in range(2):
            a = g.standard_normal((D, D))
            qm, rm = np.linalg.qr(a)
            rot[h, kv] = qm * np.sign(np.diag(rm))[None, :]
    return {
        "scale": scale, "alpha": alpha, "sigma": np.asarray(w.sigma, dtype=np.float64),
        "rot64": rot, "rot32": rot.astype(np.float32),
    }


# --------------------------------------------------------- bulk draws: numpy
def kv_numpy(w: Workload, layer: int = 0, batch=None, context=None, st=None) -> np.ndarray:
    """K/V of all loops for context+1 tokens per sequence (the last token is the
    current one, held uncompressed), rounded to the storage dtype.

    Shape [L][2][B][N+1][H][D], float64 holding bf16/fp32 values.
    """
    B = w.batch if batch is None else batch
    N = w.context if context is None else context
    st = structure(w, layer) if st is None else st
    H, D, L = w.heads, w.head_dim, w.loops
    g = _rng(w, layer, 1)
    ref = st["scale"][:, None, None, :, :] * g.standard_normal((2, B, N + 1, H, D))
    out = np.empty((L, 2, B, N + 1, H, D))
    for l in range(L - 1):
        a = st["alpha"][l][:, None, None, :, None]
        out[l] = _store_round(w, a * ref + st["sigma"][l] * g.standard_normal(ref.shape))
    out[L - 1] = _store_round(w, ref)
    return out


def queries_numpy(w: Workload, layer: int = 0, batch=None) -> np.ndarray:
    """Decode queries, one per loop: [L][B][H][D] float64 holding bf16/fp32 values."""
    B = w.batch if batch is None else batch
    g = _rng(w, layer, 2)
    q = g.standard_normal((w.loops, B, w.heads, w.head_dim)) / np.sqrt(w.head_dim)
    return _store_round(w, q)


def outlier_queries(w: Workload, q: np.ndarray, mult: float, zero_rows=(), seed: int = 0) -> np.ndarray:
    """Queries with one large channel: per (loop, sequence, head) one seeded
    channel of q is multiplied by ``mult`` (then rounded to the storage dtype);
    the sequences in ``zero_rows`` get an all-zero query. q: [L][B][H][D]."""
    q = np.array(q, dtype=np.float64)
    L, B, H, D = q.shape
    g = np.random.default_rng([w.seed, 31, seed])
    ch = g.integers(0, D, size=(L, B, H))
    li, bi, hi = np.meshgrid(np.arange(L), np.arange(B), np.arange(H), indexing="ij")
    q[li, bi, hi, ch] *= mult
    q = _store_round(w, q)
    for b in zero_rows:
        q[:, b] = 0.0
    return q


# ------------------------------------------------------------------- paging
def block_table(w: Workload, batch=None, context=None, spare_blocks: int = 0,
                shuffled=None) -> tuple:
    """Block table [B][max_blocks] (int32) and pool size.

    Each sequence gets ceil((N+1)/block) pages, so that the current token also
    has a slot once it is written. Identity order (b-major) unless shuffled, in
    which case physical ids are a seeded permutation of the pool.
    """
    B = w.batch if batch is None else batch
    N = w.context if context is None else context
    bs = w.block_size
    per = -(-(N + 1) // bs)
    nblk = B * per + spare_blocks
    ids = np.arange(nblk, dtype=np.int64)
    if (w.shuffled_table if shuffled is None else shuffled):
        ids = np.random.default_rng([w.seed, 99]).permutation(nblk)
    table = ids[: B * per].reshape(B, per).astype(np.int32)
    return table, nblk


def slot_mapping(table: np.ndarray, positions: np.ndarray, block_size: int = 16) -> np.ndarray:
    """Slots (page * block_size + offset) of token positions [B][T] under ``table``."""
    positions = np.asarray(positions)
    b = np.arange(table.shape[0])[:, None]
    page = table[b, positions // block_size].astype(np.int64)
    return (page * block_size + positions % block_size).astype(np.int64)


# --------------------------------------------------------- bulk draws: torch
def kv_torch(w: Workload, layer: int, b: int, st: dict, device, context=None, tok0: int = 0,
             ntok=None):
    """Device K/V of all loops for tokens [tok0, tok0+ntok) of sequence b.

    Same recipe as ``kv_numpy``; drawn with a seeded torch generator on the
    device (one generator per (layer, sequence), positioned by token range so
    that any slice can be redrawn on its own). Shape [L][2][T][H][D], storage
    dtype (bfloat16 or float32).
    """
    import torch
    N = w.context if context is None else context
    T = (N + 1 - tok0) if ntok is None else ntok
    H, D, L = w.heads, w.head_dim, w.loops
    dt = torch.bfloat16 if w.kv_dtype == "bf16" else torch.float32
    out = torch.empty((L, 2, T, H, D), dtype=dt, device=device)
    scale = torch.as_tensor(st["scale"], dtype=torch.float32, device=device)  # [2][H][D]
    chunk = 4096
    for c0 in range(0, T, chunk):
        t0 = tok0 + c0
        n = min(chunk, T - c0)
        gen = torch.Generator(device=device)
        gen.manual_seed(int(np.random.SeedSequence([w.seed, layer, b, t0 // chunk]).generate_state(1)[0]))
        ref = torch.randn((2, n, H, D), generator=gen, device=device) * scale[:, None]
        for l in range(L - 1):
            a = torch.as_tensor(st["alpha"][l], dtype=torch.float32, device=device)[:, None, :, None]
            noise = torch.randn((2, n, H, D), generator=gen, device=device)
            out[l, :, c0:c0 + n] = (a * ref + float(st["sigma"][l]) * noise).to(dt)
        out[L - 1, :, c0:c0 + n] = ref.to(dt)
    return out


def queries_torch(w: Workload, layer: int, device, batch=None):
    """Device decode queries [L][B][H][D] in the storage dtype (seeded)."""
    import torch
    B = w.batch if batch is None else batch
    dt = torch.bfloat16 if w.kv_dtype == "bf16" else torch.float32
    gen = torch.Generator(device=device)
    gen.manual_seed(int(np.random.SeedSequence([w.seed, layer, 7]).generate_state(1)[0]))
    q = torch.randn((w.loops, B, w.heads, w.head_dim), generator=gen, device=device)
    return (q / float(np.sqrt(w.head_dim))).to(dt)
