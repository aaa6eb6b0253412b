"""Decode-step benchmark of ResidualQuant attention over a packed INT4/INT2 KV
cache on one MI355X.

One step of the looped model's decode for one layer at the long-context
Ouro-like shape (batch 16, context 32768, 16 heads x 128, 4 loops, 16-token
pages): four decode-attention calls, one per loop, each over that loop's
packed cache plus the current token's uncompressed K/V, then the deferred
compression of the current token (all loops) into the paged pool. Inputs are
seeded synthetic draws resident in HBM before timing starts.

Prints one JSON line (see the keys below). `value` is this per-loop step (the
loops of a looped model run one after another). Also measured: the same step
with the 4 loops' queries in one multi-loop call (each reference page read
once; `multi_loop`), the in-library bf16 baseline step at the same batch
(append the token's 4 loops of bf16 K/V + 4 decode calls), the dominant
kernel's bandwidth against the 8 TB/s HBM peak (HIP events stamped by each
residual-loop split-K dispatch during the timed steps), measured HBM traffic
from committed rocprofv3 counter summaries when they match the kernel source,
and the fp64 oracle timed on the host on a bounded sample.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
DEFAULT_WORKLOAD = "ouro_h16_d128_l4_b16_n32768"


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


class HipEvents:
    """hipEvent_t pairs for timing kernels launched inside the library."""

    # timing-only events: no system-scope fence (cache write-back and
    # invalidate) when they are recorded, which would otherwise stall the
    # stream between the kernels they bracket
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        self.h = ctypes.CDLL("libamdhip64.so")
        self.h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.h.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.h.hipEventSynchronize.argtypes = [ctypes.c_void_p]

    def create(self):
        e = ctypes.c_void_p()
        assert self.h.hipEventCreateWithFlags(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE) == 0
        return e

    def ms(self, a, b):
        assert self.h.hipEventSynchronize(b) == 0
        f = ctypes.c_float()
        assert self.h.hipEventElapsedTime(ctypes.byref(f), a, b) == 0
        return float(f.value)

    def destroy(self, e):
        self.h.hipEventDestroy(e)


def token_head_bytes(w, loop):
    """Algorithmic packed bytes one decode call reads per token-head: the
    reference loop's record share (INT4 codes + scale/zero) for K and V, plus
    for a residual loop its own record share (codes + scale/zero + alpha)."""
    D, G = w.head_dim, w.group_size
    m = 2 if w.meta_dtype == "f16" else 4
    ref = 2 * (D * 4 // 8 + 2 * m * (D // G))
    if loop == w.loops - 1:
        return ref
    b = w.res_bits[loop]
    return ref + 2 * (D * b // 8 + 2 * m * (D // G) + m)


def setup_rq(w, dev, split_pages, split_pages_multi, layer=0, pool_only=False):
    import torch
    import looped_transformer_decode_rq_amd as R
    import workloads as W
    B, N, H, D, L = w.batch, w.context, w.heads, w.head_dim, w.loops
    st = W.structure(w, layer)
    table, nblk = W.block_table(w)
    lay = R.make_layout(H, D, w.group_size, L, w.res_bits, nblk, w.meta_dtype, w.kv_dtype)
    pool = torch.zeros(R.pool_bytes(lay), dtype=torch.uint8, device=dev)
    rot = torch.from_numpy(st["rot32"]).to(dev)
    kvdt = torch.bfloat16 if w.kv_dtype == "bf16" else torch.float32
    cur = torch.empty((L, 2, B, H, D), dtype=kvdt, device=dev)      # current token, all loops
    pos = np.arange(N)
    for b in range(B):
        kvb = W.kv_torch(w, layer, b, st, dev)
        slots = torch.from_numpy(table[b, pos // 16].astype(np.int64) * 16 + pos % 16).to(dev)
        R.encode_pack(lay, pool, kvb[:, :, :N].contiguous(), rot, slots)
        cur[:, :, b] = kvb[:, :, N]
        del kvb
    torch.cuda.synchronize()
    if pool_only:
        return dict(pool=pool, rot=rot, cur=cur)
    q = W.queries_torch(w, layer, dev)
    s = dict(lay=lay, pool=pool, rot=rot, cur=cur, q=q, table=table, nblk=nblk, st=st,
             d_table=torch.from_numpy(table).to(dev), d_seq=torch.full((B,), N, dtype=torch.int32, device=dev),
             slots_new=torch.from_numpy(table[:, N // 16].astype(np.int64) * 16 + N % 16).to(dev))
    s["qs"] = [q[l:l + 1].contiguous() for l in range(L)]
    s["tk"] = [cur[l, 0][None].contiguous() for l in range(L)]
    s["tv"] = [cur[l, 1][None].contiguous() for l in range(L)]
    s["kv_new"] = cur                                                  # [L][2][T=B][H][D]
    s["out"] = torch.empty((L, 1, B, H, D), device=dev)
    s["ws"] = torch.empty(R.decode_workspace_bytes(lay, 1, B, table.shape[1], split_pages), dtype=torch.uint8,
                          device=dev)
    # multi-loop mode: all loops' queries and current tokens in one call
    s["q_all"] = q.contiguous()
    s["tk_all"] = cur[:, 0].contiguous()
    s["tv_all"] = cur[:, 1].contiguous()
    s["out_all"] = torch.empty((L, B, H, D), device=dev)
    s["ws_all"] = torch.empty(R.decode_workspace_bytes(lay, L, B, table.shape[1], split_pages_multi),
                              dtype=torch.uint8, device=dev)
    return s


def rq_step(w, s, split_pages, events=None, fused=True, pool=None):
    """One decode step: the loops' attention calls in order; the new tokens'
    compression rides in the reference-loop call (fused) or follows it."""
    import looped_transformer_decode_rq_amd as R
    tau = 1.0 / np.sqrt(w.head_dim)
    ref = w.loops - 1
    # pool: one packed cache for every call, or a list with one per loop call
    pools = pool if isinstance(pool, list) else [s["pool"] if pool is None else pool] * w.loops
    for l in range(w.loops):
        ev = None if events is None else events[l]
        enc = dict(kv_new=s["kv_new"], slot_mapping=s["slots_new"]) if fused and l == ref else {}
        R.decode_attention(s["lay"], pools[l], [l], s["qs"][l], s["rot"], s["d_table"], s["d_seq"],
                           s["tk"][l], s["tv"][l], tau, s["out"][l], s["ws"], split_pages=split_pages, events=ev,
                           **enc)
    if not fused:
        R.encode_pack(s["lay"], pools[ref], s["kv_new"], s["rot"], s["slots_new"])


def rq_multi_step(w, s, split_pages, events=None, fused=True, pool=None):
    import looped_transformer_decode_rq_amd as R
    tau = 1.0 / np.sqrt(w.head_dim)
    pool = s["pool"] if pool is None else pool
    enc = dict(kv_new=s["kv_new"], slot_mapping=s["slots_new"]) if fused else {}
    R.decode_attention(s["lay"], pool, list(range(w.loops)), s["q_all"], s["rot"], s["d_table"], s["d_seq"],
                       s["tk_all"], s["tv_all"], tau, s["out_all"], s["ws_all"], split_pages=split_pages,
                       events=events, **enc)
    if not fused:
        R.encode_pack(s["lay"], pool, s["kv_new"], s["rot"], s["slots_new"])


def setup_chunk(w, dev, rq, C):
    """A prefill chunk of C new tokens per sequence after the cached context:
    their queries and K/V of every loop (seeded, same recipe as the cache)."""
    import torch
    import looped_transformer_decode_rq_amd as R
    import workloads as W
    B, N, H, D, L = w.batch, w.context, w.heads, w.head_dim, w.loops
    ck = torch.empty((L, B, C, H, D), dtype=torch.bfloat16, device=dev)
    cv = torch.empty_like(ck)
    for b in range(B):
        kv = W.kv_torch(w, 0, b, rq["st"], dev, tok0=N, ntok=C)          # [L][2][C][H][D]
        ck[:, b] = kv[:, 0]
        cv[:, b] = kv[:, 1]
    gen = torch.Generator(device=dev)
    gen.manual_seed(int(np.random.SeedSequence([w.seed, 0, 11]).generate_state(1)[0]))
    q = (torch.randn((L, B, C, H, D), generator=gen, device=dev) / float(np.sqrt(D))).to(torch.bfloat16)
    ws = torch.empty(R.chunk_workspace_bytes(rq["lay"], C, B, rq["table"].shape[1]), dtype=torch.uint8, device=dev)
    return dict(C=C, q=q, ck=ck, cv=cv, out=torch.empty((L, B, C, H, D), device=dev), ws=ws)


def chunk_step(w, rq, ch, events=None):
    """One chunked-prefill step: every loop's chunk over that loop's packed
    cache plus the chunk itself (causal)."""
    import looped_transformer_decode_rq_amd as R
    tau = 1.0 / np.sqrt(w.head_dim)
    for l in range(w.loops):
        R.chunk_attention(rq["lay"], rq["pool"], l, ch["q"][l], rq["rot"], rq["d_table"], rq["d_seq"], ch["ck"][l],
                          ch["cv"][l], tau, ch["out"][l], ch["ws"], events=None if events is None else events[l])



QUERY_RECORD = lambda D: 64 + 11 * D // 2        # per (call, sequence, head): header + 6 + 5 limb planes


def split_kernel_bytes(w, loop, nparts):
    """Algorithmic bytes of one per-loop split-K launch: the packed records of
    every cached token-head, the query records, the block table and the
    workgroup partials written."""
    B, N, H, D = w.batch, w.context, w.heads, w.head_dim
    res = loop != w.loops - 1
    return (token_head_bytes(w, loop) * B * H * N + B * H * QUERY_RECORD(D) + B * (-(-N // 16)) * 4
            + B * H * nparts * (2 + (2 * D if res else D)) * 4)


def workload_leg(w, dev, steps, warmup, ev, copies):
    """One layer of workload w: the per-loop step (one decode call per loop,
    the new tokens' compression in the reference-loop launch), the multi-loop
    step and the bf16 baseline step at the same batch. `copies` identical
    packed layers are used in turn, call by call, so that no call finds the
    records it reads in the 256 MB last-level cache (these layers are small:
    a loop call reads 0.3-0.6 GB)."""
    import torch
    import looped_transformer_decode_rq_amd as R
    B, N, H, D, L = w.batch, w.context, w.heads, w.head_dim, w.loops
    table_w = -(-(N + 1) // 16)
    probe = R.make_layout(H, D, w.group_size, L, w.res_bits, 1, w.meta_dtype, w.kv_dtype)
    sp_loop = R.decode_auto_split_pages(probe, 1, B, table_w)
    sp_multi = R.decode_auto_split_pages(probe, L, B, table_w)
    sp_bf16 = R.bf16_auto_split_pages(H, B, table_w)
    log(f"workload {w.name}: setting up {copies} packed layers")
    rq = setup_rq(w, dev, sp_loop, sp_multi)
    pools = [rq["pool"]] + [rq["pool"].clone() for _ in range(copies - 1)]
    turn = [0]

    def next_pools(n):
        out = [pools[(turn[0] + i) % copies] for i in range(n)]
        turn[0] += n
        return out

    pairs = {(k, l): (ev.create(), ev.create()) for k in range(steps) for l in range(L)}
    t_rq = timed(lambda k: rq_step(w, rq, sp_loop, None if k is None else [pairs[(k, l)] for l in range(L)],
                                   pool=next_pools(L)), steps, warmup)
    kms = {l: [] for l in range(L)}
    for (k, l), (a, b) in pairs.items():
        kms[l].append(ev.ms(a, b))
        ev.destroy(a)
        ev.destroy(b)
    mpairs = {k: (ev.create(), ev.create()) for k in range(steps)}
    t_multi = timed(lambda k: rq_multi_step(w, rq, sp_multi, None if k is None else mpairs[k],
                                            pool=next_pools(1)[0]), steps, warmup)
    mms = []
    for k, (a, b) in mpairs.items():
        mms.append(ev.ms(a, b))
        ev.destroy(a)
        ev.destroy(b)
    nwg = -(-table_w // (4 * sp_loop))
    per_loop = []
    for l in range(L):
        ms = float(np.mean(kms[l]))
        by = split_kernel_bytes(w, l, nwg)
        per_loop.append({"loop": l, "bits": 4 if l == L - 1 else int(w.res_bits[l]), "kernel_ms": ms,
                         "bytes_per_launch": by, "gbs": by / (ms * 1e-3) / 1e9,
                         "frac_of_peak": by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS})
    # the dominant kernel: the one with the most time per step (summed over its loops)
    groups = {}
    for r in per_loop:
        key = "reference" if r["loop"] == L - 1 else f"int{r['bits']} residual"
        groups.setdefault(key, []).append(r)
    dom_key = max(groups, key=lambda k: sum(r["kernel_ms"] for r in groups[k]))
    dom = groups[dom_key]
    dom_ms = float(np.mean([r["kernel_ms"] for r in dom]))
    dom_bytes = float(np.mean([r["bytes_per_launch"] for r in dom]))
    stored = token_head_bytes(w, L - 1) + sum(token_head_bytes(w, l) - token_head_bytes(w, L - 1)
                                              for l in range(L - 1))
    nsplit = -(-table_w // sp_multi)
    multi_bytes = (stored * B * H * N + L * B * H * QUERY_RECORD(D) + B * table_w * 4
                   + (L - 1) * B * H * nsplit * (2 + 2 * D) * 4 + B * H * nsplit * (2 + D) * 4)
    out = {"workload": w.name, "batch": B, "context": N, "heads": H, "head_dim": D, "loops": L,
           "res_bits": list(w.res_bits), "group_size": w.group_size,
           "packed_layers_in_turn": copies,
           "per_loop_step": {"ms": t_rq * 1e3, "tokens_per_s": B / t_rq},
           "multi_loop_step": {"ms": t_multi * 1e3, "tokens_per_s": B / t_multi, "kernel_ms": float(np.mean(mms)),
                               "kernel_gbs": multi_bytes / (float(np.mean(mms)) * 1e-3) / 1e9},
           "split_kernels": per_loop,
           "roofline": {"bound": "hbm", "kernel": f"rq_split_kernel ({dom_key} loops)", "kernel_ms": dom_ms,
                        "bytes_per_launch": dom_bytes, "achieved": dom_bytes / (dom_ms * 1e-3) / 1e9,
                        "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": dom_bytes / (dom_ms * 1e-3) / 1e9 / HBM_PEAK_GBS}}
    out["multi_loop_step"]["kernel_frac_of_peak"] = out["multi_loop_step"]["kernel_gbs"] / HBM_PEAK_GBS
    log(f"{w.name}: per-loop step {t_rq * 1e3:.3f} ms, multi-loop step {t_multi * 1e3:.3f} ms; "
        f"{dom_key} split kernel {dom_ms:.3f} ms ({out['roofline']['frac']:.3f} of peak)")
    del pools, rq["pool"]
    b16 = setup_bf16(w, dev, rq, sp_bf16)
    t_bf = timed(lambda k: bf16_step(w, rq, b16, sp_bf16), steps, warmup)
    out["bf16_step"] = {"ms": t_bf * 1e3, "tokens_per_s": B / t_bf}
    out["speedup_per_loop_vs_bf16"] = t_bf / t_rq
    out["speedup_multi_loop_vs_bf16"] = t_bf / t_multi
    log(f"{w.name}: bf16 step {t_bf * 1e3:.3f} ms; per-loop {t_bf / t_rq:.2f}x, multi-loop {t_bf / t_multi:.2f}x")
    del b16, rq
    torch.cuda.empty_cache()
    return out


def peak_batch_leg(w, dev, steps, warmup):
    """The 24-layer peak-batch decode step: every layer's packed pool resident
    (generated layer by layer from the workload recipe), timed as the KV path
    of a full model step (per layer: one decode call per loop with the new
    tokens' compression in the reference-loop launch; also the multi-loop
    form); then the bf16 baseline at the largest batch whose 24 layers of
    bf16 cache fit in the memory left, timed the same way."""
    import torch
    import looped_transformer_decode_rq_amd as R
    import workloads as W
    B, N, H, D, L, NL = w.batch, w.context, w.heads, w.head_dim, w.loops, w.layers
    table_w = -(-(N + 1) // 16)
    probe = R.make_layout(H, D, w.group_size, L, w.res_bits, 1, w.meta_dtype, w.kv_dtype)
    sp_loop = R.decode_auto_split_pages(probe, 1, B, table_w)
    sp_multi = R.decode_auto_split_pages(probe, L, B, table_w)
    t0 = time.perf_counter()
    base = setup_rq(w, dev, sp_loop, sp_multi, layer=0)
    layers = [dict(pool=base["pool"], rot=base["rot"], cur=base["cur"])]
    for layer in range(1, NL):
        layers.append(setup_rq(w, dev, sp_loop, sp_multi, layer=layer, pool_only=True))
        log(f"{w.name}: {layer + 1} of {NL} layers packed")
    torch.cuda.synchronize()
    packed_bytes = sum(int(x["pool"].numel()) for x in layers)
    log(f"{w.name}: {NL} packed layers resident, {packed_bytes / 1e9:.1f} GB ({time.perf_counter() - t0:.0f} s)")
    tau = 1.0 / np.sqrt(D)

    def rq_full(k, multi):
        for x in layers:
            s = dict(base, pool=x["pool"], rot=x["rot"], kv_new=x["cur"])
            if multi:
                rq_multi_step(w, s, sp_multi)
            else:
                rq_step(w, s, sp_loop)

    t_rq = timed(lambda k: rq_full(k, False), steps, warmup)
    t_multi = timed(lambda k: rq_full(k, True), steps, warmup)
    step_bytes = NL * sum(token_head_bytes(w, l) for l in range(L)) * B * H * N
    out = {"workload": w.name, "layers": NL, "batch": B, "context": N, "packed_bytes_resident": packed_bytes,
           "per_loop_step": {"ms": t_rq * 1e3, "tokens_per_s": B / t_rq,
                             "effective_gbs": step_bytes / t_rq / 1e9},
           "multi_loop_step": {"ms": t_multi * 1e3, "tokens_per_s": B / t_multi},
           "step": f"{NL} layers x ({L} per-loop decode calls + compression of {B} new tokens); "
                   "the KV path only (no projections or MLP: no model weights)"}
    log(f"{w.name}: packed {NL}-layer step {t_rq * 1e3:.2f} ms per-loop, {t_multi * 1e3:.2f} ms multi-loop")
    del layers, base
    torch.cuda.empty_cache()
    # bf16 baseline: 24 layers x L loops x K|V caches of [pages][H][16][D] bf16
    per_seq = NL * L * 2 * table_w * 16 * H * D * 2
    free, total = torch.cuda.mem_get_info()
    reserve = 6 << 30
    bmax = int(min(B, (free - reserve) // per_seq))
    out["rq_largest_batch_that_fits"] = int((total - reserve) // (NL * table_w * H * int(
        R.pool_bytes(probe) // H)))
    out["bf16_bytes_per_sequence_all_layers"] = per_seq
    if bmax < 1:
        out["bf16_baseline"] = {"error": "no bf16 batch fits"}
        return out
    wb = w.replace(batch=bmax)
    table, nblk = W.block_table(wb)
    d_table = torch.from_numpy(table).to(dev)
    d_seq = torch.full((bmax,), N, dtype=torch.int32, device=dev)
    sp_bf16 = R.bf16_auto_split_pages(H, bmax, table_w)
    ws = torch.empty(R.bf16_workspace_bytes(H, D, bmax, table_w, sp_bf16), dtype=torch.uint8, device=dev)
    t0 = time.perf_counter()
    caches = []
    pos = np.arange(N)
    for layer in range(NL):
        st = W.structure(w, layer)
        kc = [torch.empty((nblk, H, 16, D), dtype=torch.bfloat16, device=dev) for _ in range(L)]
        vc = [torch.empty_like(kc[0]) for _ in range(L)]
        cur = torch.empty((L, 2, bmax, H, D), dtype=torch.bfloat16, device=dev)
        for b in range(bmax):
            kvb = W.kv_torch(wb, layer, b, st, dev)
            slots = torch.from_numpy(table[b, pos // 16].astype(np.int64) * 16 + pos % 16).to(dev)
            for l in range(L):
                R.bf16_write(kc[l], vc[l], kvb[l, :, :N].contiguous(), slots)
            cur[:, :, b] = kvb[:, :, N]
            del kvb
        caches.append((kc, vc, cur))
        log(f"{w.name}: bf16 layer {layer + 1} of {NL} written")
    torch.cuda.synchronize()
    log(f"{w.name}: bf16 caches of {NL} layers at batch {bmax} resident, "
        f"{bmax * per_seq / 1e9:.1f} GB ({time.perf_counter() - t0:.0f} s)")
    q = W.queries_torch(wb, 0, dev)
    qs = [q[l].contiguous() for l in range(L)]
    outb = torch.empty((bmax, H, D), device=dev)
    slots_new = torch.from_numpy(table[:, N // 16].astype(np.int64) * 16 + N % 16).to(dev)
    tails = [[(c[2][l, 0].contiguous(), c[2][l, 1].contiguous(), c[2][l].contiguous()) for l in range(L)]
             for c in caches]

    def bf_full(k):
        for (kc, vc, _), tl in zip(caches, tails):
            for l in range(L):
                R.bf16_decode_attention(kc[l], vc[l], qs[l], d_table, d_seq, tl[l][0], tl[l][1], tau, outb, ws,
                                        split_pages=sp_bf16)
                R.bf16_write(kc[l], vc[l], tl[l][2], slots_new)

    t_bf = timed(bf_full, steps, warmup)
    out["bf16_baseline"] = {"batch": bmax, "ms_per_step": t_bf * 1e3, "tokens_per_s": bmax / t_bf,
                            "cache_bytes_resident": bmax * per_seq}
    out["peak_throughput_ratio_per_loop"] = (B / t_rq) / (bmax / t_bf)
    out["peak_throughput_ratio_multi_loop"] = (B / t_multi) / (bmax / t_bf)
    log(f"{w.name}: bf16 {NL}-layer step at batch {bmax}: {t_bf * 1e3:.2f} ms; peak-throughput ratio "
        f"{out['peak_throughput_ratio_per_loop']:.2f}x per-loop, {out['peak_throughput_ratio_multi_loop']:.2f}x multi-loop")
    del caches, tails
    torch.cuda.empty_cache()
    return out


def direct_baseline(w, dev, rq, bits, split_pages, steps, warmup):
    """The direct per-loop quantization baseline on the same synthetic K/V:
    every loop quantized on its own at `bits[l]` (no reference, alpha or
    rotation). Times the same step (one decode call per loop + compression of
    the new tokens) and returns its outputs for the error comparison."""
    import torch
    import looped_transformer_decode_rq_amd as R
    import workloads as W
    B, N, H, D, L = w.batch, w.context, w.heads, w.head_dim, w.loops
    table, nblk = rq["table"], rq["nblk"]
    lay = R.make_layout(H, D, w.group_size, L, bits, nblk, w.meta_dtype, w.kv_dtype, mode=R.RQ_MODE_DIRECT)
    pool = torch.zeros(R.pool_bytes(lay), dtype=torch.uint8, device=dev)
    pos = np.arange(N)
    for b in range(B):
        kvb = W.kv_torch(w, 0, b, rq["st"], dev)
        slots = torch.from_numpy(table[b, pos // 16].astype(np.int64) * 16 + pos % 16).to(dev)
        R.encode_pack(lay, pool, kvb[:, :, :N].contiguous(), None, slots)
        del kvb
    out = torch.empty((L, 1, B, H, D), device=dev)
    ws = torch.empty(R.decode_workspace_bytes(lay, 1, B, table.shape[1], split_pages), dtype=torch.uint8,
                     device=dev)
    tau = 1.0 / np.sqrt(D)

    def step(k):
        for l in range(L):
            R.decode_attention(lay, pool, [l], rq["qs"][l], None, rq["d_table"], rq["d_seq"], rq["tk"][l],
                               rq["tv"][l], tau, out[l], ws, split_pages=split_pages)
        R.encode_pack(lay, pool, rq["kv_new"], None, rq["slots_new"])

    t = timed(step, steps, warmup)
    stored = sum(2 * (D * b // 8 + 2 * (2 if w.meta_dtype == "f16" else 4) * (D // w.group_size)) for b in bits)
    res = {"bits": list(bits), "ms_per_step": t * 1e3, "tokens_per_s": B / t,
           "stored_bytes_per_token_head": stored}
    del pool
    return res, out[:, 0].clone()


def rel_l2(a, b):
    return float((a.double() - b.double()).norm() / b.double().norm())


def setup_bf16(w, dev, rq, split_pages):
    import torch
    import looped_transformer_decode_rq_amd as R
    import workloads as W
    B, N, H, D, L = w.batch, w.context, w.heads, w.head_dim, w.loops
    table, nblk = rq["table"], rq["nblk"]
    kc = [torch.zeros((nblk, H, 16, D), dtype=torch.bfloat16, device=dev) for _ in range(L)]
    vc = [torch.zeros_like(kc[0]) for _ in range(L)]
    pos = np.arange(N)
    for b in range(B):
        kvb = W.kv_torch(w, 0, b, rq["st"], dev)
        slots = torch.from_numpy(table[b, pos // 16].astype(np.int64) * 16 + pos % 16).to(dev)
        for l in range(L):
            R.bf16_write(kc[l], vc[l], kvb[l, :, :N].contiguous(), slots)
        del kvb
    torch.cuda.synchronize()
    return dict(kc=kc, vc=vc, out=torch.empty((B, H, D), device=dev),
                ws=torch.empty(R.bf16_workspace_bytes(H, D, B, table.shape[1], split_pages), dtype=torch.uint8,
                               device=dev),
                q=[rq["q"][l].contiguous() for l in range(L)],
                new=[rq["cur"][l].contiguous() for l in range(L)])


def bf16_step(w, rq, b, split_pages, events=None):
    import looped_transformer_decode_rq_amd as R
    tau = 1.0 / np.sqrt(w.head_dim)
    for l in range(w.loops):
        R.bf16_decode_attention(b["kc"][l], b["vc"][l], b["q"][l], rq["d_table"], rq["d_seq"],
                                rq["tk"][l][0], rq["tv"][l][0], tau, b["out"], b["ws"], split_pages=split_pages,
                                events=None if events is None else events[l])
        R.bf16_write(b["kc"][l], b["vc"][l], b["new"][l], rq["slots_new"])


SETTLE_S = 0.1          # minimum untimed run of a leg's step before its timed steps
SETTLE_MAX_S = 1.0      # at most this long: then the clocks are taken as settled
SETTLE_BATCH = 5        # steps per settle batch
SETTLE_TOL = 0.01       # settled: two batches in a row within 1% of each other


def timed(fn, steps, warmup):
    """Seconds per step over `steps` timed steps. The GPU's clocks ramp up
    over the first ~40 ms of sustained load after an idle spell (measured on
    MI355X: a per-loop step of the benchmark layer takes ~2.0 ms cold, 1.19 ms
    10 ms later, ~1.15 ms from ~40 ms on; on some boxes the ramp takes
    longer), so each leg first runs its step untimed for at least SETTLE_S
    seconds and until two consecutive batches of SETTLE_BATCH steps agree
    within SETTLE_TOL (at most SETTLE_MAX_S), then the `warmup` steps, then
    the timed ones, all back to back."""
    import torch
    t_start = time.perf_counter()
    prev = None
    nb = 0
    while True:
        t0 = time.perf_counter()
        for _ in range(SETTLE_BATCH):
            fn(None)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        cur = t1 - t0
        settled = prev is not None and abs(cur - prev) <= SETTLE_TOL * prev
        prev = cur
        nb += 1
        if t1 - t_start >= SETTLE_MAX_S or (settled and t1 - t_start >= SETTLE_S):
            log(f"settle: {nb} batches in {t1 - t_start:.2f} s, last batch {cur / SETTLE_BATCH * 1e3:.3f} ms per step")
            break
    for _ in range(warmup):
        fn(None)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        fn(k)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def graph_leg(w, rq, split_pages, layers, steps, warmup):
    """The per-loop step of `layers` layers captured in one HIP graph and
    replayed. Every layer's calls go to the one packed cache (each call streams
    its full records, far beyond any cache), so the replay times the same work
    as `layers` distinct layers."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(layers):
            rq_step(w, rq, split_pages)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(layers):
            rq_step(w, rq, split_pages)
    torch.cuda.synchronize()
    t = timed(lambda k: g.replay(), steps, warmup)
    del g
    return {"layers": layers, "ms_per_replay": t * 1e3, "ms_per_layer_step": t * 1e3 / layers,
            "tokens_per_s_one_layer": w.batch / (t / layers),
            "step": f"{layers} layers x (4 per-loop decode calls + encode of {w.batch} new tokens), one graph"}


def _oracle_unit(task):
    """One (sequence, head) unit of a workload's decode step in the fp64
    oracle, in a worker process: draw the unit's K/V and query with the
    workload's recipe (batch 1, one head, the unit's own seed), pack its
    cache with the oracle encoder (not timed: the cache exists before the
    step), then time the oracle's decode attention of every loop over it."""
    import oracle as O
    import workloads as W
    name, seed = task
    w = W.get(name).replace(batch=1, heads=1, seed=seed)
    N, D, L = w.context, w.head_dim, w.loops
    st = W.structure(w)
    kv = W.kv_numpy(w, st=st)                                   # [L][2][1][N+1][1][D]
    q = W.queries_numpy(w)                                      # [L][1][1][D]
    npages = -(-N // 16)
    lay = O.PoolLayout(1, D, w.group_size, L, w.res_bits, w.meta_dtype, npages)
    enc = O.encode(kv[:, :, 0, :N], st["rot32"], w.res_bits, w.group_size, w.meta_dtype)
    pool = np.zeros(lay.pool_bytes, np.uint8)
    O.write_tokens(pool, lay, enc, np.arange(N))
    tau = 1.0 / np.sqrt(D)
    t0 = time.perf_counter()
    for l in range(L):
        O.decode_attention(pool, lay, l, q[l], st["rot32"], np.arange(npages)[None], [N], tau,
                           kv[l, 0, :, N], kv[l, 1, :, N])
    return time.perf_counter() - t0


def start_oracle_pools():
    """Spawn-started worker pools for the oracle timing, created before this
    process touches the GPU (the workers are fresh interpreters that never do):
    one single-threaded worker per core of this process's CPU share (at most
    16), and one more single worker for the 1-core figure."""
    import multiprocessing as mp
    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    saved = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    for k in saved:
        os.environ[k] = "1"
    try:
        ctx = mp.get_context("spawn")
        return cores, ctx.Pool(cores), ctx.Pool(1)
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def _oracle_encode_step(w):
    """Oracle time of one step's compression: every sequence's new token, all
    loops and heads (one vectorized encode)."""
    import oracle as O
    import workloads as W
    st = W.structure(w)
    kv = W.kv_numpy(w.replace(context=0), st=st)[:, :, :, 0]     # [L][2][B][H][D]: one token per sequence
    t0 = time.perf_counter()
    O.encode(kv, st["rot32"], w.res_bits, w.group_size, w.meta_dtype)
    return time.perf_counter() - t0


def cpu_baseline(w, pools, budget_s=12.0):
    """The fp64 oracle timed on the host's cores.

    The decode step's (sequence, head) units are independent: they run in a
    pool of single-threaded worker processes, one per core of this process's
    CPU share. For the benchmark workload, waves of one unit per worker run
    until the time budget is spent and the step time is extrapolated from the
    mean unit time; the tiny and the Ouro-like 4096-token workloads run in
    full; the Huginn-like layer and the 24-layer cache time one unit per
    worker and are extrapolated to their full step (all layers' units and
    encodes). A single worker gives the 1-core figure."""
    import workloads as W
    cores, pool, pool1 = pools
    B, H = w.batch, w.heads
    out = {"unit": "tokens/s", "cores": cores, "kind": "oracle", "threads_per_core": 1}
    t_enc = _oracle_encode_step(w)
    times = []
    t0 = time.perf_counter()
    seed = 1000
    while len(times) < B * H and (not times or time.perf_counter() - t0 < budget_s):
        n = min(cores, B * H - len(times))
        times += pool.map(_oracle_unit, [(w.name, seed + i) for i in range(n)])
        seed += n
    step = B * H * float(np.mean(times)) / cores + t_enc
    out["value"] = B / step
    out["sample"] = (f"{len(times)} of {B * H} (sequence, head) units of {w.name} (each drawn with the workload's "
                     f"recipe under its own seed; fp64 decode attention of all {w.loops} loops over its "
                     f"{w.context} packed tokens) on {cores} single-threaded worker processes, plus the fp64 "
                     f"encode of one step's {B} new tokens; step time {step:.1f} s extrapolated to all units")
    one = pool1.map(_oracle_unit, [(w.name, 7)])
    step1 = B * H * float(np.mean(one)) + t_enc
    out["one_core"] = {"value": B / step1, "ms_per_step": step1 * 1e3,
                       "sample": f"1 unit on one single-threaded worker, extrapolated to {B * H} units"}
    full = {}
    for key in (0, 1):
        wf = W.get(key)
        te = _oracle_encode_step(wf)
        t0 = time.perf_counter()
        ut = pool.map(_oracle_unit, [(wf.name, 2000 + i) for i in range(wf.batch * wf.heads)])
        wall = time.perf_counter() - t0
        full[wf.name] = {"units": len(ut), "decode_s_sum": float(np.sum(ut)), "wall_s_with_packing": wall,
                         "step_s_on_cores": float(np.sum(ut)) / cores + te,
                         "tokens_per_s": wf.batch / (float(np.sum(ut)) / cores + te)}
    out["full_workloads"] = full
    # the Huginn-like layer and the 24-layer cache: one wave of units per worker, extrapolated
    sampled = {}
    for key in (3, 4):
        ws = W.get(key)
        layers = getattr(ws, "layers", 1)
        te = _oracle_encode_step(ws)
        ut = pool.map(_oracle_unit, [(ws.name, 3000 + i) for i in range(cores)])
        units = layers * ws.batch * ws.heads
        st = units * float(np.mean(ut)) / cores + layers * te
        sampled[ws.name] = {"units_timed": len(ut), "units_per_step": units, "layers": layers,
                            "step_s_on_cores": st, "tokens_per_s": ws.batch / st, "extrapolated": True}
    out["sampled_workloads"] = sampled
    return out


def traffic_from_profiles(kernel_src_hash):
    """HBM bytes per launch of the decode kernels (residual loop, reference
    loop, multi-loop) from committed rocprofv3 counter summaries, valid only
    for the kernel source they were taken on (else None)."""
    p = os.path.join(ROOT, "profiles", "split_kernel_traffic.json")
    try:
        d = json.load(open(p))
    except Exception:
        return None
    if d.get("kernel_src_sha256") != kernel_src_hash:
        return None
    return d


def kernel_src_hash(files=("rq_decode.hip", "rq_device.h", "rq_internal.h", "rq_vmfma.h")):
    """sha256 of the kernel sources' code: comments and blank lines are left
    out, so that a comment edit does not void the counter summaries taken on
    the same code."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in files:
        src = open(os.path.join(ROOT, "looped_transformer_decode_rq_amd", "csrc", f)).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        src = re.sub(r"//[^\n]*", "", src)
        code = "\n".join(line.rstrip() for line in src.splitlines() if line.strip())
        h.update(code.encode())
    return h.hexdigest()


def chunk_src_hash():
    return kernel_src_hash(("rq_chunk.hip", "rq_device.h", "rq_internal.h", "rq_vmfma.h"))


def chunk_traffic_from_profiles():
    """HBM bytes per launch of the residual-loop chunked-prefill split kernel
    from the committed counter summary, valid only for the chunk kernel source
    it was taken on (else None)."""
    try:
        d = json.load(open(os.path.join(ROOT, "profiles", "split_kernel_traffic.json")))
    except Exception:
        return None
    if d.get("chunk_src_sha256") != chunk_src_hash():
        return None
    return d.get("chunk_residual", {}).get("hbm_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--split-pages", type=int, default=0)
    ap.add_argument("--no-bf16", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-direct", action="store_true", help="skip the direct per-loop quantization baselines")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the per-layer legs of the 4096-token Ouro-like and the Huginn-like workloads")
    ap.add_argument("--no-peak-batch", action="store_true",
                    help="skip the 24-layer peak-batch leg (146.6 GB of packed cache resident)")
    ap.add_argument("--chunk", type=int, default=64,
                    help="queries per sequence of the chunked-prefill leg (0 skips it)")
    ap.add_argument("--graph-layers", type=int, default=4,
                    help="layers of the per-loop step captured in one HIP graph for the graph leg (0 skips it)")
    ap.add_argument("--separate-encode", action="store_true",
                    help="compress the new tokens in a launch of their own after the attention calls "
                         "instead of in the reference-loop call's launch")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after setup, copy a buffer of this many MiB device to device (a plain copy of known "
                         "size, used to calibrate HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this path has no multi-GPU mode (asked for --gpus {args.gpus}); "
              "run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    # the oracle's worker processes start before anything touches the GPU
    pools = None if args.no_cpu else start_oracle_pools()

    import torch
    import looped_transformer_decode_rq_amd as R
    import workloads as W
    R.lib()
    w = W.get(args.workload)
    dev = torch.device("cuda:0")
    B, N, H, D, L = w.batch, w.context, w.heads, w.head_dim, w.loops
    table_w = -(-(N + 1) // 16)
    # pages per split: the library's own choice for each mode unless forced
    probe = R.make_layout(H, D, w.group_size, L, w.res_bits, 1, w.meta_dtype, w.kv_dtype)
    sp_loop = args.split_pages or R.decode_auto_split_pages(probe, 1, B, table_w)
    sp_multi = args.split_pages or R.decode_auto_split_pages(probe, L, B, table_w)
    sp_bf16 = args.split_pages or R.bf16_auto_split_pages(H, B, table_w)
    log(f"workload {w.name}: setting up packed cache (split pages: per-loop {sp_loop}, multi-loop {sp_multi}, "
        f"bf16 {sp_bf16})")
    rq = setup_rq(w, dev, sp_loop, sp_multi)
    if args.copy_probe_mib:
        src = torch.empty(args.copy_probe_mib << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    ev = HipEvents()
    res_loops = [l for l in range(L) if l != L - 1]
    pairs = {(k, l): (ev.create(), ev.create()) for k in range(args.steps) for l in range(L)}

    def rq_fn(k):
        rq_step(w, rq, sp_loop, None if k is None else [pairs[(k, l)] for l in range(L)],
                fused=not args.separate_encode)

    log("timing packed step")
    t_rq = timed(rq_fn, args.steps, args.warmup)
    split_ms = {l: [] for l in range(L)}
    for (k, l), (a, b) in pairs.items():
        split_ms[l].append(ev.ms(a, b))
        ev.destroy(a)
        ev.destroy(b)
    res_ms = float(np.mean([m for l in res_loops for m in split_ms[l]]))
    ref_ms = float(np.mean(split_ms[L - 1]))
    nwg = -(-rq["table"].shape[1] // (4 * sp_loop))     # one partial per 4-wave split workgroup
    nsplit = -(-rq["table"].shape[1] // sp_multi)       # multi-loop: one partial per split and loop
    qp = QUERY_RECORD(D)
    res_bytes = split_kernel_bytes(w, 0, nwg)
    ref_bytes = split_kernel_bytes(w, L - 1, nwg)
    achieved = res_bytes / (res_ms * 1e-3) / 1e9
    # whole step: packed reads of the 4 calls + q/out/tails + rotations + encode traffic
    kvsz = 2 if w.kv_dtype == "bf16" else 4
    step_bytes = sum(token_head_bytes(w, l) * B * H * N for l in range(L))
    step_bytes += L * B * H * D * (kvsz * 3 + 4) + L * H * 2 * D * D * 4
    ref_share = token_head_bytes(w, L - 1)
    stored = ref_share + sum(token_head_bytes(w, l) - ref_share for l in range(L - 1))
    step_bytes += L * 2 * B * H * D * kvsz + B * H * stored          # encode: read new K/V, write records
    step_gbs = step_bytes / t_rq / 1e9
    log(f"packed step {t_rq * 1e3:.3f} ms; residual split kernel {res_ms:.3f} ms ({achieved:.0f} GB/s)")

    # the streaming reference of the per-loop split kernel: the same grid, ring
    # and loads over the same page records, no attention arithmetic
    stream_ref = {}
    for key, l in (("residual", 0), ("reference", L - 1)):
        sp_ev = [(ev.create(), ev.create()) for _ in range(args.steps)]

        def probe_fn(k, l=l, sp_ev=sp_ev):
            R.decode_stream_probe(rq["lay"], rq["pool"], l, rq["d_table"], rq["d_seq"], rq["ws"],
                                  split_pages=sp_loop, events=None if k is None else sp_ev[k])

        timed(probe_fn, args.steps, args.warmup)
        pms = float(np.mean([ev.ms(a, b) for a, b in sp_ev]))
        for a, b in sp_ev:
            ev.destroy(a)
            ev.destroy(b)
        pbytes = token_head_bytes(w, l) * B * H * N + B * (-(-N // 16)) * 4
        stream_ref[key] = {"kernel_ms": pms, "bytes_per_launch": pbytes, "gbs": pbytes / (pms * 1e-3) / 1e9,
                           "frac_of_peak": pbytes / (pms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    stream_ref["split_kernel_frac_of_reference"] = {
        "residual": (res_bytes / (res_ms * 1e-3) / 1e9) / stream_ref["residual"]["gbs"],
        "reference": (ref_bytes / (ref_ms * 1e-3) / 1e9) / stream_ref["reference"]["gbs"]}
    # the roof of any access pattern: a plain contiguous read of a 4 GiB buffer
    cbytes = 4 << 30
    cbuf = torch.empty(cbytes, dtype=torch.uint8, device=dev)
    csink = torch.zeros(32 * 256, dtype=torch.int32, device=dev)   # one word per wave
    c_ev = [(ev.create(), ev.create()) for _ in range(args.steps)]

    def cread_fn(k):
        R.read_probe(cbuf, csink, events=None if k is None else c_ev[k])

    timed(cread_fn, args.steps, args.warmup)
    cms = float(np.mean([ev.ms(a, b) for a, b in c_ev]))
    for a, b in c_ev:
        ev.destroy(a)
        ev.destroy(b)
    del cbuf
    c_gbs = cbytes / (cms * 1e-3) / 1e9
    stream_ref["contiguous_read"] = {"kernel_ms": cms, "bytes_per_launch": cbytes, "gbs": c_gbs,
                                     "frac_of_peak": c_gbs / HBM_PEAK_GBS}
    stream_ref["split_kernel_frac_of_contiguous_read"] = {
        "residual": (res_bytes / (res_ms * 1e-3) / 1e9) / c_gbs,
        "reference": (ref_bytes / (ref_ms * 1e-3) / 1e9) / c_gbs}
    log(f"streaming reference (same loads, no arithmetic): residual {stream_ref['residual']['kernel_ms']:.3f} ms "
        f"({stream_ref['residual']['gbs']:.0f} GB/s), reference {stream_ref['reference']['kernel_ms']:.3f} ms "
        f"({stream_ref['reference']['gbs']:.0f} GB/s); contiguous read {c_gbs:.0f} GB/s")

    # multi-loop mode: the same step with the 4 loops' queries in one call
    mpairs = {k: (ev.create(), ev.create()) for k in range(args.steps)}

    def multi_fn(k):
        rq_multi_step(w, rq, sp_multi, None if k is None else mpairs[k], fused=not args.separate_encode)

    log("timing packed multi-loop step")
    t_multi = timed(multi_fn, args.steps, args.warmup)
    mk = []
    for k, (a, b) in mpairs.items():
        mk.append(ev.ms(a, b))
        ev.destroy(a)
        ev.destroy(b)
    multi_ms = float(np.mean(mk))
    multi_bytes = (stored * B * H * N + L * B * H * qp + B * N // 16 * 4
                   + (L - 1) * B * H * nsplit * (2 + 2 * D) * 4 + B * H * nsplit * (2 + D) * 4)
    if not args.separate_encode:                 # the new tokens' encode runs in this launch
        multi_bytes += L * 2 * B * H * D * kvsz + B * H * stored
    multi_gbs = multi_bytes / (multi_ms * 1e-3) / 1e9
    log(f"multi-loop step {t_multi * 1e3:.3f} ms; multi-loop kernel {multi_ms:.3f} ms ({multi_gbs:.0f} GB/s)")

    graph = None
    if args.graph_layers > 0:
        log(f"timing the per-loop step of {args.graph_layers} layers replayed from one HIP graph")
        try:
            graph = graph_leg(w, rq, sp_loop, args.graph_layers, args.steps, args.warmup)
            graph["eager_ms_per_step"] = t_rq * 1e3
            log(f"graph replay {graph['ms_per_layer_step']:.3f} ms per layer step (eager {t_rq * 1e3:.3f} ms)")
        except Exception as e:          # graph capture unavailable: report it and go on
            log(f"graph leg failed: {e}")
            graph = {"error": str(e)[:300]}

    chunked = None
    if args.chunk > 0:
        log(f"timing chunked prefill ({args.chunk} new tokens per sequence and loop)")
        ch = setup_chunk(w, dev, rq, args.chunk)
        cpairs = {k: [(ev.create(), ev.create()) for _ in range(L)] for k in range(args.steps)}

        def ch_fn(k):
            chunk_step(w, rq, ch, None if k is None else cpairs[k])

        t_ch = timed(ch_fn, args.steps, args.warmup)
        cms = {l: [] for l in range(L)}
        for k, evs in cpairs.items():
            for l, (a, b) in enumerate(evs):
                cms[l].append(ev.ms(a, b))
                ev.destroy(a)
                ev.destroy(b)
        ch_res_ms = float(np.mean([m for l in res_loops for m in cms[l]]))
        C = args.chunk
        ch_bytes = token_head_bytes(w, 0) * B * H * N
        # attention-equivalent work: q.k and p.v, 2D flops each per (query, cached token); the packed
        # residual loop does both for the reference and for the rotated residual
        ch_flops = 2 * 2 * 2 * D * B * H * N * C
        chunked = {"chunk": C, "ms_per_step": t_ch * 1e3, "new_tokens_per_s": B * C / t_ch,
                   "step": f"{L} chunked-prefill calls (one per loop): {C} queries per sequence over its "
                           f"{N} packed tokens + the chunk's own bf16 K/V, causal",
                   "residual_split_kernel_ms": ch_res_ms,
                   "residual_split_kernel_gbs": ch_bytes / (ch_res_ms * 1e-3) / 1e9,
                   "residual_split_kernel_tflops": ch_flops / (ch_res_ms * 1e-3) / 1e12,
                   "residual_split_kernel_traffic": (chunk_traffic_from_profiles()
                                                     if w.name == DEFAULT_WORKLOAD and C == 64 else None),
                   "residual_split_kernel_bound": "valu (per query-token score, softmax and weight work; "
                                                  "matrix cores about a quarter busy)",
                   "reference_split_kernel_ms": float(np.mean(cms[L - 1]))}
        log(f"chunked prefill step {t_ch * 1e3:.3f} ms; residual chunk kernel {ch_res_ms:.3f} ms "
            f"({chunked['residual_split_kernel_gbs']:.0f} GB/s packed, {chunked['residual_split_kernel_tflops']:.1f} TFLOP/s)")
        del ch
        torch.cuda.empty_cache()

    direct, direct_outs, errors = {}, {}, {}
    if not args.no_direct:
        for name, bits in (("direct_int2", (2,) * L), ("direct_int4", (4,) * L)):
            log(f"timing the {name} baseline")
            direct[name], direct_outs[name] = direct_baseline(w, dev, rq, bits, args.split_pages, args.steps,
                                                              args.warmup)
            log(f"{name} step {direct[name]['ms_per_step']:.3f} ms")
        torch.cuda.empty_cache()

    bf16 = None
    if not args.no_bf16:
        log("setting up bf16 baseline cache")
        b16 = setup_bf16(w, dev, rq, sp_bf16)
        bpairs = {k: [(ev.create(), ev.create()) for _ in range(L)] for k in range(args.steps)}

        def bf_fn(k):
            bf16_step(w, rq, b16, sp_bf16, None if k is None else bpairs[k])

        t_bf = timed(bf_fn, args.steps, args.warmup)
        bms = []
        for k, evs in bpairs.items():
            for a, b in evs:
                bms.append(ev.ms(a, b))
                ev.destroy(a)
                ev.destroy(b)
        bf_kernel_bytes = 2 * D * 2 * B * H * N
        bf16 = {"tokens_per_s": B / t_bf, "ms_per_step": t_bf * 1e3,
                "split_kernel_ms": float(np.mean(bms)),
                "split_kernel_gbs": bf_kernel_bytes / (float(np.mean(bms)) * 1e-3) / 1e9,
                "speedup_packed_vs_bf16": t_bf / t_rq,
                "speedup_multi_loop_vs_bf16": t_bf / t_multi}
        log(f"bf16 step {t_bf * 1e3:.3f} ms; packed/bf16 speedup {t_bf / t_rq:.2f}x")
        # exact attention over the bf16 cache, per loop: the reference for the error comparison
        tau = 1.0 / np.sqrt(D)
        exact = []
        for l in range(L):
            R.bf16_decode_attention(b16["kc"][l], b16["vc"][l], b16["q"][l], rq["d_table"], rq["d_seq"],
                                    rq["tk"][l][0], rq["tv"][l][0], tau, b16["out"], b16["ws"],
                                    split_pages=sp_bf16)
            exact.append(b16["out"].clone())
        errors["rq_per_loop"] = [rel_l2(rq["out"][l, 0], exact[l]) for l in range(L)]
        errors["rq_multi_loop"] = [rel_l2(rq["out_all"][l], exact[l]) for l in range(L)]
        for key, o in direct_outs.items():
            errors[key] = [rel_l2(o[l], exact[l]) for l in range(L)]
        log("attention rel-L2 vs bf16: " + ", ".join(f"{k} {max(v):.2e}" for k, v in errors.items()))
        del b16
        torch.cuda.empty_cache()

    others = {}
    if not args.no_other_workloads:
        for key, copies in (("ouro_h16_d128_l4_b32_n4096", 3), ("huginn_h55_d96_l8_b8_n8192_mixed", 2)):
            others[key] = workload_leg(W.get(key), dev, args.steps, args.warmup, ev, copies)
    peak = None
    if not args.no_peak_batch:
        peak = peak_batch_leg(W.get("ouro_24layer_h16_d128_l4_b128_n8192"), dev, max(3, args.steps // 4),
                              min(args.warmup, 2))

    cpu = None
    if not args.no_cpu:
        log("timing the fp64 oracle on the host")
        cpu = cpu_baseline(w, pools)
        for p in pools[1:]:
            p.close()
            p.join()

    traffic = traffic_from_profiles(kernel_src_hash()) if w.name == DEFAULT_WORKLOAD else None

    def measured(key):
        return None if traffic is None else traffic.get(key, {}).get("hbm_bytes_per_launch")
    line = {
        "metric": "decode-attn tokens/s + effective HBM GB/s (% of peak) on packed INT4/INT2 KV",
        "value": B / t_rq,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": t_rq * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("int4/int2 codes; scores: exact int32 dot products (v_dot8_i32_i4) of the codes with a "
                  "per-slice fixed-point query (24-bit q, 20-bit q' = R_K q); fp32 softmax; V on f16 matrix cores "
                  "(weights split into fp16 hi+lo, codes exact) with fp32 accumulation; bf16 inputs, fp16 "
                  "metadata, fp32 output"),
        "data": "synthetic (seeded generator; no model weights)",
        "config": {"workload": w.name, "layers": 1, "batch": B, "context": N, "heads": H, "head_dim": D,
                   "loops": L, "group_size": w.group_size, "res_bits": list(w.res_bits), "block_size": 16,
                   "split_pages": {"per_loop": sp_loop, "multi_loop": sp_multi, "bf16": sp_bf16},
                   "step": "4 per-loop decode calls (each + bf16 current token) + encode of 16 new tokens "
                           + ("(own launch)" if args.separate_encode else "(in the reference-loop call's launch)")},
        "effective_hbm_gbs": step_gbs,
        "effective_hbm_frac": step_gbs / HBM_PEAK_GBS,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": measured("residual"),
                     "kernel": f"rq_split_kernel<{D},{w.res_bits[0]},{w.meta_dtype == 'f32'}> (residual loop)",
                     "kernel_ms": res_ms, "bytes_per_launch": res_bytes},
        "stream_reference": stream_ref,
        "ref_loop_kernel": {"ms": ref_ms, "gbs": ref_bytes / (ref_ms * 1e-3) / 1e9, "bytes_per_launch": ref_bytes,
                            "traffic": measured("reference")},
        "multi_loop": {"tokens_per_s": B / t_multi, "ms_per_step": t_multi * 1e3,
                       "note": "needs every loop's query of a layer at once; a looped model produces them one "
                               "after another, so its decode step is the per-loop step (value)",
                       "step": f"one decode call with all {L} loops' queries (each reference page read once) "
                               f"+ encode of {B} new tokens in the same launch",
                       "kernel": f"rq_multi_kernel<{D}> ({L} waves per split workgroup)",
                       "kernel_ms": multi_ms, "bytes_per_launch": multi_bytes, "traffic": measured("multi_loop"),
                       "kernel_gbs": multi_gbs,
                       "kernel_frac_of_peak": multi_gbs / HBM_PEAK_GBS},
        "chunked_prefill": chunked,
        "graph": graph,
        "bf16_baseline": bf16,
        "direct_baselines": direct or None,
        "attention_rel_l2_vs_bf16": errors or None,
        "stored_bytes_per_token_head": {"rq": stored, "bf16": 2 * D * 2 * L},
        "other_workloads": others or None,
        "peak_batch": peak,
        "cpu_baseline": cpu,
        "context_from_pages": {"kv_storage_reduction": "80.7% (theoretical, mixed precision)",
                               "fixed_batch_decode_speedup": "up to 2.73x on RTX 5090",
                               "peak_throughput_speedup": "up to 4.15x on RTX 5090"},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
