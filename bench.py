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


def setup_rq(w, dev, split_pages, split_pages_multi):
    import torch
    import looped_transformer_decode_rq_amd as R
    import workloads as W
    B, N, H, D, L = w.batch, w.context, w.heads, w.head_dim, w.loops
    st = W.structure(w, 0)
    table, nblk = W.block_table(w)
    lay = R.make_layout(H, D, w.group_size, L, w.res_bits, nblk, w.meta_dtype, w.kv_dtype)
    pool = torch.zeros(R.pool_bytes(lay), dtype=torch.uint8, device=dev)
    rot = torch.from_numpy(st["rot32"]).to(dev)
    kvdt = torch.bfloat16 if w.kv_dtype == "bf16" else torch.float32
    cur = torch.empty((L, 2, B, H, D), dtype=kvdt, device=dev)      # current token, all loops
    pos = np.arange(N)
    for b in range(B):
        kvb = W.kv_torch(w, 0, b, st, dev)
        slots = torch.from_numpy(table[b, pos // 16].astype(np.int64) * 16 + pos % 16).to(dev)
        R.encode_pack(lay, pool, kvb[:, :, :N].contiguous(), rot, slots)
        cur[:, :, b] = kvb[:, :, N]
        del kvb
    torch.cuda.synchronize()
    q = W.queries_torch(w, 0, dev)
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


def rq_step(w, s, split_pages, events=None, fused=True):
    """One decode step: the loops' attention calls in order; the new tokens'
    compression rides in the reference-loop call (fused) or follows it."""
    import looped_transformer_decode_rq_amd as R
    tau = 1.0 / np.sqrt(w.head_dim)
    ref = w.loops - 1
    for l in range(w.loops):
        ev = None if events is None else events[l]
        enc = dict(kv_new=s["kv_new"], slot_mapping=s["slots_new"]) if fused and l == ref else {}
        R.decode_attention(s["lay"], s["pool"], [l], s["qs"][l], s["rot"], s["d_table"], s["d_seq"],
                           s["tk"][l], s["tv"][l], tau, s["out"][l], s["ws"], split_pages=split_pages, events=ev,
                           **enc)
    if not fused:
        R.encode_pack(s["lay"], s["pool"], s["kv_new"], s["rot"], s["slots_new"])


def rq_multi_step(w, s, split_pages, events=None, fused=True):
    import looped_transformer_decode_rq_amd as R
    tau = 1.0 / np.sqrt(w.head_dim)
    enc = dict(kv_new=s["kv_new"], slot_mapping=s["slots_new"]) if fused else {}
    R.decode_attention(s["lay"], s["pool"], list(range(w.loops)), s["q_all"], s["rot"], s["d_table"], s["d_seq"],
                       s["tk_all"], s["tv_all"], tau, s["out_all"], s["ws_all"], split_pages=split_pages,
                       events=events, **enc)
    if not fused:
        R.encode_pack(s["lay"], s["pool"], s["kv_new"], s["rot"], s["slots_new"])


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


def timed(fn, steps, warmup):
    import torch
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


def cpu_baseline(w, rq, budget_s=12.0):
    """The fp64 oracle on a bounded sample: decode attention of one (sequence,
    head) unit per loop, repeated over units until the budget is spent, plus
    the oracle encode of one step's new tokens; extrapolated to a full step."""
    import torch
    import oracle as O
    import workloads as W
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = 1
    B, N, H, D, L = w.batch, w.context, w.heads, w.head_dim, w.loops
    st = rq["st"]
    tau = 1.0 / np.sqrt(D)
    times = {l: [] for l in range(L)}
    units = 0
    t_start = time.perf_counter()
    npages = -(-N // 16)
    pos = np.arange(N)
    mini = O.PoolLayout(1, D, w.group_size, L, w.res_bits, w.meta_dtype, npages)
    q_h = rq["q"].float().cpu().numpy().astype(np.float64)
    cur = rq["cur"].float().cpu().numpy().astype(np.float64)
    for h in range(H):
        kvb = W.kv_torch(w, 0, 0, st, torch.device("cuda:0"))
        kvh = kvb[:, :, :N, h:h + 1].float().cpu().numpy().astype(np.float64)
        del kvb
        enc = O.encode(kvh, st["rot32"][h:h + 1], w.res_bits, w.group_size, w.meta_dtype)
        opool = np.zeros(mini.pool_bytes, np.uint8)
        O.write_tokens(opool, mini, enc, pos)
        for l in range(L):
            t0 = time.perf_counter()
            O.decode_attention(opool, mini, l, q_h[l, 0:1, h:h + 1], st["rot32"][h:h + 1],
                               np.arange(npages)[None], [N], tau, cur[l, 0, 0:1, h:h + 1], cur[l, 1, 0:1, h:h + 1])
            times[l].append(time.perf_counter() - t0)
        units += 1
        if time.perf_counter() - t_start > budget_s:
            break
    t0 = time.perf_counter()
    enc_new = O.encode(cur[:, :, :, :, :], st["rot32"], w.res_bits, w.group_size, w.meta_dtype)
    t_enc = time.perf_counter() - t0
    step = sum(B * H * float(np.mean(times[l])) for l in range(L)) + t_enc
    del enc_new
    return {"value": B / step, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{units} (sequence, head) units x {L} loops of fp64 decode attention over {N} packed tokens "
                      f"+ fp64 encode of one step's {B} new tokens; step time extrapolated to {B}x{H} units "
                      f"({step:.1f} s per step)"}


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


def kernel_src_hash():
    import hashlib
    h = hashlib.sha256()
    for f in ("rq_decode.hip", "rq_device.h", "rq_internal.h", "rq_vmfma.h"):
        h.update(open(os.path.join(ROOT, "looped_transformer_decode_rq_amd", "csrc", f), "rb").read())
    return h.hexdigest()


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
    qp = 64 + 11 * D // 2                              # query record: header + 6 + 5 limb planes
    res_bytes = (token_head_bytes(w, 0) * B * H * N + B * H * qp + B * N // 16 * 4
                 + B * H * nwg * (2 + 2 * D) * 4)
    ref_bytes = (token_head_bytes(w, L - 1) * B * H * N + B * H * qp + B * N // 16 * 4
                 + B * H * nwg * (2 + D) * 4)
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

    cpu = None
    if not args.no_cpu:
        log("timing the fp64 oracle on the host")
        cpu = cpu_baseline(w, rq)

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
        "dtype": "int4/int2 codes x fp32 (bf16 inputs, fp16 metadata)",
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
        "ref_loop_kernel": {"ms": ref_ms, "gbs": ref_bytes / (ref_ms * 1e-3) / 1e9, "bytes_per_launch": ref_bytes,
                            "traffic": measured("reference")},
        "multi_loop": {"tokens_per_s": B / t_multi, "ms_per_step": t_multi * 1e3,
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
        "cpu_baseline": cpu,
        "context_from_pages": {"kv_storage_reduction": "80.7% (theoretical, mixed precision)",
                               "fixed_batch_decode_speedup": "up to 2.73x on RTX 5090",
                               "peak_throughput_speedup": "up to 4.15x on RTX 5090"},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
