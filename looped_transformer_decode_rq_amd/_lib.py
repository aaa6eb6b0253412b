"""ctypes binding of librq.so (argument marshalling only).

Tensors are passed as raw device pointers (``tensor.data_ptr()``); the stream is
torch's current HIP stream unless one is given. Shapes and dtypes are checked
here only as far as needed to hand the library consistent sizes; the library
validates again and returns a status, which is turned into ``RqError``.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_float, c_int32, c_int64, c_size_t, c_uint8, c_void_p

HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(HERE, "librq.so")

RQ_DTYPE_BF16, RQ_DTYPE_F16, RQ_DTYPE_F32 = 0, 1, 2
RQ_MAX_LOOPS = 16
RQ_MODE_RESIDUAL, RQ_MODE_DIRECT = 0, 1

EXPORTED = [
    "rq_status_string", "rq_layout_check", "rq_pool_bytes", "rq_record_bytes", "rq_record_offset",
    "rq_encode_pack", "rq_decode_workspace_bytes", "rq_decode_auto_split_pages", "rq_decode_attention",
    "rq_decode_attention_ex", "rq_decode_attention_encode", "rq_fit_rotation", "rq_bf16_workspace_bytes",
    "rq_bf16_auto_split_pages", "rq_bf16_decode_attention", "rq_bf16_decode_attention_ex", "rq_bf16_write",
    "rq_chunk_workspace_bytes", "rq_chunk_attention", "rq_decode_attention_noalloc",
    "rq_fit_rotation_device", "rq_fit_workspace_bytes", "rq_decode_stream_probe", "rq_encode_workspace_bytes",
    "rq_read_probe",
]
RQ_NOALLOC_SCRATCH_BYTES = 64 << 20


class RqError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn}: {status_string(status)} ({status})")


class RqLayout(ctypes.Structure):
    _fields_ = [("num_heads", c_int32), ("head_dim", c_int32), ("group_size", c_int32),
                ("num_loops", c_int32), ("block_size", c_int32), ("num_blocks", c_int32),
                ("meta_dtype", c_int32), ("kv_dtype", c_int32), ("loop_bits", c_uint8 * RQ_MAX_LOOPS),
                ("mode", c_int32)]


class RqDecodeOpts(ctypes.Structure):
    _fields_ = [("split_pages", c_int32), ("reserved", c_int32),
                ("event_main_begin", c_void_p), ("event_main_end", c_void_p)]


_LIB = None


def lib():
    """The loaded library; raises if it has not been built (no fallback)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(library_path):
            raise RuntimeError(f"librq.so not found at {library_path}; build it with "
                               "python -m looped_transformer_decode_rq_amd.build")
        L = ctypes.CDLL(library_path)
        P = c_void_p
        sig = {
            "rq_status_string": (ctypes.c_char_p, [c_int32]),
            "rq_layout_check": (c_int32, [POINTER(RqLayout)]),
            "rq_pool_bytes": (c_size_t, [POINTER(RqLayout)]),
            "rq_record_bytes": (c_size_t, [POINTER(RqLayout), c_int32]),
            "rq_record_offset": (c_int64, [POINTER(RqLayout), c_int32, c_int32, c_int32, c_int32]),
            "rq_encode_pack": (c_int32, [POINTER(RqLayout), P, P, P, P, c_int32, P]),
            "rq_encode_workspace_bytes": (c_size_t, [POINTER(RqLayout), c_int32]),
            "rq_decode_workspace_bytes": (c_size_t, [POINTER(RqLayout), c_int32, c_int32, c_int32, c_int32]),
            "rq_decode_auto_split_pages": (c_int32, [POINTER(RqLayout), c_int32, c_int32, c_int32]),
            "rq_decode_attention": (c_int32, [POINTER(RqLayout), P, P, c_int32, P, P, P, P, c_int32, c_int32,
                                              P, P, c_float, P, P, c_size_t, P]),
            "rq_decode_attention_ex": (c_int32, [POINTER(RqLayout), P, P, c_int32, P, P, P, P, c_int32, c_int32,
                                                 P, P, c_float, P, P, c_size_t, POINTER(RqDecodeOpts), P]),
            "rq_decode_attention_encode": (c_int32, [POINTER(RqLayout), P, P, c_int32, P, P, P, P, c_int32, c_int32,
                                                     P, P, c_float, P, P, c_size_t, P, P, c_int32,
                                                     POINTER(RqDecodeOpts), P]),
            "rq_decode_attention_noalloc": (c_int32, [POINTER(RqLayout), P, P, c_int32, P, P, P, P, c_int32,
                                                      c_int32, P, P, c_float, P, POINTER(RqDecodeOpts), P]),
            "rq_chunk_workspace_bytes": (c_size_t, [POINTER(RqLayout), c_int32, c_int32, c_int32, c_int32]),
            "rq_chunk_attention": (c_int32, [POINTER(RqLayout), P, c_int32, c_int32, P, P, P, P, c_int32, c_int32,
                                             P, P, c_float, P, P, c_size_t, POINTER(RqDecodeOpts), P]),
            "rq_fit_rotation": (c_int32, [P, c_int64, c_int32, c_int32, c_int32, c_int32, P, c_int32, P, P]),
            "rq_fit_rotation_device": (c_int32, [P, c_int64, c_int32, c_int32, c_int32, c_int32, P, c_int32, P, P,
                                                 P, c_size_t, P]),
            "rq_fit_workspace_bytes": (c_size_t, [c_int32]),
            "rq_decode_stream_probe": (c_int32, [POINTER(RqLayout), P, c_int32, P, P, c_int32, c_int32, P, c_size_t,
                                                 POINTER(RqDecodeOpts), P]),
            "rq_read_probe": (c_int32, [P, c_size_t, P, c_int32, POINTER(RqDecodeOpts), P]),
            "rq_bf16_workspace_bytes": (c_size_t, [c_int32, c_int32, c_int32, c_int32, c_int32]),
            "rq_bf16_auto_split_pages": (c_int32, [c_int32, c_int32, c_int32]),
            "rq_bf16_decode_attention": (c_int32, [c_int32, c_int32, c_int32, c_int32, P, P, P, P, P, c_int32,
                                                   c_int32, P, P, c_float, P, P, c_size_t, P]),
            "rq_bf16_decode_attention_ex": (c_int32, [c_int32, c_int32, c_int32, c_int32, P, P, P, P, P, c_int32,
                                                      c_int32, P, P, c_float, P, P, c_size_t,
                                                      POINTER(RqDecodeOpts), P]),
            "rq_bf16_write": (c_int32, [c_int32, c_int32, c_int32, c_int32, P, P, P, P, c_int32, P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _LIB = L
    return _LIB


def status_string(status: int) -> str:
    return lib().rq_status_string(int(status)).decode()


def _check(fn, status):
    if status != 0:
        raise RqError(fn, status)


def _ptr(t):
    if t is None:
        return None
    if not getattr(t, "is_cuda", False):
        raise ValueError("librq takes device tensors only (got a host tensor)")
    return c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return c_void_p(int(stream))
    import torch
    return c_void_p(torch.cuda.current_stream().cuda_stream)


_DT = {"bf16": RQ_DTYPE_BF16, "f16": RQ_DTYPE_F16, "f32": RQ_DTYPE_F32}


def make_layout(num_heads, head_dim, group_size, num_loops, res_bits, num_blocks,
                meta_dtype="f16", kv_dtype="bf16", block_size=16, mode=0) -> RqLayout:
    """rq_layout. mode 0 (RQ_MODE_RESIDUAL): res_bits are the L-1 residual
    widths; mode 1 (RQ_MODE_DIRECT): res_bits are the L per-loop widths."""
    lay = RqLayout()
    lay.mode = int(mode)
    lay.num_heads, lay.head_dim, lay.group_size = num_heads, head_dim, group_size
    lay.num_loops, lay.block_size, lay.num_blocks = num_loops, block_size, num_blocks
    lay.meta_dtype = _DT[meta_dtype] if isinstance(meta_dtype, str) else meta_dtype
    lay.kv_dtype = _DT[kv_dtype] if isinstance(kv_dtype, str) else kv_dtype
    for i, b in enumerate(res_bits):
        lay.loop_bits[i] = int(b)
    return lay


def layout_check(layout) -> int:
    return lib().rq_layout_check(ctypes.byref(layout))


def pool_bytes(layout) -> int:
    return lib().rq_pool_bytes(ctypes.byref(layout))


def record_bytes(layout, loop) -> int:
    return lib().rq_record_bytes(ctypes.byref(layout), loop)


def record_offset(layout, block, head, loop, kv) -> int:
    return lib().rq_record_offset(ctypes.byref(layout), block, head, loop, kv)


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _nbytes(t):
    return t.numel() * t.element_size()


def _kv_bytes(layout):
    return 4 if layout.kv_dtype == RQ_DTYPE_F32 else 2


def _check_rot(layout, rot):
    H, D = layout.num_heads, layout.head_dim
    _need(tuple(rot.shape) == (H, 2, D, D) and rot.element_size() == 4 and rot.is_contiguous(),
          f"rot must be contiguous fp32 [{H}][2][{D}][{D}]")


def encode_pack(layout, pool, kv_new, rot, slot_mapping, stream=None):
    """rq_encode_pack: kv_new [L][2][T][H][D], rot [H][2][D][D] fp32, slots [T] int64."""
    T = 0 if kv_new is None else int(kv_new.shape[2])
    if T:
        L, H, D = layout.num_loops, layout.num_heads, layout.head_dim
        _need(_nbytes(pool) >= pool_bytes(layout) > 0, "pool smaller than rq_pool_bytes(layout)")
        _need(tuple(kv_new.shape) == (L, 2, T, H, D) and kv_new.element_size() == _kv_bytes(layout)
              and kv_new.is_contiguous(), f"kv_new must be contiguous [{L}][2][T][{H}][{D}] in kv_dtype")
        _need(slot_mapping.numel() == T and slot_mapping.element_size() == 8, "slot_mapping must be int64 [T]")
        if L > 1 and layout.mode == RQ_MODE_RESIDUAL:
            _check_rot(layout, rot)
    _check("rq_encode_pack", lib().rq_encode_pack(
        ctypes.byref(layout), _ptr(pool), _ptr(kv_new), _ptr(rot), _ptr(slot_mapping), T, _stream(stream)))


def encode_workspace_bytes(layout, num_tokens) -> int:
    """rq_encode_workspace_bytes: 0 for a valid layout (the encoder needs no device workspace)."""
    return lib().rq_encode_workspace_bytes(ctypes.byref(layout), num_tokens)


def decode_workspace_bytes(layout, n_loops, batch, max_blocks_per_seq, split_pages=0) -> int:
    return lib().rq_decode_workspace_bytes(ctypes.byref(layout), n_loops, batch, max_blocks_per_seq, split_pages)


def decode_auto_split_pages(layout, n_loops, batch, max_blocks_per_seq) -> int:
    """Pages per split the decode call picks for split_pages=0 on the current device."""
    return lib().rq_decode_auto_split_pages(ctypes.byref(layout), n_loops, batch, max_blocks_per_seq)


def _opts(split_pages, events):
    o = RqDecodeOpts()
    o.split_pages = int(split_pages or 0)
    if events is not None:
        o.event_main_begin, o.event_main_end = events
    return o


def decode_attention_noalloc(layout, pool, loops, q, rot, block_table, seq_lens, tail_k, tail_v,
                             softmax_scale, out, split_pages=0, stream=None):
    """rq_decode_attention_noalloc: decode attention with the library's fixed
    device scratch instead of a caller workspace (nothing is allocated)."""
    n = len(loops)
    arr = (c_int32 * max(n, 1))(*[int(x) for x in loops])
    B, mb = int(block_table.shape[0]), int(block_table.shape[1])
    H, D = layout.num_heads, layout.head_dim
    _need(_nbytes(pool) >= pool_bytes(layout) > 0, "pool smaller than rq_pool_bytes(layout)")
    shp = (n, B, H, D)
    _need(tuple(q.shape) == shp and q.element_size() == _kv_bytes(layout) and q.is_contiguous(),
          f"q must be contiguous {shp} in kv_dtype")
    _need(tuple(out.shape) == shp and out.element_size() == 4 and out.is_contiguous(), f"out must be fp32 {shp}")
    _need(block_table.element_size() == 4 and block_table.is_contiguous(), "block_table must be int32 [B][M]")
    _need(seq_lens.numel() == B and seq_lens.element_size() == 4, "seq_lens must be int32 [B]")
    _need((tail_k is None) == (tail_v is None), "tail_k and tail_v go together")
    for t in (tail_k, tail_v):
        if t is not None:
            _need(tuple(t.shape) == shp and t.element_size() == _kv_bytes(layout) and t.is_contiguous(),
                  f"tails must be contiguous {shp} in kv_dtype")
    if layout.mode == RQ_MODE_RESIDUAL and any(int(l) != layout.num_loops - 1 for l in loops):
        _check_rot(layout, rot)
    o = _opts(split_pages, None)
    _check("rq_decode_attention_noalloc", lib().rq_decode_attention_noalloc(
        ctypes.byref(layout), _ptr(pool), arr, n, _ptr(q), _ptr(rot), _ptr(block_table), _ptr(seq_lens),
        B, mb, _ptr(tail_k), _ptr(tail_v), float(softmax_scale), _ptr(out), ctypes.byref(o), _stream(stream)))


def decode_attention(layout, pool, loops, q, rot, block_table, seq_lens, tail_k, tail_v,
                     softmax_scale, out, workspace, split_pages=0, events=None, stream=None,
                     kv_new=None, slot_mapping=None):
    """rq_decode_attention_ex; loops is a host sequence of loop indices. With
    kv_new / slot_mapping (as in encode_pack) it is rq_decode_attention_encode:
    the current tokens are also compressed into `pool`, in the same launches."""
    n = len(loops)
    arr = (c_int32 * max(n, 1))(*[int(x) for x in loops])
    B, mb = int(block_table.shape[0]), int(block_table.shape[1])
    ws_bytes = workspace.numel() * workspace.element_size()
    H, D = layout.num_heads, layout.head_dim
    _need(_nbytes(pool) >= pool_bytes(layout) > 0, "pool smaller than rq_pool_bytes(layout)")
    shp = (n, B, H, D)
    _need(tuple(q.shape) == shp and q.element_size() == _kv_bytes(layout) and q.is_contiguous(),
          f"q must be contiguous {shp} in kv_dtype")
    _need(tuple(out.shape) == shp and out.element_size() == 4 and out.is_contiguous(), f"out must be fp32 {shp}")
    _need(block_table.element_size() == 4 and block_table.is_contiguous(), "block_table must be int32 [B][M]")
    _need(seq_lens.numel() == B and seq_lens.element_size() == 4, "seq_lens must be int32 [B]")
    _need((tail_k is None) == (tail_v is None), "tail_k and tail_v go together")
    for t in (tail_k, tail_v):
        if t is not None:
            _need(tuple(t.shape) == shp and t.element_size() == _kv_bytes(layout) and t.is_contiguous(),
                  f"tails must be contiguous {shp} in kv_dtype")
    if layout.mode == RQ_MODE_RESIDUAL and any(int(l) != layout.num_loops - 1 for l in loops):
        _check_rot(layout, rot)
    o = _opts(split_pages, events)
    if kv_new is None and slot_mapping is None:
        _check("rq_decode_attention", lib().rq_decode_attention_ex(
            ctypes.byref(layout), _ptr(pool), arr, n, _ptr(q), _ptr(rot), _ptr(block_table), _ptr(seq_lens),
            B, mb, _ptr(tail_k), _ptr(tail_v), float(softmax_scale), _ptr(out), _ptr(workspace), ws_bytes,
            ctypes.byref(o), _stream(stream)))
        return
    _need(kv_new is not None and slot_mapping is not None, "kv_new and slot_mapping go together")
    L = layout.num_loops
    T = int(kv_new.shape[2])
    _need(tuple(kv_new.shape) == (L, 2, T, H, D) and kv_new.element_size() == _kv_bytes(layout)
          and kv_new.is_contiguous(), f"kv_new must be contiguous [{L}][2][T][{H}][{D}] in kv_dtype")
    _need(slot_mapping.numel() == T and slot_mapping.element_size() == 8, "slot_mapping must be int64 [T]")
    if L > 1 and layout.mode == RQ_MODE_RESIDUAL:
        _check_rot(layout, rot)
    _check("rq_decode_attention_encode", lib().rq_decode_attention_encode(
        ctypes.byref(layout), _ptr(pool), arr, n, _ptr(q), _ptr(rot), _ptr(block_table), _ptr(seq_lens),
        B, mb, _ptr(tail_k), _ptr(tail_v), float(softmax_scale), _ptr(out), _ptr(workspace), ws_bytes,
        _ptr(kv_new), _ptr(slot_mapping), T, ctypes.byref(o), _stream(stream)))


def bf16_workspace_bytes(num_heads, head_dim, batch, max_blocks_per_seq, split_pages=0) -> int:
    return lib().rq_bf16_workspace_bytes(num_heads, head_dim, batch, max_blocks_per_seq, split_pages)


def chunk_workspace_bytes(layout, chunk, batch, max_blocks_per_seq, split_pages=0) -> int:
    return lib().rq_chunk_workspace_bytes(ctypes.byref(layout), chunk, batch, max_blocks_per_seq, split_pages)


def chunk_attention(layout, pool, loop, q, rot, block_table, seq_lens, chunk_k, chunk_v, softmax_scale, out,
                    workspace, split_pages=0, events=None, stream=None):
    """rq_chunk_attention: q, chunk_k, chunk_v [B][C][H][D] bf16 (chunk K/V may
    both be None), out [B][C][H][D] fp32."""
    B, C, H, D = (int(x) for x in q.shape)
    _need(H == layout.num_heads and D == layout.head_dim and q.element_size() == 2 and q.is_contiguous(),
          "q must be contiguous bf16 [B][C][H][D]")
    _need(tuple(out.shape) == (B, C, H, D) and out.element_size() == 4 and out.is_contiguous(), "out must be fp32 [B][C][H][D]")
    _need(int(block_table.shape[0]) == B and block_table.element_size() == 4 and block_table.is_contiguous(),
          "block_table must be int32 [B][M]")
    _need(seq_lens.numel() == B and seq_lens.element_size() == 4, "seq_lens must be int32 [B]")
    _need((chunk_k is None) == (chunk_v is None), "chunk_k and chunk_v go together")
    for t in (chunk_k, chunk_v):
        if t is not None:
            _need(tuple(t.shape) == (B, C, H, D) and t.element_size() == 2 and t.is_contiguous(),
                  "chunk K/V must be contiguous bf16 [B][C][H][D]")
    _need(_nbytes(pool) >= pool_bytes(layout) > 0, "pool smaller than rq_pool_bytes(layout)")
    if int(loop) != layout.num_loops - 1:
        _check_rot(layout, rot)
    o = _opts(split_pages, events)
    _check("rq_chunk_attention", lib().rq_chunk_attention(
        ctypes.byref(layout), _ptr(pool), int(loop), C, _ptr(q), _ptr(rot), _ptr(block_table), _ptr(seq_lens), B,
        int(block_table.shape[1]), _ptr(chunk_k), _ptr(chunk_v), float(softmax_scale), _ptr(out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), ctypes.byref(o), _stream(stream)))


def bf16_auto_split_pages(num_heads, batch, max_blocks_per_seq) -> int:
    return lib().rq_bf16_auto_split_pages(num_heads, batch, max_blocks_per_seq)


def bf16_decode_attention(k_cache, v_cache, q, block_table, seq_lens, tail_k, tail_v, softmax_scale, out,
                          workspace, split_pages=0, events=None, stream=None):
    nblk, H, bs, D = (int(x) for x in k_cache.shape)
    B, mb = int(block_table.shape[0]), int(block_table.shape[1])
    ws_bytes = workspace.numel() * workspace.element_size()
    _need(tuple(v_cache.shape) == tuple(k_cache.shape) and k_cache.element_size() == 2
          and v_cache.element_size() == 2 and k_cache.is_contiguous() and v_cache.is_contiguous(),
          "k_cache/v_cache must be contiguous bf16 [num_blocks][H][16][D]")
    shp = (B, H, D)
    _need(tuple(q.shape) == shp and q.element_size() == 2 and q.is_contiguous(), f"q must be bf16 {shp}")
    _need(tuple(out.shape) == shp and out.element_size() == 4 and out.is_contiguous(), f"out must be fp32 {shp}")
    _need(block_table.element_size() == 4 and block_table.is_contiguous(), "block_table must be int32 [B][M]")
    _need(seq_lens.numel() == B and seq_lens.element_size() == 4, "seq_lens must be int32 [B]")
    _need((tail_k is None) == (tail_v is None), "tail_k and tail_v go together")
    for t in (tail_k, tail_v):
        if t is not None:
            _need(tuple(t.shape) == shp and t.element_size() == 2 and t.is_contiguous(), f"tails must be bf16 {shp}")
    o = _opts(split_pages, events)
    _check("rq_bf16_decode_attention", lib().rq_bf16_decode_attention_ex(
        H, D, bs, nblk, _ptr(k_cache), _ptr(v_cache), _ptr(q), _ptr(block_table), _ptr(seq_lens), B, mb,
        _ptr(tail_k), _ptr(tail_v), float(softmax_scale), _ptr(out), _ptr(workspace), ws_bytes,
        ctypes.byref(o), _stream(stream)))


def bf16_write(k_cache, v_cache, kv_new, slot_mapping, stream=None):
    nblk, H, bs, D = (int(x) for x in k_cache.shape)
    T = int(kv_new.shape[1])
    _need(tuple(kv_new.shape) == (2, T, H, D) and kv_new.element_size() == 2 and kv_new.is_contiguous(),
          f"kv_new must be contiguous bf16 [2][T][{H}][{D}]")
    _need(tuple(v_cache.shape) == tuple(k_cache.shape), "k_cache/v_cache shapes differ")
    _need(slot_mapping.numel() == T and slot_mapping.element_size() == 8, "slot_mapping must be int64 [T]")
    _check("rq_bf16_write", lib().rq_bf16_write(
        H, D, bs, nblk, _ptr(k_cache), _ptr(v_cache), _ptr(kv_new), _ptr(slot_mapping),
        int(kv_new.shape[1]), _stream(stream)))


def fit_rotation(samples, rot0, bits, group_size, meta_dtype="f16", iters=10):
    """rq_fit_rotation on HOST arrays (calibration, not the decode path):
    samples [n][D] float32, rot0 [D][D] float32 -> (fitted R [D][D] float32,
    objective [iters + 1] float64)."""
    import numpy as np
    x = np.ascontiguousarray(samples, dtype=np.float32)
    r0 = np.ascontiguousarray(rot0, dtype=np.float32)
    n, D = x.shape
    _need(r0.shape == (D, D), "rot0 must be [D][D]")
    out = np.empty((D, D), np.float32)
    obj = np.empty(int(iters) + 1, np.float64)
    md = _DT[meta_dtype] if isinstance(meta_dtype, str) else meta_dtype
    _check("rq_fit_rotation", lib().rq_fit_rotation(
        x.ctypes.data_as(c_void_p), n, D, int(bits), int(group_size), md, r0.ctypes.data_as(c_void_p),
        int(iters), out.ctypes.data_as(c_void_p), obj.ctypes.data_as(c_void_p)))
    return out, obj


def fit_workspace_bytes(head_dim) -> int:
    return lib().rq_fit_workspace_bytes(int(head_dim))


def fit_rotation_device(samples, rot0, bits, group_size, workspace, meta_dtype="f16", iters=10, stream=None):
    """rq_fit_rotation_device: samples a DEVICE tensor [n][D] float32, rot0 a
    host array [D][D] float32, workspace a device uint8 tensor of
    fit_workspace_bytes(D) -> (fitted R [D][D] float32, objective
    [iters + 1] float64), both on the host."""
    import numpy as np
    n, D = (int(v) for v in samples.shape)
    _need(samples.element_size() == 4 and samples.is_contiguous(), "samples must be contiguous float32 [n][D]")
    r0 = np.ascontiguousarray(rot0, dtype=np.float32)
    _need(r0.shape == (D, D), "rot0 must be [D][D]")
    out = np.empty((D, D), np.float32)
    obj = np.empty(int(iters) + 1, np.float64)
    md = _DT[meta_dtype] if isinstance(meta_dtype, str) else meta_dtype
    _check("rq_fit_rotation_device", lib().rq_fit_rotation_device(
        _ptr(samples), n, D, int(bits), int(group_size), md, r0.ctypes.data_as(c_void_p), int(iters),
        out.ctypes.data_as(c_void_p), obj.ctypes.data_as(c_void_p), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return out, obj


def decode_stream_probe(layout, pool, loop, block_table, seq_lens, workspace, split_pages=0, events=None,
                        stream=None):
    """rq_decode_stream_probe: the per-loop decode kernel's loads of loop
    `loop` with no attention arithmetic (an HBM-rate reference)."""
    B, mb = int(block_table.shape[0]), int(block_table.shape[1])
    _need(_nbytes(pool) >= pool_bytes(layout) > 0, "pool smaller than rq_pool_bytes(layout)")
    _need(block_table.element_size() == 4 and block_table.is_contiguous(), "block_table must be int32 [B][M]")
    _need(seq_lens.numel() == B and seq_lens.element_size() == 4, "seq_lens must be int32 [B]")
    o = _opts(split_pages, events)
    _check("rq_decode_stream_probe", lib().rq_decode_stream_probe(
        ctypes.byref(layout), _ptr(pool), int(loop), _ptr(block_table), _ptr(seq_lens), B, mb, _ptr(workspace),
        workspace.numel() * workspace.element_size(), ctypes.byref(o), _stream(stream)))


def read_probe(buf, sink, events=None, stream=None):
    """rq_read_probe: a plain contiguous read of the device tensor `buf` (an
    HBM-rate reference). sink: a contiguous 32-bit device tensor zeroed by the
    caller (one word per wave: 32 per compute unit); the XOR of its words
    becomes the XOR of the buffer's 32-bit words."""
    _need(buf.is_cuda and buf.is_contiguous(), "buf must be a contiguous device tensor")
    _need(sink.is_cuda and sink.is_contiguous() and sink.element_size() == 4 and sink.numel() >= 1,
          "sink must be a contiguous 32-bit device tensor")
    o = _opts(0, events)
    _check("rq_read_probe", lib().rq_read_probe(_ptr(buf), _nbytes(buf), _ptr(sink), int(sink.numel()),
                                                ctypes.byref(o), _stream(stream)))
