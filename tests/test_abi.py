"""C-ABI checks that need no GPU: the library loads, exports every function
include/rq.h declares, its host-side pool geometry matches the oracle's own
implementation of the format, and invalid calls are rejected with the
documented status before any device work is enqueued."""
import ctypes
import os
import re
from ctypes import c_float, c_void_p

import numpy as np
import pytest

import oracle as O
from conftest import ROOT

import looped_transformer_decode_rq_amd as R
from looped_transformer_decode_rq_amd import build as B
from looped_transformer_decode_rq_amd._lib import RqDecodeOpts


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(R.library_path):
        B.build_library()
    return R.lib()


def _declared():
    src = open(os.path.join(ROOT, "include", "rq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(rq_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(R.EXPORTED)


LAYOUTS = [
    dict(H=1, D=64, G=32, L=2, bits=(2,), meta="f32", kv="f32", nblk=17),
    dict(H=16, D=128, G=128, L=4, bits=(2, 2, 2), meta="f16", kv="bf16", nblk=300),
    dict(H=55, D=96, G=96, L=8, bits=(4, 4, 2, 2, 2, 2, 2), meta="f16", kv="bf16", nblk=5),
    dict(H=3, D=128, G=32, L=3, bits=(4, 2), meta="f32", kv="bf16", nblk=9),
    dict(H=2, D=64, G=16, L=1, bits=(), meta="f16", kv="f32", nblk=4),
]


def _lay(d):
    return R.make_layout(d["H"], d["D"], d["G"], d["L"], d["bits"], d["nblk"], d["meta"], d["kv"])


@pytest.mark.parametrize("d", LAYOUTS)
def test_pool_geometry_matches_oracle(L, d):
    lay = _lay(d)
    assert R.layout_check(lay) == 0
    ol = O.PoolLayout(d["H"], d["D"], d["G"], d["L"], d["bits"], d["meta"], d["nblk"])
    assert R.pool_bytes(lay) == ol.pool_bytes
    for l in range(d["L"]):
        assert R.record_bytes(lay, l) == ol.rec_bytes(l)
    rng = np.random.default_rng(0)
    for _ in range(50):
        blk, h, l, kv = (int(rng.integers(0, d["nblk"])), int(rng.integers(0, d["H"])),
                         int(rng.integers(0, d["L"])), int(rng.integers(0, 2)))
        assert R.record_offset(lay, blk, h, l, kv) == int(ol.record_offset(blk, h, l, kv))
    assert R.record_offset(lay, d["nblk"], 0, 0, 0) == -1
    assert R.record_offset(lay, 0, 0, d["L"], 0) == -1


@pytest.mark.parametrize("bits", [(2, 2, 2, 2), (4, 2, 4, 2), (4, 4, 4, 4)])
def test_direct_pool_geometry_matches_oracle(L, bits):
    lay = R.make_layout(16, 128, 128, 4, bits, 37, "f16", "bf16", mode=R.RQ_MODE_DIRECT)
    assert R.layout_check(lay) == 0
    ol = O.PoolLayout(16, 128, 128, 4, (), "f16", 37, direct_bits=bits)
    assert R.pool_bytes(lay) == ol.pool_bytes
    for l in range(4):
        assert R.record_bytes(lay, l) == ol.rec_bytes(l)
        for blk, h, kv in ((0, 0, 0), (36, 15, 1), (7, 3, 0)):
            assert R.record_offset(lay, blk, h, l, kv) == int(ol.record_offset(blk, h, l, kv))
    bad = R.make_layout(16, 128, 128, 4, bits, 37, "f16", "bf16", mode=2)
    assert R.layout_check(bad) == -3


@pytest.mark.parametrize("field,value,status", [
    ("head_dim", 256, -3), ("head_dim", 80, -2), ("head_dim", 0, -2), ("group_size", 16, -3), ("group_size", 48, -2),
    ("num_loops", 17, -2), ("num_loops", 0, -2), ("block_size", 32, -3), ("num_blocks", 0, -2),
    ("meta_dtype", 0, -3), ("kv_dtype", 1, -3), ("num_heads", 0, -2),
])
def test_layout_rejections(L, field, value, status):
    lay = _lay(LAYOUTS[1])
    setattr(lay, field, value)
    assert R.layout_check(lay) == status
    assert R.pool_bytes(lay) == 0


def test_bits_rejection(L):
    lay = _lay(LAYOUTS[1])
    lay.loop_bits[1] = 3
    assert R.layout_check(lay) == -3
    lay.loop_bits[1] = 2
    lay.loop_bits[3] = 7          # entry of the reference loop is ignored
    assert R.layout_check(lay) == 0


def test_status_strings(L):
    for s in (0, -1, -2, -3, -4, -5, 99):
        assert isinstance(R.status_string(s), str) and R.status_string(s)


def _fake(i):
    return c_void_p(0x100000 * (i + 1))     # 16-aligned non-null; never dereferenced on these paths


def test_decode_validation(L):
    lay = _lay(LAYOUTS[1])
    loops = (ctypes.c_int32 * 1)(1)
    ws_need = R.decode_workspace_bytes(lay, 1, 4, 10)
    assert ws_need > 0
    base = [ctypes.byref(lay), _fake(0), loops, 1, _fake(1), _fake(2), _fake(3), _fake(4), 4, 10,
            None, None, c_float(0.1), _fake(5), _fake(6), ws_need, None, None]

    def call(**kw):
        a = list(base)
        idx = dict(pool=1, loops=2, n=3, q=4, rot=5, table=6, seq=7, batch=8, mb=9, tk=10, tv=11,
                   scale=12, out=13, ws=14, wsb=15)
        for k, v in kw.items():
            a[idx[k]] = v
        return L.rq_decode_attention_ex(*a)

    assert call(wsb=ws_need - 1) == -4
    assert call(pool=None) == -1
    assert call(q=None) == -1
    assert call(out=None) == -1
    assert call(ws=None) == -1
    assert call(loops=None) == -1
    assert call(tk=_fake(7)) == -1             # one tail without the other
    assert call(n=0) == -2
    assert call(n=17) == -2
    assert call(loops=(ctypes.c_int32 * 1)(4)) == -2
    assert call(loops=(ctypes.c_int32 * 1)(-1)) == -2
    assert call(mb=0) == -2
    assert call(batch=-1) == -2
    assert call(scale=c_float(float("inf"))) == -2
    assert call(pool=c_void_p(0x100008)) == -2  # misaligned pool
    assert call(batch=0) == 0                   # nothing to do, nothing launched
    # rot may be NULL only when every requested loop is the reference
    assert call(rot=None) == -1
    assert call(rot=None, loops=(ctypes.c_int32 * 1)(3), wsb=0) == -4
    bad = R.make_layout(16, 80, 80, 4, (2, 2, 2), 300)
    a = list(base)
    a[0] = ctypes.byref(bad)
    assert L.rq_decode_attention_ex(*a) == -3
    # at most 64 pages per split wave: one block-table entry per lane
    for sp, want in ((-1, -2), (65, -3)):
        a = list(base)
        a[16] = ctypes.byref(RqDecodeOpts(sp, 0, None, None))
        assert L.rq_decode_attention_ex(*a) == want


def test_decode_encode_validation(L):
    lay = _lay(LAYOUTS[1])
    loops = (ctypes.c_int32 * 1)(3)
    ws = R.decode_workspace_bytes(lay, 1, 4, 10)
    base = [ctypes.byref(lay), _fake(0), loops, 1, _fake(1), _fake(2), _fake(3), _fake(4), 4, 10,
            None, None, c_float(0.1), _fake(5), _fake(6), ws, _fake(7), _fake(8), 4, None, None]

    def call(**kw):
        a = list(base)
        idx = dict(pool=1, rot=5, kv=16, slots=17, T=18)
        for k, v in kw.items():
            a[idx[k]] = v
        return L.rq_decode_attention_encode(*a)

    assert call(kv=None) == -1
    assert call(slots=None) == -1
    assert call(pool=None) == -1
    assert call(rot=None) == -1                # L > 1: the encode needs R
    assert call(T=-1) == -2


def test_encode_validation(L):
    lay = _lay(LAYOUTS[1])
    f = L.rq_encode_pack
    assert f(ctypes.byref(lay), _fake(0), _fake(1), _fake(2), _fake(3), -1, None) == -2
    assert f(ctypes.byref(lay), _fake(0), _fake(1), _fake(2), _fake(3), 0, None) == 0
    assert f(ctypes.byref(lay), None, _fake(1), _fake(2), _fake(3), 5, None) == -1
    assert f(ctypes.byref(lay), _fake(0), None, _fake(2), _fake(3), 5, None) == -1
    assert f(ctypes.byref(lay), _fake(0), _fake(1), None, _fake(3), 5, None) == -1
    assert f(ctypes.byref(lay), _fake(0), _fake(1), _fake(2), None, 5, None) == -1
    assert f(None, _fake(0), _fake(1), _fake(2), _fake(3), 5, None) == -1


def test_bf16_validation(L):
    f = L.rq_bf16_decode_attention_ex
    need = R.bf16_workspace_bytes(16, 128, 4, 10)
    base = [16, 128, 16, 100, _fake(0), _fake(1), _fake(2), _fake(3), _fake(4), 4, 10, None, None,
            c_float(0.1), _fake(5), _fake(6), need, None, None]
    assert f(*base[:16], need - 4, None, None) == -4
    a = list(base); a[1] = 100
    assert f(*a) == -3
    a = list(base); a[2] = 8
    assert f(*a) == -3
    a = list(base); a[4] = None
    assert f(*a) == -1
    a = list(base); a[9] = 0
    assert f(*a) == 0
    assert L.rq_bf16_write(16, 128, 16, 100, _fake(0), _fake(1), _fake(2), None, 3, None) == -1
    assert L.rq_bf16_write(16, 128, 16, 100, _fake(0), _fake(1), _fake(2), _fake(3), 0, None) == 0


def test_workspace_sizes_monotone(L):
    lay = _lay(LAYOUTS[1])
    a = R.decode_workspace_bytes(lay, 1, 16, 2049)
    b = R.decode_workspace_bytes(lay, 4, 16, 2049)
    assert 0 < a < b
    assert R.decode_workspace_bytes(lay, 1, 16, 2049, 8) > R.decode_workspace_bytes(lay, 1, 16, 2049, 64)
    assert R.decode_workspace_bytes(lay, 0, 16, 2049) == 0
    assert R.decode_workspace_bytes(lay, 1, 16, 2049, 65) == 0      # at most 64 pages per split


def test_encode_needs_no_workspace(L):
    lay = _lay(LAYOUTS[1])
    assert R.encode_workspace_bytes(lay, 0) == 0
    assert R.encode_workspace_bytes(lay, 1 << 20) == 0
    size_max = (1 << (8 * ctypes.sizeof(ctypes.c_size_t))) - 1
    assert R.encode_workspace_bytes(lay, -1) == size_max
    bad = _lay(LAYOUTS[1]); bad.head_dim = 80
    assert R.encode_workspace_bytes(bad, 4) == size_max


def test_binding_refuses_host_tensors(L):
    torch = pytest.importorskip("torch")
    lay = _lay(LAYOUTS[0])
    with pytest.raises(ValueError):
        R.encode_pack(lay, torch.zeros(R.pool_bytes(lay), dtype=torch.uint8),
                      torch.zeros(2, 2, 1, 1, 64), torch.zeros(1, 2, 64, 64),
                      torch.zeros(1, dtype=torch.int64))


def test_auto_split_fills_several_rounds(L):
    """The automatic split: pages spread evenly over enough split workgroups
    for several rounds per launch, rounded up to a multiple of 8 pages, and
    the workspace query sized with the same rule. Without a GPU the device
    query falls back to 256 compute units."""
    lay = _lay(LAYOUTS[1])
    units, mb = 16 * 16, 2049
    sp1 = R.decode_auto_split_pages(lay, 1, 16, mb)
    spm = R.decode_auto_split_pages(lay, 4, 16, mb)
    assert 1 <= sp1 <= 64 and 1 <= spm <= 64
    assert sp1 % 8 == 0 and spm % 8 == 0
    wg1 = -(-mb // (4 * sp1))
    assert units * wg1 >= 7 * 3 * 256                     # >= 7 rounds of 3 workgroups per CU
    assert units * -(-mb // spm) >= 12 * 3 * 256          # one-split units: >= 12 rounds
    assert (sp1, spm) == (24, 56)                          # 22 and 49 pages spread evenly, rounded up
    assert R.decode_workspace_bytes(lay, 1, 16, mb, 0) == R.decode_workspace_bytes(lay, 1, 16, mb, sp1)
    assert R.decode_workspace_bytes(lay, 4, 16, mb, 0) == R.decode_workspace_bytes(lay, 4, 16, mb, spm)
    assert R.bf16_auto_split_pages(16, 16, mb) == spm
    assert R.bf16_workspace_bytes(16, 128, 16, mb, 0) == R.bf16_workspace_bytes(16, 128, 16, mb, spm)
    # small problems keep at least one page per split and never exceed 64
    for B_, mb_ in ((1, 1), (1, 17), (2, 257), (128, 513), (8, 513)):
        for n in (1, 4):
            sp = R.decode_auto_split_pages(lay, n, B_, mb_)
            assert 1 <= sp <= 64, (B_, mb_, n, sp)
    assert R.decode_auto_split_pages(lay, 0, 16, mb) == 0
    assert R.bf16_auto_split_pages(0, 16, mb) == 0


def test_chunk_validation(L):
    """rq_chunk_attention rejects bad calls with the documented status and
    enqueues nothing (no GPU needed); unsupported layouts are refused."""
    lay = _lay(LAYOUTS[1])                      # D128, G128, bf16 K/V: supported
    C, B, mb = 8, 4, 10
    ws = R.chunk_workspace_bytes(lay, C, B, mb)
    assert ws > 0
    base = [ctypes.byref(lay), _fake(0), 1, C, _fake(1), _fake(2), _fake(3), _fake(4), B, mb,
            _fake(5), _fake(6), c_float(0.1), _fake(7), _fake(8), ws, None, None]

    def call(**kw):
        a = list(base)
        idx = dict(pool=1, loop=2, C=3, q=4, rot=5, table=6, seq=7, batch=8, mb=9, ck=10, cv=11, scale=12,
                   out=13, ws=14, wsb=15, opts=16)
        for k, v in kw.items():
            a[idx[k]] = v
        return L.rq_chunk_attention(*a)

    assert call(wsb=ws - 1) == -4
    assert call(pool=None) == -1 and call(q=None) == -1 and call(out=None) == -1 and call(ws=None) == -1
    assert call(ck=None) == -1                  # chunk K without V
    assert call(ck=None, cv=None, wsb=0) == -4  # neither: allowed (then the workspace check fires)
    assert call(loop=4) == -2 and call(loop=-1) == -2
    assert call(C=0) == -2 and call(C=257) == -3
    assert call(batch=-1) == -2 and call(mb=0) == -2
    assert call(scale=c_float(float("nan"))) == -2
    assert call(q=c_void_p(0x100008)) == -2     # misaligned query
    assert call(rot=None) == -1                 # residual loop needs R
    assert call(rot=None, loop=3, wsb=0) == -4  # the reference loop does not
    assert call(batch=0) == 0
    assert call(opts=ctypes.byref(RqDecodeOpts(-1, 0, None, None))) == -2
    # launch grids beyond 65535 blocks in a dimension: refused before any launch
    assert call(batch=65535, C=256, wsb=1 << 62) == -3                     # batch x 64-query groups
    assert call(batch=8192, C=256, wsb=1 << 62) == -3                      # 16-row tiles
    assert call(mb=70000, opts=ctypes.byref(RqDecodeOpts(1, 0, None, None)), wsb=1 << 62) == -3   # splits
    # supported layouts only: direct mode, groups smaller than the head, fp32 K/V
    for bad in (R.make_layout(16, 128, 128, 4, (2, 2, 2), 300, "f16", "bf16", mode=R.RQ_MODE_DIRECT),
                R.make_layout(16, 128, 32, 4, (2, 2, 2), 300, "f16", "bf16"),
                R.make_layout(16, 128, 128, 4, (2, 2, 2), 300, "f16", "f32")):
        a = list(base)
        a[0] = ctypes.byref(bad)
        assert L.rq_chunk_attention(*a) == -3
        assert R.chunk_workspace_bytes(bad, C, B, mb) == 0


def test_read_probe_validation(L):
    f = L.rq_read_probe
    assert f(_fake(0), 4096, None, 1, None, None) == -1            # no sink
    assert f(None, 4096, _fake(1), 1, None, None) == -1            # no buffer for a non-empty read
    assert f(_fake(0), 4100, _fake(1), 1, None, None) == -2        # size not a multiple of 16
    assert f(c_void_p(0x1008), 4096, _fake(1), 1, None, None) == -2  # buffer not 16-byte aligned
    assert f(_fake(0), 4096, _fake(1), 0, None, None) == -2        # no sink words
