"""C-ABI boundary on the CPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host (no kernel launch;
each case below fails a host-side check before anything is enqueued)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fm_api.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w[\w\s\*]*?\b(fm_\w+)\s*\(", text, flags=re.M)))


def test_header_symbols_exported():
    pv = pytest.importorskip("packed_varlen_masked_amd")
    names = _declared()
    assert len(names) >= 12
    lib = ctypes.CDLL(pv.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(pv.EXPORTED)


@pytest.fixture(scope="module")
def pv():
    return pytest.importorskip("packed_varlen_masked_amd")


def test_copy_tables(pv):
    """The bf16 kernel's copy table: every K/V block copied once, every lane
    reading a row inside its 64-row tile (checked on the host)."""
    pv.self_check()


def test_tile_config(pv):
    import torch
    assert pv.tile_config(torch.bfloat16, 128) == (256, 64)
    assert pv.tile_config(torch.float32, 32) == (64, 32)
    with pytest.raises(pv.FMError) as e:
        pv.tile_config(torch.bfloat16, 64)
    assert e.value.code == pv.FM_E_UNSUPPORTED


def test_auto_split(pv):
    import torch
    assert pv.auto_split(4352, 3, 2, torch.bfloat16, 128) > 0        # few items: split long rows
    assert pv.auto_split(131072, 8, 8, torch.bfloat16, 128) == 0     # plenty of items
    assert pv.auto_split(16, 1, 1, torch.float32, 32) == 0


def test_layout_bounds(pv):
    lay = pv.workspace_layout(4352, 3, 2, 128, 128, 64, 0, True)
    assert lay.kb_cap >= 4352 // 64 + 3 and lay.item_cap >= 2 * (4352 // 128 + 3)
    offs = [lay.off_hdr, lay.off_kb_off, lay.off_extrema, lay.off_items, lay.off_tile_class, lay.off_scratch]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    assert lay.bytes >= lay.off_scratch + lay.scratch_bytes
    lay2 = pv.workspace_layout(4352, 3, 2, 128, 128, 64, 4, False)
    assert lay2.partial_bytes >= lay2.slot_cap * 2 * (128 * 128 * 2 + 3 * 128 * 4)
    for bad in [dict(N=-1), dict(B=0), dict(H=0), dict(bq=0), dict(S=-2)]:
        a = dict(N=100, B=1, H=1, bq=16, bk=16, S=0)
        a.update(bad)
        with pytest.raises(pv.FMError) as e:
            pv.workspace_layout(a["N"], a["B"], a["H"], 32, a["bq"], a["bk"], a["S"], False)
        assert e.value.code == pv.FM_E_INVAL
    with pytest.raises(pv.FMError) as e:   # one q tile could visit > FM_MAX_COST key blocks
        pv.workspace_layout(2 ** 21, 1, 1, 128, 128, 64, 0, False)
    assert e.value.code == pv.FM_E_UNSUPPORTED


FAKE = ctypes.c_void_p(4096)  # never dereferenced: every call below fails on the host


def _attn(pv, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, dtype=pv.FM_BF16, N=256, H=2, D=128, cu=FAKE, B=1, sv=FAKE,
             n_vec=1, causal=1, scale=0.1, out=FAKE, lse=FAKE, bq=0, bk=0, S=0, ws=FAKE,
             ws_bytes=1 << 40, flags=0)
    a.update(kw)
    rc = pv._lib.fm_attn_fwd(a["q"], a["k"], a["v"], a["dtype"], a["N"], a["H"], a["D"], a["cu"], a["B"],
                             a["sv"], a["n_vec"], a["causal"], ctypes.c_float(a["scale"]), a["out"], a["lse"],
                             a["bq"], a["bk"], a["S"], a["ws"], a["ws_bytes"], a["flags"], None)
    return rc, pv._lib.fm_last_error().decode()


@pytest.mark.parametrize("kw,code", [
    (dict(n_vec=4), 1), (dict(n_vec=3, causal=0), 1), (dict(n_vec=1, causal=0), 1),
    (dict(D=64), 2), (dict(dtype=7), 2), (dict(bq=64), 2), (dict(bq=128), 2), (dict(dtype=1, D=32, bq=65), 2),
    (dict(scale=0.0), 1), (dict(scale=float("inf")), 1), (dict(scale=-1.0), 1),
    (dict(flags=0x80), 1), (dict(flags=1, S=4), 1), (dict(dtype=1, D=32, S=3), 2),
    (dict(cu=None), 1), (dict(q=None), 1), (dict(ws=None), 1), (dict(ws_bytes=1024), 3),
    (dict(B=0), 1), (dict(B=20000), 1), (dict(N=-5), 1), (dict(H=0), 1), (dict(N=2 ** 31), 1),
])
def test_attn_rejects_on_host(pv, kw, code):
    rc, msg = _attn(pv, **kw)
    assert rc == code, msg
    assert msg


@pytest.mark.parametrize("kw,code", [
    (dict(flags=2), 1),                         # FM_FLAG_PLAN_READY: the array holds no plan of the caller's
    (dict(N=16384, H=32, B=14, S=6), 3),        # a 6 GB workspace does not fit the 64 MiB array
    (dict(D=64), 2), (dict(B=0), 1), (dict(H=0), 1),
])
def test_noalloc_rejects_on_host(pv, kw, code):
    """The allocation-free forward rejects a ready-plan flag and problems
    whose workspace exceeds its array before it touches the device."""
    a = dict(dtype=pv.FM_BF16, N=256, H=2, D=128, B=1, S=0, flags=0)
    a.update(kw)
    rc = pv._lib.fm_attn_fwd_noalloc(FAKE, FAKE, FAKE, a["dtype"], a["N"], a["H"], a["D"], FAKE, a["B"], FAKE, 1, 1,
                                     ctypes.c_float(0.1), FAKE, FAKE, 0, 0, a["S"], a["flags"], None)
    msg = pv._lib.fm_last_error().decode()
    assert rc == code, msg
    assert msg
    if code == 3:
        assert str(pv.NOALLOC_SCRATCH_BYTES) in msg


def test_preprocess_rejects_on_host(pv):
    L = pv._lib
    r = L.fm_preprocess_mask(FAKE, 3, 1, FAKE, 1, 64, 16, FAKE, FAKE, 100, FAKE, FAKE, None)
    assert r == pv.FM_E_INVAL
    r = L.fm_preprocess_mask(FAKE, 1, 1, FAKE, 1, 64, 0, FAKE, FAKE, 100, FAKE, FAKE, None)
    assert r == pv.FM_E_INVAL
    r = L.fm_preprocess_mask(FAKE, 1, 1, FAKE, 1, 64, 16, FAKE, FAKE, 4, FAKE, FAKE, None)
    assert r == pv.FM_E_WORKSPACE     # needs ceil(64/16) + 1 = 5 blocks
    r = L.fm_preprocess_mask(None, 1, 1, FAKE, 1, 64, 16, FAKE, FAKE, 100, FAKE, FAKE, None)
    assert r == pv.FM_E_INVAL


def test_worklist_rejects_on_host(pv):
    L = pv._lib
    lay = pv.workspace_layout(1000, 2, 3, 1, 16, 16, 0, True)
    args = lambda **kw: [kw.get("cu", FAKE), 2, 1000, 3, 16, 16, FAKE, FAKE, FAKE, 1, kw.get("S", 0), FAKE,
                         kw.get("items_cap", lay.item_cap), FAKE, FAKE, kw.get("map", None),
                         kw.get("map_cap", 0), FAKE, kw.get("scratch", lay.scratch_bytes), None]
    assert L.fm_build_worklist(*args(scratch=16)) == pv.FM_E_WORKSPACE
    assert L.fm_build_worklist(*args(items_cap=1)) == pv.FM_E_WORKSPACE
    assert L.fm_build_worklist(*args(map=FAKE, map_cap=1)) == pv.FM_E_WORKSPACE
    assert L.fm_build_worklist(*args(S=-1)) == pv.FM_E_INVAL
    assert L.fm_build_worklist(*args(cu=None)) == pv.FM_E_INVAL
    assert L.fm_worklist_scratch_size(1000, 2, 3, 16, 16, 0) == lay.scratch_bytes


def _bwd(pv, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, dout=FAKE, lse=FAKE, dtype=pv.FM_BF16, N=256, H=2, D=128,
             cu=FAKE, B=1, sv=FAKE, n_vec=1, causal=1, scale=0.1, dq=FAKE, dk=FAKE, dv=FAKE, ws=FAKE,
             ws_bytes=1 << 40)
    a.update(kw)
    rc = pv._lib.fm_attn_bwd(a["q"], a["k"], a["v"], a["out"], a["dout"], a["lse"], a["dtype"], a["N"], a["H"],
                             a["D"], a["cu"], a["B"], a["sv"], a["n_vec"], a["causal"], ctypes.c_float(a["scale"]),
                             a["dq"], a["dk"], a["dv"], a["ws"], a["ws_bytes"], None)
    return rc, pv._lib.fm_last_error().decode()


@pytest.mark.parametrize("kw,code", [
    (dict(n_vec=4), 1), (dict(n_vec=1, causal=0), 1), (dict(D=64), 2), (dict(dtype=1, D=32), 2),
    (dict(dtype=9), 2), (dict(scale=0.0), 1), (dict(scale=float("nan")), 1), (dict(cu=None), 1),
    (dict(dout=None), 1), (dict(lse=None), 1), (dict(dk=None), 1), (dict(ws=None), 1),
    (dict(ws_bytes=1024), 3), (dict(B=0), 1), (dict(H=0), 1), (dict(N=-1), 1),
])
def test_bwd_rejects_on_host(pv, kw, code):
    rc, msg = _bwd(pv, **kw)
    assert rc == code, msg
    assert msg


@pytest.mark.parametrize("streams,code", [
    ((None, FAKE, FAKE), 1),          # no dQ stream: the one-stream call is fm_attn_bwd
    ((FAKE, None, FAKE), 1),          # missing event
    ((FAKE, FAKE, None), 1),
])
def test_bwd_streams_rejects_on_host(pv, streams, code):
    """The two-stream backward needs the caller's second stream and both
    events; it rejects a missing one before enqueueing anything."""
    dq_stream, fork, join = streams
    rc = pv._lib.fm_attn_bwd_streams(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, pv.FM_BF16, 256, 2, 128, FAKE, 1, FAKE, 1, 1,
                                     ctypes.c_float(0.1), FAKE, FAKE, FAKE, FAKE, 1 << 40, ctypes.c_void_p(8192),
                                     dq_stream, fork, join)
    msg = pv._lib.fm_last_error().decode()
    assert rc == code, msg
    assert msg


def test_bwd_workspace_size(pv):
    """Header, kb_off, extrema at 64-key blocks, Delta fp32 [H][N]."""
    L = pv._lib
    n = L.fm_bwd_workspace_size(4352, 3, 2, 128, pv.FM_BF16)
    assert n >= 256 + 4 * 4 + (4352 // 64 + 3) * 32 + 2 * 4352 * 4 and n % 256 == 0
    assert L.fm_bwd_workspace_size(4352, 3, 2, 64, pv.FM_BF16) == 0
    assert L.fm_bwd_workspace_size(4352, 0, 2, 128, pv.FM_BF16) == 0
    assert L.fm_bwd_workspace_size(16, 1, 1, 32, pv.FM_F32) == 0


def _rope(pv, **kw):
    a = dict(q=FAKE, k=FAKE, dtype=pv.FM_BF16, N=64, Hq=2, Hk=1, D=128, cu=FAKE, B=1, cos=FAKE, sin=FAKE,
             max_pos=64, inverse=0, status=None)
    a.update(kw)
    rc = pv._lib.fm_rope_qk(a["q"], a["k"], a["dtype"], a["N"], a["Hq"], a["Hk"], a["D"], a["cu"], a["B"],
                            a["cos"], a["sin"], a["max_pos"], a["inverse"], a["status"], None)
    return rc, pv._lib.fm_last_error().decode()


@pytest.mark.parametrize("kw,code", [
    (dict(D=120), 2), (dict(D=8), 2), (dict(dtype=1, D=12), 2), (dict(D=1024), 2), (dict(dtype=5), 2),
    (dict(Hq=0, Hk=0), 1), (dict(Hq=-1), 1), (dict(B=0), 1), (dict(N=-1), 1), (dict(max_pos=0), 1),
    (dict(cu=None), 1), (dict(cos=None), 1), (dict(q=None), 1), (dict(q=ctypes.c_void_p(4104)), 1),
    (dict(sin=ctypes.c_void_p(4100)), 1),
])
def test_rope_rejects_on_host(pv, kw, code):
    rc, msg = _rope(pv, **kw)
    assert rc == code, msg
    assert msg
