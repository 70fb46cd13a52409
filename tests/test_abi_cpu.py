"""The C-ABI library loads on a machine without a GPU, exports every function
include/fdllm.h declares, and rejects bad arguments on the host before any HIP
call.  No GPU is touched here."""

import ctypes
import os
import re

import pytest

from kv_cache_attention_flash_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "fdllm.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in {"defined"}))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_header_lists_the_four_calls():
    names = declared_functions()
    for n in ("flash_cache_step", "scheduled_attention", "track_topb", "verify_accept",
              "fdl_attention_workspace_bytes", "fdl_flash_cache_workspace_bytes",
              "fdl_status_string", "fdl_last_hip_error",
              "fdl_version"):
        assert n in names, names


def test_every_declared_symbol_is_exported(lib):
    for n in declared_functions():
        assert hasattr(lib, n), n
    assert set(declared_functions()) == set(_lib.EXPORTS)


def test_status_strings(lib):
    for code in range(6):
        s = lib.fdl_status_string(code).decode()
        assert s and s != "unknown status"
    assert lib.fdl_status_string(99).decode() == "unknown status"
    assert b"gfx950" in lib.fdl_version()


def _cache(h=4, d=64, bs=32, nb=4, mb=4, k=0x1000, v=0x2000, bt=0x3000):
    return _lib.KVCacheStruct(h, d, bs, nb, mb, k, v, bt)


def test_flash_cache_step_validation(lib):
    fake = 0x10000
    ws = lib.fdl_flash_cache_workspace_bytes(4, 256, 4, 64)
    args = lambda c, hid=256, batch=1, rows=4, base=1e4, wsb=ws: lib.flash_cache_step(
        ctypes.byref(c), fake, hid, fake, batch, rows, fake, fake, fake, base, fake, None, fake,
        wsb, None)
    assert args(_cache(d=96)) == _lib.FDL_EUNSUPPORTED
    assert args(_cache(bs=48)) == _lib.FDL_EUNSUPPORTED
    assert args(_cache(), hid=200) == _lib.FDL_EUNSUPPORTED
    assert args(_cache(), hid=-128) == _lib.FDL_EINVAL
    assert args(_cache(), base=0.0) == _lib.FDL_EINVAL
    assert args(_cache(), base=float("nan")) == _lib.FDL_EINVAL
    assert args(_cache(h=0)) == _lib.FDL_EINVAL
    assert args(_cache(bt=0)) == _lib.FDL_EINVAL
    assert args(_cache(k=0)) == _lib.FDL_EINVAL
    assert args(_cache(), rows=-1) == _lib.FDL_EINVAL
    # X, W, Q and the pools are read and written in 16-byte pieces
    for at in range(3):
        ptrs = [fake, fake, fake]
        ptrs[at] = fake + 8
        assert lib.flash_cache_step(ctypes.byref(_cache()), ptrs[0], 256, ptrs[1], 1, 4, fake,
                                    fake, fake, 1e4, ptrs[2], None, fake, ws,
                                    None) == _lib.FDL_EINVAL
    assert args(_cache(k=fake + 2)) == _lib.FDL_EINVAL
    # empty calls are no-ops and touch nothing
    assert args(_cache(), rows=0) == _lib.FDL_OK
    assert args(_cache(), batch=0) == _lib.FDL_OK
    assert lib.flash_cache_step(ctypes.byref(_cache()), None, 256, fake, 1, 3, fake, fake, fake,
                                1e4, fake, None, fake, ws, None) == _lib.FDL_EINVAL
    assert lib.flash_cache_step(None, fake, 256, fake, 1, 3, fake, fake, fake, 1e4, fake, None,
                                fake, ws, None) == _lib.FDL_EINVAL
    # a narrow layer with few rows splits its reduction and needs scratch
    ws2 = lib.fdl_flash_cache_workspace_bytes(40, 1024, 2, 128)
    assert ws2 > 0
    c2 = _cache(h=2, d=128)
    assert lib.flash_cache_step(ctypes.byref(c2), fake, 1024, fake, 1, 40, fake, fake, fake, 1e4,
                                fake, None, fake, ws2 - 1, None) == _lib.FDL_EWORKSPACE
    assert lib.flash_cache_step(ctypes.byref(c2), fake, 1024, fake, 1, 40, fake, fake, fake, 1e4,
                                fake, None, None, ws2, None) == _lib.FDL_EWORKSPACE
    assert lib.fdl_flash_cache_workspace_bytes(65, 4096, 32, 128) == 0   # tiled kernel
    assert lib.fdl_flash_cache_workspace_bytes(-1, 4096, 32, 128) == 0


def test_unfused_ablation_validation(lib):
    """The unfused ablation validates like the fused step and needs its fp32
    intermediate and staging buffers in the workspace."""
    fake = 0x10000
    r, hid, h, d = 64, 4096, 32, 128
    ws = lib.fdl_flash_cache_unfused_workspace_bytes(r, hid, h, d)
    assert ws >= r * 3 * h * d * 4 + 2 * r * h * d * 2      # fp32 Y + bf16 K/V staging
    assert lib.fdl_flash_cache_unfused_workspace_bytes(-1, hid, h, d) == 0
    c = _cache(h=h, d=d)
    call = lambda wsb, wsp=fake, hid_=hid, rows=r: lib.flash_cache_step_unfused(
        ctypes.byref(c), fake, hid_, fake, 1, rows, fake, fake, fake, 5e5, fake, None, wsp, wsb,
        None)
    assert call(ws - 1) == _lib.FDL_EWORKSPACE
    assert call(ws, wsp=None) == _lib.FDL_EWORKSPACE
    assert call(ws, hid_=200) == _lib.FDL_EUNSUPPORTED
    assert call(ws, rows=0) == _lib.FDL_OK


def test_attention_validation_and_workspace(lib):
    fake = 0x10000
    ws = lib.fdl_attention_workspace_bytes(1, 64, 32, 128, 768, 64, 768)
    assert ws > 0
    # without the mass the split partials still need scratch at this shape
    assert lib.fdl_attention_workspace_bytes(1, 64, 32, 128, 768, 64, 0) > 0
    assert lib.fdl_attention_workspace_bytes(-1, 64, 32, 128, 768, 64, 0) == 0
    c = _cache(h=32, d=128, nb=24, mb=24)
    call = lambda **kw: lib.scheduled_attention(
        ctypes.byref(kw.get("c", c)), fake, kw.get("batch", 1), kw.get("rows", 64), fake, fake,
        kw.get("max_kv", 768), kw.get("max_rows", 64), None, kw.get("scale", 0.0), fake,
        kw.get("mass", fake), kw.get("stride", 768), kw.get("ws", fake), kw.get("wsb", ws), None)
    assert call(wsb=ws - 1) == _lib.FDL_EWORKSPACE
    assert call(ws=None) == _lib.FDL_EWORKSPACE
    assert call(stride=700) == _lib.FDL_EINVAL         # mass stride below max_kv_len
    assert call(max_kv=24 * 32 + 1) == _lib.FDL_EINVAL  # exceeds what the block table can map
    assert call(scale=-1.0) == _lib.FDL_EINVAL
    assert call(max_rows=0) == _lib.FDL_EINVAL
    assert call(c=_cache(h=32, d=80)) == _lib.FDL_EUNSUPPORTED
    assert call(batch=0) == _lib.FDL_OK


def test_topb_and_verify_validation(lib):
    fake = 0x10000
    assert lib.track_topb(fake, 128, fake, 1, 0, fake, None) == _lib.FDL_EINVAL
    assert lib.track_topb(fake, 0, fake, 1, 8, fake, None) == _lib.FDL_EINVAL
    assert lib.track_topb(None, 128, fake, 1, 8, fake, None) == _lib.FDL_EINVAL
    assert lib.track_topb(fake, 128, fake, 0, 8, fake, None) == _lib.FDL_OK
    assert lib.verify_accept(fake, fake, fake, -1, 4, 0.9, fake, None) == _lib.FDL_EINVAL
    assert lib.verify_accept(None, fake, fake, 2, 4, 0.9, fake, None) == _lib.FDL_EINVAL
    assert lib.verify_accept(fake, fake, fake, 2, 4, 0.9, None, None) == _lib.FDL_EINVAL
    assert lib.verify_accept(fake, fake, fake, 0, 4, 0.9, fake, None) == _lib.FDL_OK


def test_decode_plan_validation(lib):
    fake = 0x10000
    def plan(batch=2, w=16, bs=32, k=2, step=1, tracked=fake, topb=8, acc=fake, front=fake,
             cu=fake, pos=fake, slots=fake, cap=None):
        cap = batch * (w + topb) if cap is None else cap
        return lib.decode_plan(batch, fake, w, bs, k, step, tracked, topb, acc, front, cu, pos,
                               slots, None, cap, None)
    assert plan(w=0) == _lib.FDL_EINVAL
    assert plan(bs=0) == _lib.FDL_EINVAL
    assert plan(k=-1) == _lib.FDL_EINVAL
    assert plan(step=-1) == _lib.FDL_EINVAL
    assert plan(topb=-1) == _lib.FDL_EINVAL
    assert plan(batch=-1) == _lib.FDL_EINVAL
    assert plan(cap=2 * 24 - 1) == _lib.FDL_EINVAL          # capacity below batch * (W + topb)
    assert plan(batch=4097) == _lib.FDL_EUNSUPPORTED        # one workgroup plans at most 4096
    assert plan(tracked=None) == _lib.FDL_EINVAL            # topb > 0 needs the tracked set
    assert plan(acc=None) == _lib.FDL_EINVAL                # step > 0 reads accept lengths
    assert plan(front=None) == _lib.FDL_EINVAL
    assert plan(cu=None) == _lib.FDL_EINVAL
    assert plan(pos=None) == _lib.FDL_EINVAL
    assert plan(slots=None) == _lib.FDL_EINVAL
    assert plan(batch=0) == _lib.FDL_OK


def test_gather_hidden_validation(lib):
    fake = 0x10000
    def gather(batch=2, cap=10, max_len=64, hid=256, hc=fake, hm=fake, x=fake, cu=fake):
        return lib.gather_hidden(batch, cap, cu, fake, fake, hc, hm, max_len, hid, x, None)
    assert gather(hid=100) == _lib.FDL_EINVAL               # not a multiple of 8
    assert gather(hid=0) == _lib.FDL_EINVAL
    assert gather(max_len=0) == _lib.FDL_EINVAL
    assert gather(batch=-1) == _lib.FDL_EINVAL
    assert gather(hc=None) == _lib.FDL_EINVAL
    assert gather(cu=None) == _lib.FDL_EINVAL
    assert gather(hm=fake + 8) == _lib.FDL_EINVAL           # tables must be 16-byte aligned
    assert gather(x=fake + 2) == _lib.FDL_EINVAL
    assert gather(batch=0) == _lib.FDL_OK
    assert gather(cap=0) == _lib.FDL_OK


def test_lm_head_validation(lib):
    fake = 0x10000
    ws = lib.fdl_lm_head_workspace_bytes(4, 1000)
    assert ws > 0 and lib.fdl_lm_head_workspace_bytes(-1, 10) == 0
    def call(rows=4, vocab=1000, hid=256, h=fake, w=fake, tok=fake, conf=fake, wsp=fake, wsb=ws):
        return lib.lm_head_confidence(h, w, rows, vocab, hid, tok, conf, wsp, wsb, None)
    assert call(hid=100) == _lib.FDL_EUNSUPPORTED            # not a multiple of 32
    assert call(hid=65536 + 32) == _lib.FDL_EUNSUPPORTED
    assert call(vocab=0) == _lib.FDL_EINVAL
    assert call(rows=-1) == _lib.FDL_EINVAL
    assert call(h=None) == _lib.FDL_EINVAL
    assert call(conf=None) == _lib.FDL_EINVAL
    assert call(wsb=ws - 1) == _lib.FDL_EWORKSPACE
    assert call(wsp=None) == _lib.FDL_EWORKSPACE
    assert call(rows=0) == _lib.FDL_OK


def test_fused_step_validation(lib):
    """Host-side refusals of the one-call step and of its single-launch form
    (nothing is launched)."""
    fake = 0x10000
    c = _cache(h=2, d=128, bs=32, nb=4, mb=4)
    ws = lib.fdl_fused_step_workspace_bytes(1, 40, 2, 128, 96, 40, 96)
    assert ws >= 256 and lib.fdl_fused_step_workspace_bytes(1, 40, 2, 128, 96, 40, 0) == 0
    def call(fn, hid=1024, mass=fake, wsb=ws, rows=40):
        return fn(ctypes.byref(c), fake, hid, fake, 1, rows, fake, fake, fake, 1e4, fake, None,
                  fake, 96, 40, None, 0.0, fake, mass, 96, fake, wsb, None)
    for fn in (lib.flash_cache_attention_step, lib.flash_cache_attention_step_single_launch):
        assert call(fn, mass=None) == _lib.FDL_EINVAL      # the step always forms the mass
        assert call(fn, wsb=16) == _lib.FDL_EWORKSPACE
        assert call(fn, hid=200) == _lib.FDL_EUNSUPPORTED   # as flash_cache_step
    assert call(lib.flash_cache_attention_step, wsb=ws - 1) == _lib.FDL_EWORKSPACE
    # a narrow layer at 40 rows splits its projection's reduction: not one launch
    assert call(lib.flash_cache_attention_step_single_launch) == _lib.FDL_EUNSUPPORTED


def test_attention_path_selection(lib):
    """The planner's choice for the workload shapes (host only)."""
    import kv_cache_attention_flash_amd as fd
    # batch-1 layer, cache 768, mass: row groups
    assert fd.attention_path(1, 64, 32, 128, 768, 64, 768) == "row_groups"
    # batch 32 ragged up to 1024 keys, mass: scores on chip, one split per sequence
    assert fd.attention_path(32, 2048, 32, 128, 1024, 64, 1024) == "split_mass_exchange"
    # two-view batch 8, no mass: split path with merges
    assert fd.attention_path(8, 512, 32, 128, 1056, 64, 0) == "split"
    # 32-layer stack's layer: batch 16, cache 4096, 512 units: second pass over K
    assert fd.attention_path(16, 1024, 32, 128, 4096, 64, 4096) == "split_mass_reread"
    # long caches with few units: splits exchanging row statistics
    assert fd.attention_path(2, 48, 2, 64, 1500, 24, 1500) == "split_mass_exchange"
    assert lib.fdl_attention_path(-1, 0, 1, 64, 0, 0, 0) == 0
