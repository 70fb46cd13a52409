"""GPU tests of the FDL_DEBUG=1 index checks: with the variable set, calls
whose device index arrays are out of range (a logical slot past the block
table row, a negative position, two rows on one physical slot, a block id
outside the pool, a negative length, decreasing row offsets) return
FDL_EINVAL before launching anything, and valid calls give the same results
as without the variable.  Every bad input here is refused on the host; none
reaches a kernel.
"""

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from tests import gpu_util as G  # noqa: E402

DEV = "cuda:0"


def _fd():
    import kv_cache_attention_flash_amd as fd
    fd.load()
    return fd


def _refused(fd, fn):
    with pytest.raises(fd.FdlError) as e:
        fn()
    assert e.value.status == 1, str(e.value)  # FDL_EINVAL


def test_debug_checks_refuse_bad_indices(monkeypatch):
    fd = _fd()
    wl = synth.WORKLOADS["small_ragged_b5"]()
    print(f"[debug] {wl.name}: batch {wl.batch}, {wl.rows} rows", flush=True)
    run = G.GpuRun(wl, DEV)
    q0, sm0 = fd.flash_cache_step(run.cache, run.x, run.w, run.cu, run.pos, run.slots, wl.rope_base)
    o0, m0 = fd.scheduled_attention(run.cache, q0, run.cu, run.kv_len, wl.max_kv_len, run.max_rows,
                                    want_mass=True)
    torch.cuda.synchronize()
    k_ref, v_ref = run.cache.k_cache.clone(), run.cache.v_cache.clone()

    monkeypatch.setenv("FDL_DEBUG", "1")
    # valid inputs: accepted, same results
    q1, sm1 = fd.flash_cache_step(run.cache, run.x, run.w, run.cu, run.pos, run.slots, wl.rope_base)
    o1, m1 = fd.scheduled_attention(run.cache, q1, run.cu, run.kv_len, wl.max_kv_len, run.max_rows,
                                    want_mass=True)
    torch.cuda.synchronize()
    act = int(wl.cu_rows[-1])
    assert torch.equal(q1[:act], q0[:act]) and torch.equal(sm1[:act], sm0[:act])
    assert torch.equal(o1[:act], o0[:act]) and torch.equal(m1, m0)

    cu = wl.cu_rows
    b2 = next(b for b in range(wl.batch) if cu[b + 1] - cu[b] >= 2)  # a sequence with 2+ rows
    r0 = int(cu[b2])
    fc = lambda cache=run.cache, cu_t=run.cu, pos=run.pos, slots=run.slots: fd.flash_cache_step(
        cache, run.x, run.w, cu_t, pos, slots, wl.rope_base)
    bad = run.slots.clone()
    bad[r0] = wl.max_blocks * wl.block_size  # past the block-table row
    _refused(fd, lambda: fc(slots=bad))
    dup = run.slots.clone()
    dup[r0 + 1] = dup[r0]  # two rows on one physical slot
    _refused(fd, lambda: fc(slots=dup))
    neg = run.pos.clone()
    neg[r0] = -1
    _refused(fd, lambda: fc(pos=neg))
    cu_bad = run.cu.clone()
    cu_bad[1], cu_bad[2] = cu_bad[2], cu_bad[1]  # decreasing offsets
    if int(cu_bad[1]) != int(cu_bad[2]):
        _refused(fd, lambda: fc(cu_t=cu_bad))
    # a block id outside the pool, in a page both calls use
    bt = wl.block_table.copy()
    slot = int(wl.slots[r0])
    bt[b2, slot // wl.block_size] = wl.num_blocks
    cache_bad = fd.PagedKVCache(run.cache.k_cache, run.cache.v_cache, G.i32(bt, DEV))
    _refused(fd, lambda: fc(cache=cache_bad))
    _refused(fd, lambda: fd.scheduled_attention(cache_bad, q1, run.cu, run.kv_len, wl.max_kv_len,
                                                run.max_rows, want_mass=True))
    kv_bad = run.kv_len.clone()
    kv_bad[0] = -5
    _refused(fd, lambda: fd.scheduled_attention(run.cache, q1, run.cu, kv_bad, wl.max_kv_len,
                                                run.max_rows))
    # a sequence with more rows than max_rows_per_seq (its extra rows would
    # otherwise be left unwritten)
    _refused(fd, lambda: fd.scheduled_attention(run.cache, q1, run.cu, run.kv_len,
                                                wl.max_kv_len, run.max_rows - 1, want_mass=True))
    torch.cuda.synchronize()
    # nothing was written by the refused calls
    assert torch.equal(run.cache.k_cache, k_ref) and torch.equal(run.cache.v_cache, v_ref)


def test_debug_checks_refuse_bad_two_view_descriptors(monkeypatch):
    """Two-view descriptors that break window_start + window_len <=
    draft_slot_start or draft_slot_start + window_len <= kv_len, or hold a
    negative entry, are refused on the host; valid ones pass."""
    fd = _fd()
    wl = synth.WORKLOADS["small_verify_b3"]()
    print(f"[debug] {wl.name}: two-view descriptors", flush=True)
    run = G.GpuRun(wl, DEV)
    q, _ = fd.flash_cache_step(run.cache, run.x, run.w, run.cu, run.pos, run.slots, wl.rope_base)
    o0, _ = fd.scheduled_attention(run.cache, q, run.cu, run.kv_len, wl.max_kv_len, run.max_rows,
                                   views=run.views)
    torch.cuda.synchronize()
    monkeypatch.setenv("FDL_DEBUG", "1")
    o1, _ = fd.scheduled_attention(run.cache, q, run.cu, run.kv_len, wl.max_kv_len, run.max_rows,
                                   views=run.views)
    torch.cuda.synchronize()
    assert torch.equal(o1, o0)
    w0, wlen, d0 = (int(v) for v in wl.views[0])
    for bad_row in ([d0 - wlen + 1, wlen, d0],            # window runs into the draft slots
                    [w0, wlen, int(wl.kv_len[0]) - wlen + 1],  # draft slots past kv_len
                    [-1, wlen, d0]):                      # negative entry
        v = wl.views.copy()
        v[0] = bad_row
        vt = G.i32(v, DEV)
        _refused(fd, lambda: fd.scheduled_attention(run.cache, q, run.cu, run.kv_len,
                                                    wl.max_kv_len, run.max_rows, views=vt))
