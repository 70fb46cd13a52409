"""GPU tests of the single-launch step (flash_cache_attention_step): bitwise the
results of flash_cache_step followed by scheduled_attention with the mass (the
phases run the same workgroup code), over both projection kinds (split-K at
<= 64 rows, tiled above), both head sizes, ragged sequences and the two-view
mask; repeated calls leave the workspace counters at zero with no timed-out
wait; the call on a side stream; shapes outside its scope are refused before
anything is launched.
Parity with the CPU oracle follows from the separate calls' parity tests and
is also checked directly on the batch-1 layer.
"""

import numpy as np
import pytest

import oracle as O
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from tests import gpu_util as G  # noqa: E402

DEV = "cuda:0"


def _fd():
    import kv_cache_attention_flash_amd as fd
    fd.load()
    return fd


def _banner(msg):
    print(f"[fused] {msg}", flush=True)


def _two_calls(fd, wl):
    run = G.GpuRun(wl, DEV)
    q, sm = fd.flash_cache_step(run.cache, run.x, run.w, run.cu, run.pos, run.slots, wl.rope_base)
    out, mass = fd.scheduled_attention(run.cache, q, run.cu, run.kv_len, wl.max_kv_len,
                                       run.max_rows, views=run.views, want_mass=True)
    torch.cuda.synchronize()
    return run, q, sm, out, mass


def _fused(fd, wl, workspace=None):
    run = G.GpuRun(wl, DEV)
    q, sm, out, mass = fd.flash_cache_attention_step(
        run.cache, run.x, run.w, run.cu, run.pos, run.slots, wl.rope_base, run.kv_len,
        wl.max_kv_len, run.max_rows, views=run.views, workspace=workspace)
    torch.cuda.synchronize()
    return run, q, sm, out, mass


@pytest.mark.parametrize("name", ["tiny_h256_l128", "llada8b_b1_l768", "small_d64_rows150",
                                  "small_ragged_b5", "small_verify_b3"])
def test_bitwise_equal_to_the_two_calls(name):
    fd = _fd()
    wl = synth.WORKLOADS[name]()
    _banner(f"{name}: {wl.rows} rows, batch {wl.batch}")
    r1, q1, sm1, o1, m1 = _two_calls(fd, wl)
    ws = torch.zeros((fd.fused_step_workspace_bytes(wl.batch, wl.rows, wl.num_heads, wl.head_dim,
                                                    wl.max_kv_len, r1.max_rows, wl.max_kv_len),),
                     dtype=torch.uint8, device=DEV)
    for rep in range(3):  # the counters reset themselves between calls
        r2, q2, sm2, o2, m2 = _fused(fd, wl, ws)
        assert torch.equal(q2, q1) and torch.equal(sm2, sm1), (name, rep, "projection")
        assert torch.equal(r2.cache.k_cache, r1.cache.k_cache), (name, rep, "K cache")
        assert torch.equal(r2.cache.v_cache, r1.cache.v_cache), (name, rep, "V cache")
        assert torch.equal(o2, o1), (name, rep, "attention output")
        assert torch.equal(m2, m1), (name, rep, "mass")
    counters = ws[:20].view(torch.int32).cpu().tolist()
    assert counters == [0, 0, 0, 0, 0], counters  # counts and ticket reset, error word clear


def test_on_a_side_stream():
    """The call on a stream other than torch's current one (its outputs and
    zero-filled workspace allocated in that stream's order): bitwise the two
    calls' results, no timed-out wait."""
    fd = _fd()
    wl = synth.llada8b_b1()
    _banner("side stream")
    r1, q1, sm1, o1, m1 = _two_calls(fd, wl)
    run = G.GpuRun(wl, DEV)
    torch.cuda.synchronize()  # inputs uploaded before the side stream reads them
    side = torch.cuda.Stream()
    q2, sm2, o2, m2 = fd.flash_cache_attention_step(
        run.cache, run.x, run.w, run.cu, run.pos, run.slots, wl.rope_base, run.kv_len,
        wl.max_kv_len, run.max_rows, views=run.views, stream=side)
    side.synchronize()
    assert torch.equal(q2, q1) and torch.equal(sm2, sm1)
    assert torch.equal(run.cache.k_cache, r1.cache.k_cache)
    assert torch.equal(o2, o1) and torch.equal(m2, m1)


def test_batch1_layer_against_the_oracle():
    fd = _fd()
    wl = synth.llada8b_b1()
    run, q, sm, out, mass = _fused(fd, wl)
    ref = G.oracle_step(wl)
    assert np.array_equal(sm.cpu().numpy(), ref["slot_mapping"])
    G.assert_close(O.bf16_bits_to_f64(G.bits_of(q)), O.bf16_bits_to_f64(ref["q"]), "Q")
    G.compare_cache(wl, ref, G.bits_of(run.cache.k_cache), G.bits_of(run.cache.v_cache),
                    wl.k_cache, wl.v_cache)
    G.assert_close(out.cpu().numpy(), ref["out"], "attention output")
    mh = mass.cpu().numpy().astype(np.float64)
    G.assert_close(mh, ref["mass"], "mass")
    idx = fd.track_topb(mass, run.kv_len, wl.topb)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy()[0], O.top_b(mh[0], int(wl.kv_len[0]), wl.topb))


@pytest.mark.parametrize("name", ["small_splitk_h1024", "llada8b_ragged_b32"])
def test_out_of_scope_shapes_are_refused(name):
    """A projection with a split reduction, or attention on the split path:
    refused on the host, nothing written."""
    fd = _fd()
    wl = synth.WORKLOADS[name]()
    run = G.GpuRun(wl, DEV)
    k0 = run.cache.k_cache.clone()
    with pytest.raises(fd.FdlError) as e:
        fd.flash_cache_attention_step(run.cache, run.x, run.w, run.cu, run.pos, run.slots,
                                      wl.rope_base, run.kv_len, wl.max_kv_len, run.max_rows)
    assert "unsupported" in str(e.value)
    torch.cuda.synchronize()
    assert torch.equal(run.cache.k_cache, k0)
