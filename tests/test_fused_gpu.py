"""GPU tests of the one-call step.

flash_cache_attention_step launches flash_cache_step's kernels and then
scheduled_attention's (with the mass) on one stream, for every shape: its
results are bitwise those of the two separate calls, over both projection
kinds (split-K at <= 64 rows, with and without a split reduction, tiled
above), both head sizes, ragged sequences, the two-view mask and every
attention path (row groups, split with scores on chip, split with exchanged
row statistics); repeated calls on one workspace agree; the call on a side
stream.

flash_cache_attention_step_single_launch runs the same step as one
persistent launch on row-group shapes: bitwise the two calls' results (the
phases run the same workgroup code), repeated calls leave the workspace
counters at zero with no timed-out wait, the call on a side stream; shapes
outside its scope are refused before anything is launched.

Parity with the CPU oracle follows from the separate calls' parity tests and
is also checked directly on the batch-1 layer for both forms.
"""

import numpy as np
import pytest

import oracle as O
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from tests import gpu_util as G  # noqa: E402

DEV = "cuda:0"

ROW_GROUP_SHAPES = ["tiny_h256_l128", "llada8b_b1_l768", "small_d64_rows150", "small_ragged_b5",
                    "small_verify_b3"]
EVERY_PATH_SHAPES = ROW_GROUP_SHAPES + ["small_splitk_h1024", "llada8b_ragged_b32",
                                        "small_long_l1500"]


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


def _one_call(fd, wl, single, workspace=None, stream=None, run=None):
    run = run or G.GpuRun(wl, DEV)
    fn = fd.flash_cache_attention_step_single_launch if single else fd.flash_cache_attention_step
    q, sm, out, mass = fn(run.cache, run.x, run.w, run.cu, run.pos, run.slots, wl.rope_base,
                          run.kv_len, wl.max_kv_len, run.max_rows, views=run.views,
                          workspace=workspace, stream=stream)
    if stream is None:
        torch.cuda.synchronize()
    else:
        stream.synchronize()
    return run, q, sm, out, mass


def _workspace(fd, wl, max_rows):
    return torch.zeros((fd.fused_step_workspace_bytes(wl.batch, wl.rows, wl.num_heads,
                                                      wl.head_dim, wl.max_kv_len, max_rows,
                                                      wl.max_kv_len),),
                       dtype=torch.uint8, device=DEV)


def _assert_same(name, rep, ref, got):
    r1, q1, sm1, o1, m1 = ref
    r2, q2, sm2, o2, m2 = got
    assert torch.equal(q2, q1) and torch.equal(sm2, sm1), (name, rep, "projection")
    assert torch.equal(r2.cache.k_cache, r1.cache.k_cache), (name, rep, "K cache")
    assert torch.equal(r2.cache.v_cache, r1.cache.v_cache), (name, rep, "V cache")
    assert torch.equal(o2, o1), (name, rep, "attention output")
    assert torch.equal(m2, m1), (name, rep, "mass")


@pytest.mark.parametrize("name", EVERY_PATH_SHAPES)
def test_back_to_back_equal_to_the_two_calls(name):
    fd = _fd()
    wl = synth.WORKLOADS[name]()
    path = fd.attention_path(wl.batch, wl.rows, wl.num_heads, wl.head_dim, wl.max_kv_len,
                             int(np.diff(wl.cu_rows).max()), wl.max_kv_len)
    _banner(f"back to back {name}: {wl.rows} rows, batch {wl.batch}, attention path {path}")
    ref = _two_calls(fd, wl)
    ws = _workspace(fd, wl, ref[0].max_rows)
    for rep in range(2):  # one workspace reused: nothing carries over
        _assert_same(name, rep, ref, _one_call(fd, wl, False, ws))
    if path == "split_mass_exchange" and wl.max_kv_len > 1024:  # splits that wait
        assert fd.attention_error(ws[256:], torch.cuda.current_stream().cuda_stream) == 0


def test_back_to_back_on_a_side_stream():
    fd = _fd()
    wl = synth.WORKLOADS["small_long_l1500"]()
    _banner("back to back, side stream")
    ref = _two_calls(fd, wl)
    run = G.GpuRun(wl, DEV)
    torch.cuda.synchronize()  # inputs uploaded before the side stream reads them
    _assert_same("side", 0, ref, _one_call(fd, wl, False, stream=torch.cuda.Stream(), run=run))


@pytest.mark.parametrize("name", ROW_GROUP_SHAPES)
def test_single_launch_equal_to_the_two_calls(name):
    fd = _fd()
    wl = synth.WORKLOADS[name]()
    _banner(f"single launch {name}: {wl.rows} rows, batch {wl.batch}")
    ref = _two_calls(fd, wl)
    ws = _workspace(fd, wl, ref[0].max_rows)
    for rep in range(3):  # the counters reset themselves between calls
        _assert_same(name, rep, ref, _one_call(fd, wl, True, ws))
    counters = ws[:20].view(torch.int32).cpu().tolist()
    assert counters == [0, 0, 0, 0, 0], counters  # counts and ticket reset, error word clear


def test_single_launch_on_a_side_stream():
    """Outputs and the zero-filled workspace allocated in the side stream's
    order: bitwise the two calls' results, no timed-out wait."""
    fd = _fd()
    wl = synth.llada8b_b1()
    _banner("single launch, side stream")
    ref = _two_calls(fd, wl)
    run = G.GpuRun(wl, DEV)
    torch.cuda.synchronize()
    _assert_same("side", 0, ref, _one_call(fd, wl, True, stream=torch.cuda.Stream(), run=run))


@pytest.mark.parametrize("single", [False, True])
def test_batch1_layer_against_the_oracle(single):
    fd = _fd()
    wl = synth.llada8b_b1()
    run, q, sm, out, mass = _one_call(fd, wl, single)
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
def test_single_launch_refuses_out_of_scope_shapes(name):
    """A projection with a split reduction, or attention on the split path:
    refused on the host, nothing written."""
    fd = _fd()
    wl = synth.WORKLOADS[name]()
    run = G.GpuRun(wl, DEV)
    k0 = run.cache.k_cache.clone()
    with pytest.raises(fd.FdlError) as e:
        fd.flash_cache_attention_step_single_launch(run.cache, run.x, run.w, run.cu, run.pos,
                                                    run.slots, wl.rope_base, run.kv_len,
                                                    wl.max_kv_len, run.max_rows)
    assert "unsupported" in str(e.value)
    torch.cuda.synchronize()
    assert torch.equal(run.cache.k_cache, k0)
