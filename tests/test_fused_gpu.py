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
persistent launch on row-group shapes (items dealt to the XCDs by head, head
counts as hand-offs inside an XCD), checked against the oracle and the two
calls (bitwise with the tiled projection; with the split-K projection, whose
column groups it forms per XCD, up to the order of the fp32 chunk sums) over
head counts below, at and above the XCD count, both projection kinds and both
head sizes; repeated calls are bitwise equal and leave the workspace counters
at zero with no timed-out wait; the call on a side stream equals the call on
the default stream; shapes outside its scope are refused before anything is
launched.

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
        assert fd.attention_error(ws[fd.FUSED_SYNC_BYTES:],
                                  torch.cuda.current_stream().cuda_stream) == 0


def test_back_to_back_on_a_side_stream():
    fd = _fd()
    wl = synth.WORKLOADS["small_long_l1500"]()
    _banner("back to back, side stream")
    ref = _two_calls(fd, wl)
    run = G.GpuRun(wl, DEV)
    torch.cuda.synchronize()  # inputs uploaded before the side stream reads them
    _assert_same("side", 0, ref, _one_call(fd, wl, False, stream=torch.cuda.Stream(), run=run))


def _tiled_projection(wl):
    return wl.rows > 64 or wl.hid % 256 != 0


def _check_single_launch(fd, wl, name, reps=3):
    """Single-launch calls on one workspace against the two calls and the
    oracle.  The tiled projection's sums do not depend on the tile, so there
    every output is bitwise the two calls'; the split-K column groups are
    formed per XCD, so there Q, K and V may differ from the two calls' in the
    last bit (another order of the fp32 chunk sums) and the outputs are
    compared at the oracle tolerance.  Every call equals the first bitwise."""
    ref = _two_calls(fd, wl)
    ws = _workspace(fd, wl, ref[0].max_rows)
    oref = G.oracle_step(wl)
    first = None
    for rep in range(reps):  # the counters reset themselves between calls
        got = _one_call(fd, wl, True, ws)
        if _tiled_projection(wl):
            _assert_same(name, rep, ref, got)
        run, q, sm, out, mass = got
        assert torch.equal(sm, ref[2]), (name, rep, "slot mapping")
        G.assert_close(O.bf16_bits_to_f64(G.bits_of(q)), O.bf16_bits_to_f64(G.bits_of(ref[1])),
                       f"{name} Q vs the two calls")
        G.compare_cache(wl, oref, G.bits_of(run.cache.k_cache), G.bits_of(run.cache.v_cache),
                        wl.k_cache, wl.v_cache)
        G.assert_close(out.cpu().numpy(), oref["out"], f"{name} attention output")
        G.assert_close(mass.cpu().numpy().astype(np.float64), oref["mass"], f"{name} mass")
        G.assert_close(out.cpu().numpy(), ref[3].cpu().numpy().astype(np.float64),
                       f"{name} attention output vs the two calls")
        if first is None:
            first = got
        else:
            _assert_same(name, rep, first, got)
    assert fd.fused_step_error(ws) == 0
    # tickets, per-XCD and per-head counts reset; error word clear
    counters = ws[:fd.FUSED_SYNC_BYTES].view(torch.int32).cpu()
    assert int(counters.abs().sum()) == 0, counters.nonzero().flatten().tolist()


@pytest.mark.parametrize("name", ROW_GROUP_SHAPES)
def test_single_launch_against_the_two_calls_and_the_oracle(name):
    fd = _fd()
    wl = synth.WORKLOADS[name]()
    _banner(f"single launch {name}: {wl.rows} rows, batch {wl.batch}, {wl.num_heads} heads")
    _check_single_launch(fd, wl, name)


def _heads_off_the_xcd_count(kind):
    """Head counts that do not fill the XCDs evenly: 12 heads of 64 (four XCDs
    own two heads, four own one) through the split-K projection with a
    run-time chunk count, and 20 heads of 128 (XCDs owning three or two)
    through the tiled projection, whose column tiles straddle heads."""
    from synth import SeqSpec
    g = np.random.default_rng(41)
    if kind == "splitk_h12":
        specs = [SeqSpec(kv_len=200, window=(150, 16),
                         tracked=tuple(sorted(int(v) for v in g.choice(150, 8, replace=False)))),
                 SeqSpec(kv_len=97, window=(64, 20))]
        return synth.build("single_h12", 41, 768, 12, 64, 32, 1.0e4, specs, topb=8)
    specs = [SeqSpec(kv_len=300, window=(200, 32),
                     tracked=tuple(sorted(int(v) for v in g.choice(200, 24, replace=False)))),
             SeqSpec(kv_len=130, window=(96, 30)),
             SeqSpec(kv_len=64, window=(10, 20))]
    return synth.build("single_h20", 42, 512, 20, 128, 32, 5.0e5, specs, topb=8)


@pytest.mark.parametrize("kind", ["splitk_h12", "tiled_h20"])
def test_single_launch_head_counts_off_the_xcd_count(kind):
    fd = _fd()
    wl = _heads_off_the_xcd_count(kind)
    _banner(f"single launch {kind}: {wl.rows} rows, batch {wl.batch}, {wl.num_heads} heads")
    _check_single_launch(fd, wl, kind)


def test_single_launch_on_a_side_stream():
    """Outputs and the zero-filled workspace allocated in the side stream's
    order: bitwise the same call's results on the default stream, no
    timed-out wait."""
    fd = _fd()
    wl = synth.llada8b_b1()
    _banner("single launch, side stream")
    ref = _one_call(fd, wl, True)
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
