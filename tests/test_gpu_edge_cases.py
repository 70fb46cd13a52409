"""GPU edge cases, reproducibility and structural invariants of the HIP path."""

import numpy as np
import pytest

import oracle as O
import synth
from synth import SeqSpec

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

from tests import gpu_util as G  # noqa: E402
from tests.test_parity_gpu import full_check, _banner  # noqa: E402


def _fd():
    import kv_cache_attention_flash_amd as fd
    fd.load()
    return fd


def test_ragged_edges():
    """A sequence with no active rows, one with a single cached slot, one shorter
    than the tracking budget, one not a multiple of the block size."""
    _banner("edges: empty sequence, kv_len 1, kv_len < B, ragged tail")
    specs = [SeqSpec(kv_len=40), SeqSpec(kv_len=1, window=(0, 1)),
             SeqSpec(kv_len=5, window=(3, 2)), SeqSpec(kv_len=70, window=(33, 16), tracked=(1, 2, 60))]
    wl = synth.build("edges", 21, 128, 2, 64, 32, 1.0e4, specs, topb=8)
    run, _ = full_check(wl)
    idx = run.idx.cpu().numpy()
    assert list(idx[1]) == [0] + [-1] * 7
    assert list(idx[2]) == [0, 1, 2, 3, 4, -1, -1, -1]
    assert np.all(run.mass.cpu().numpy()[0] == 0.0)  # no rows: no mass


def test_block_size_64_and_d128():
    _banner("block size 64, head_dim 128")
    g = np.random.default_rng(5)
    specs = [SeqSpec(kv_len=130, window=(64, 32), tracked=(0, 5, 9)),
             SeqSpec(kv_len=64, window=(7, 20)),
             SeqSpec(kv_len=200, window=(128, 32), tracked=tuple(sorted(g.choice(128, 30, replace=False))))]
    wl = synth.build("bs64", 22, 256, 3, 128, 64, 5.0e5, specs, topb=16)
    full_check(wl)


def test_block_size_256_both_attention_paths():
    """The largest page size: tiles are runs of one page, a page holds eight
    32-key tiles, lengths end inside a page.  Row-group path (head_dim 128,
    short cache) and split path (head_dim 64, a cache past 1024 keys)."""
    _banner("block size 256: row-group path")
    g = np.random.default_rng(7)
    specs = [SeqSpec(kv_len=600, window=(512, 32),
                     tracked=tuple(sorted(int(x) for x in g.choice(512, 24, replace=False)))),
             SeqSpec(kv_len=300, window=(200, 17)),
             SeqSpec(kv_len=257, window=(256, 1), tracked=(0, 255))]
    full_check(synth.build("bs256", 23, 256, 3, 128, 256, 5.0e5, specs, topb=16))
    _banner("block size 256: split path")
    specs = [SeqSpec(kv_len=1300, window=(1024, 32), tracked=(1, 500, 1000)),
             SeqSpec(kv_len=520, window=(256, 32))]
    full_check(synth.build("bs256_long", 24, 256, 2, 64, 256, 1.0e4, specs, topb=8))


def test_empty_calls():
    fd = _fd()
    dev = "cuda:0"
    wl = synth.tiny_h256()
    run = G.GpuRun(wl, dev)
    x0 = run.x[:0]
    q, sm = fd.flash_cache_step(run.cache, x0, run.w, G.i32([0, 0], dev), G.i32([], dev),
                                G.i32([], dev), 1e4)
    assert q.shape[0] == 0
    # rows = 0 with mass requested: mass is all zeros
    mass = torch.full((1, 128), 7.0, device=dev)
    out, m = fd.scheduled_attention(run.cache, q, G.i32([0, 0], dev), run.kv_len, 128, 0, mass=mass)
    torch.cuda.synchronize()
    assert torch.all(m == 0)


def test_deterministic_reruns():
    _banner("bitwise reruns")
    wl = synth.llada8b_b1()
    a = G.GpuRun(wl).step()
    b = G.GpuRun(wl).step()
    for f in ("q", "out", "mass", "idx", "slot_mapping"):
        assert torch.equal(getattr(a, f), getattr(b, f)), f
    assert torch.equal(a.cache.k_cache, b.cache.k_cache)


def _longest_cache_workload():
    """One sequence at the page limit (1024 pages of 64 slots, 65535 keys
    cached), 2 heads x 64, window in the middle and tracked rows spread over
    the whole cache, top-16."""
    g = np.random.default_rng(13)
    L = 1024 * 64 - 1
    w0 = 40000
    tracked = tuple(sorted(int(p) for p in g.choice(w0, 24, replace=False)))
    spec = SeqSpec(kv_len=L, window=(w0, 16), tracked=tracked)
    return synth.build("longest_l65535", 27, 256, 2, 64, 64, 5.0e5, [spec], topb=16)


@pytest.mark.parametrize("want_mass", [True, False])
def test_cache_at_the_page_limit(want_mass):
    """The longest cache the ABI takes (1024 pages): with the mass, 64
    splits exchanging row statistics; without it, 64 splits merged in order.
    Element-wise against the oracle (with the mass: top-B too)."""
    import kv_cache_attention_flash_amd as fd
    fd.load()
    wl = _longest_cache_workload()
    path = fd.attention_path(wl.batch, wl.rows, wl.num_heads, wl.head_dim, wl.max_kv_len,
                             int(np.diff(wl.cu_rows).max()), wl.max_kv_len if want_mass else 0)
    _banner(f"page limit: L {int(wl.kv_len[0])}, rows {wl.rows}, mass {want_mass}, path {path}")
    assert path == ("split_mass_exchange" if want_mass else "split")
    run = G.GpuRun(wl, "cuda:0")
    if want_mass:
        run.step()
        full_check(wl, run=run)
        return
    q, sm = fd.flash_cache_step(run.cache, run.x, run.w, run.cu, run.pos, run.slots, wl.rope_base)
    out, _ = fd.scheduled_attention(run.cache, q, run.cu, run.kv_len, wl.max_kv_len, run.max_rows,
                                    views=run.views)
    torch.cuda.synchronize()
    ref = G.oracle_step(wl)
    G.assert_close(out.cpu().numpy(), ref["out"], "attention output (no mass)")


@pytest.mark.parametrize("name", ["small_long_l1500", "long_b4_l4096", "long_b5_h32_rounds"])
def test_exchange_path_reruns_and_workspace(name):
    """The split path whose splits exchange row statistics (caches past 1024
    keys, mass asked for): bitwise the same results on three calls in a row
    through one workspace that starts filled with garbage (the call clears its
    own counters), and on a fresh workspace; the error word stays 0; the
    output and mass agree with the oracle."""
    import kv_cache_attention_flash_amd as fd
    fd.load()
    dev = "cuda:0"
    if name == "long_b4_l4096":
        g = np.random.default_rng(7)
        specs = [SeqSpec(kv_len=4096 - 37 * b, window=(int(g.integers(32, 3000)), 32),
                         tracked=tuple(sorted(int(p) for p in g.choice(32, 32, replace=False))))
                 for b in range(4)]
        wl = synth.build(name, 25, 512, 8, 128, 32, 5.0e5, specs, topb=32)
    elif name == "long_b5_h32_rounds":
        # 5 x 32 heads = 160 units of up to four 1024-key splits: more
        # workgroups than the GPU holds at once, so splits wait across rounds
        g = np.random.default_rng(11)
        specs = []
        for _ in range(5):
            L = int(g.integers(3073, 4097))
            w0 = int(g.integers(32, L - 64))
            specs.append(SeqSpec(kv_len=L, window=(w0, 32),
                                 tracked=tuple(sorted(int(p) for p in g.choice(w0, 32,
                                                                               replace=False)))))
        wl = synth.build(name, 26, 512, 32, 64, 32, 5.0e5, specs, topb=32)
    else:
        wl = synth.WORKLOADS[name]()
    _banner(f"exchange path {name}: lengths {wl.kv_len.tolist()}")
    run = G.GpuRun(wl, dev)
    assert fd.attention_path(wl.batch, wl.rows, wl.num_heads, wl.head_dim, wl.max_kv_len,
                             run.max_rows, wl.max_kv_len) == "split_mass_exchange"
    q, sm = fd.flash_cache_step(run.cache, run.x, run.w, run.cu, run.pos, run.slots, wl.rope_base)
    need = fd.attention_workspace_bytes(wl.batch, wl.rows, wl.num_heads, wl.head_dim,
                                        wl.max_kv_len, run.max_rows, wl.max_kv_len)
    ws = torch.full((need,), 0x5A, dtype=torch.uint8, device=dev)
    ws[fd.ATTENTION_ERROR_OFFSET:fd.ATTENTION_ERROR_OFFSET + 4] = 0
    outs = []
    for _ in range(3):
        o, m = fd.scheduled_attention(run.cache, q, run.cu, run.kv_len, wl.max_kv_len,
                                      run.max_rows, views=run.views, want_mass=True,
                                      workspace=ws)
        torch.cuda.synchronize()
        outs.append((o.clone(), m.clone()))
    assert fd.attention_error(ws) == 0
    o4, m4 = fd.scheduled_attention(run.cache, q, run.cu, run.kv_len, wl.max_kv_len,
                                    run.max_rows, views=run.views, want_mass=True)
    torch.cuda.synchronize()
    for o, m in outs[1:] + [(o4, m4)]:
        assert torch.equal(o, outs[0][0]) and torch.equal(m, outs[0][1])
    idx = fd.track_topb(m4, run.kv_len, wl.topb)
    torch.cuda.synchronize()
    run.q, run.out, run.mass, run.idx, run.slot_mapping = q, o4, m4, idx, sm
    full_check(wl, run=run)


def test_scores_on_chip_loop_with_empty_row_tiles():
    """Caches up to 1024 keys with the mass and more units than CUs: the
    scores-on-chip kernel loops over units per workgroup, dealt longest cache
    first.  Some sequences have two row tiles and some one, so the second row
    tile of the short ones is an empty unit that the loop skips; one sequence
    has a 40-key cache and one a cache on a tile boundary.  Element-wise
    against the oracle, and bitwise equal on a rerun."""
    import kv_cache_attention_flash_amd as fd
    fd.load()
    g = np.random.default_rng(41)
    specs = []
    for i in range(10):
        L = [40, 1024][i] if i < 2 else int(g.integers(300, 1025))
        w = int(min(L, 48 if i % 3 == 0 else 16))
        w0 = int(g.integers(0, L - w + 1))
        pool = [q for q in range(L) if not (w0 <= q < w0 + w)]
        nt = int(min(len(pool), 40 if i % 3 == 0 else 8))
        tr = tuple(sorted(int(q) for q in g.choice(pool, size=nt, replace=False))) if nt else ()
        specs.append(SeqSpec(kv_len=L, window=(w0, w), tracked=tr))
    wl = synth.build("xmass_loop", 29, 256, 32, 128, 32, 5.0e5, specs, topb=16)
    run = G.GpuRun(wl, "cuda:0")
    rows = np.diff(wl.cu_rows)
    path = fd.attention_path(wl.batch, wl.rows, wl.num_heads, wl.head_dim, wl.max_kv_len,
                             run.max_rows, wl.max_kv_len)
    _banner(f"scores-on-chip loop: rows per sequence {rows.tolist()}, "
            f"lengths {wl.kv_len.tolist()}, path {path}")
    assert path == "split_mass_exchange" and rows.max() > 64 and rows.min() <= 64
    run.step()
    o1, m1 = run.out.clone(), run.mass.clone()
    full_check(wl, run=run)
    o2, m2 = fd.scheduled_attention(run.cache, run.q, run.cu, run.kv_len, wl.max_kv_len,
                                    run.max_rows, want_mass=True)
    torch.cuda.synchronize()
    assert torch.equal(o2, o1) and torch.equal(m2, m1)


@pytest.mark.parametrize("name", ["llada8b_ragged_b32", "llada8b_verify_b8"])
def test_split_attention_reruns_bitwise(name):
    """Both split-path attention kernels at full layer size (batch 32: one
    1024-key split per unit, scores on chip; two-view batch 8: the forward
    kernel): eight calls on the same inputs give the same bits."""
    import kv_cache_attention_flash_amd as fd
    fd.load()
    wl = synth.WORKLOADS[name]()
    run = G.GpuRun(wl, "cuda:0")
    mass = name == "llada8b_ragged_b32"
    path = fd.attention_path(wl.batch, wl.rows, wl.num_heads, wl.head_dim, wl.max_kv_len,
                             run.max_rows, wl.max_kv_len if mass else 0)
    _banner(f"split attention reruns {name}: path {path}")
    q, _ = fd.flash_cache_step(run.cache, run.x, run.w, run.cu, run.pos, run.slots, wl.rope_base)
    ref = None
    for rep in range(8):
        res = fd.scheduled_attention(run.cache, q, run.cu, run.kv_len, wl.max_kv_len, run.max_rows,
                                     views=run.views, want_mass=mass)
        torch.cuda.synchronize()
        res = tuple(t.clone() for t in res if t is not None)
        if ref is None:
            ref = res
        else:
            assert all(torch.equal(x, y) for x, y in zip(res, ref)), rep


def test_block_permutation_invariance():
    _banner("block-table permutation invariance")
    wl = synth.small_ragged()
    perm = np.random.default_rng(99).permutation(wl.num_blocks)
    bt2 = np.zeros_like(wl.block_table)
    k2 = np.zeros_like(wl.k_cache)
    v2 = np.zeros_like(wl.v_cache)
    off = 0
    for b in range(wl.batch):
        n = -(-int(wl.kv_len[b]) // wl.block_size)
        bt2[b, :n] = perm[off:off + n]
        off += n
        k2[bt2[b, :n]] = wl.k_cache[wl.block_table[b, :n]]
        v2[bt2[b, :n]] = wl.v_cache[wl.block_table[b, :n]]
    a = G.GpuRun(wl).step()
    b = G.GpuRun(wl, k=G.bf16_tensor(k2, "cuda:0"), v=G.bf16_tensor(v2, "cuda:0"),
                 block_table=bt2).step()
    for f in ("q", "out", "mass", "idx"):
        assert torch.equal(getattr(a, f), getattr(b, f)), f


def test_uniform_attention_ties():
    """All hidden states zero: every score is 0, every visible key gets exactly
    the same mass, so the lower-index tie rule gives top-B = {0..B-1}."""
    _banner("exact ties")
    wl = synth.llada8b_b1()
    wl.x = np.zeros_like(wl.x)
    run = G.GpuRun(wl).step()
    m = run.mass.cpu().numpy()[0]
    assert np.all(m[:768] == m[0])
    assert list(run.idx.cpu().numpy()[0]) == list(range(32))


def test_two_view_isolation_and_causality():
    """Changing the draft rows' inputs leaves the mask rows' outputs bit-identical
    and vice versa; changing draft row j leaves draft rows i < j bit-identical."""
    _banner("two-view isolation")
    wl = synth.small_verify()
    base = G.GpuRun(wl).step()
    out0 = base.out.cpu().numpy()
    wlen = int(wl.views[0, 1])
    r0 = int(wl.cu_rows[0])
    # perturb all draft rows of sequence 0
    x = wl.x.copy()
    x[r0:r0 + wlen] = synth.normal_bf16(77, 0, 0, (wlen, wl.hid))
    run = G.GpuRun(wl, x=G.bf16_tensor(x, "cuda:0")).step()
    o = run.out.cpu().numpy()
    assert np.array_equal(o[r0 + wlen:r0 + 2 * wlen], out0[r0 + wlen:r0 + 2 * wlen])
    assert not np.array_equal(o[r0:r0 + wlen], out0[r0:r0 + wlen])
    # perturb mask rows of sequence 0
    x = wl.x.copy()
    x[r0 + wlen:r0 + 2 * wlen] = synth.normal_bf16(78, 0, 0, (wlen, wl.hid))
    run = G.GpuRun(wl, x=G.bf16_tensor(x, "cuda:0")).step()
    o = run.out.cpu().numpy()
    assert np.array_equal(o[r0:r0 + wlen], out0[r0:r0 + wlen])
    # perturb draft row 5 only
    x = wl.x.copy()
    x[r0 + 5] = synth.normal_bf16(79, 0, 0, (1, wl.hid))[0]
    run = G.GpuRun(wl, x=G.bf16_tensor(x, "cuda:0")).step()
    o = run.out.cpu().numpy()
    assert np.array_equal(o[r0:r0 + 5], out0[r0:r0 + 5])
    assert not np.array_equal(o[r0 + 5:r0 + wlen], out0[r0 + 5:r0 + wlen])


def test_topb_crafted_masses():
    """track_topb alone on crafted masses (ties, zeros, kv_len < B, long rows)."""
    fd = _fd()
    dev = "cuda:0"
    rng = np.random.default_rng(3)
    rows = [np.array([0.5, 2.0, 2.0, 0.1, 3.0, 2.0, 0.0] + [0.0] * 4089, np.float32),
            rng.integers(0, 4, 4096).astype(np.float32) / 8,
            rng.random(4096, dtype=np.float32),
            np.zeros(4096, np.float32)]
    lens = [7, 4096, 3000, 10]
    # stride 4096 (the 1024-thread workgroup) and 2000 (the 512-thread one)
    for width in (4096, 2000):
        mass = torch.from_numpy(np.ascontiguousarray(np.stack(rows)[:, :width])).to(dev)
        wl = [min(L, width) for L in lens]
        kv = G.i32(wl, dev)
        for b_ in (1, 3, 8, 32, 100):
            got = fd.track_topb(mass, kv, b_).cpu().numpy()
            for i, L in enumerate(wl):
                want = O.top_b(rows[i][:width].astype(np.float64), L, b_)
                assert np.array_equal(got[i], want), (width, b_, i)


def test_topb_uncached_rows_and_low_digits():
    """Rows longer than the LDS-cached 8192 keys (read from HBM in every pass),
    keys that differ only in their lowest byte (decided by the fourth digit
    pass), and threshold ties spread over many 64-key output chunks."""
    fd = _fd()
    dev = "cuda:0"
    rng = np.random.default_rng(11)
    width = 9000
    low = (np.uint32(0x3F800000) + rng.integers(0, 256, width).astype(np.uint32)).view(np.float32)
    ties = np.full(width, 0.25, np.float32)
    ties[rng.choice(width, 300, replace=False)] = 2.0   # 300 keys at the threshold value
    ties[rng.choice(width, 10, replace=False)] = 3.0    # ten above it
    flat = np.ones(width, np.float32)                    # every key ties
    rows = [rng.random(width, dtype=np.float32), low, ties, flat]
    lens = [width, 8999, width, 8193]
    mass = torch.from_numpy(np.ascontiguousarray(np.stack(rows))).to(dev)
    kv = G.i32(lens, dev)
    for b_ in (1, 32, 64, 150):
        got = fd.track_topb(mass, kv, b_).cpu().numpy()
        for i, L in enumerate(lens):
            want = O.top_b(rows[i].astype(np.float64), L, b_)
            assert np.array_equal(got[i], want), (b_, i)
    # the same rows cut to 2048 keys (the 512-thread workgroup, LDS-cached)
    mass2 = torch.from_numpy(np.ascontiguousarray(np.stack(rows)[:, :2048])).to(dev)
    kv2 = G.i32([2048, 2047, 2048, 1500], dev)
    for b_ in (32, 150):
        got = fd.track_topb(mass2, kv2, b_).cpu().numpy()
        for i, L in enumerate([2048, 2047, 2048, 1500]):
            want = O.top_b(rows[i][:2048].astype(np.float64), L, b_)
            assert np.array_equal(got[i], want), ("cached", b_, i)


def test_verify_long_window():
    """Windows longer than one wavefront; crafted prefixes."""
    fd = _fd()
    dev = "cuda:0"
    v = synth.verify_scan_inputs(31, 5, 150)
    d, m, c = v["draft"].copy(), v["mask"].copy(), v["conf"].copy()
    d[:3] = np.arange(150)
    m[:3] = np.arange(150)
    c[:3] = 0.99
    m[1, 97] += 1
    c[2, 64] = 0.9
    got = fd.verify_accept(*(torch.from_numpy(a).to(dev) for a in (d, m, c)), 0.9).cpu().numpy()
    want = [O.accept_length(d[i], m[i], c[i], v["threshold"]) for i in range(len(d))]
    assert list(got) == want
    assert want[:3] == [150, 97, 64]


@pytest.mark.parametrize("name", ["small_ragged_b5", "small_long_l1500", "small_verify_b3"])
def test_unused_slots_never_read(name):
    """NaN in every cache slot at or past kv_len (the tail of each sequence's
    last page): outputs stay finite and match the oracle, which never reads
    those slots.  Covers the row-group path (short caches) and the split path
    with a second mass pass (caches past 1024 keys)."""
    _banner(f"NaN past kv_len: {name}")
    wl = synth.WORKLOADS[name]()
    k, v = wl.k_cache.copy(), wl.v_cache.copy()
    bs = wl.block_size
    poisoned = 0
    for b in range(wl.batch):
        L = int(wl.kv_len[b])
        for slot in range(L, -(-L // bs) * bs):
            blk, off = wl.block_table[b, slot // bs], slot % bs
            k[blk, :, off, :] = 0x7FC0
            v[blk, :, off, :] = 0x7FC0
            poisoned += 1
    assert poisoned > 0
    dev = "cuda:0"
    run = G.GpuRun(wl, dev, k=G.bf16_tensor(k, dev), v=G.bf16_tensor(v, dev)).step()
    out = run.out.cpu().numpy()
    assert np.all(np.isfinite(out))
    ref = G.oracle_step(wl)
    G.assert_close(out[ref["rows"]], ref["out"], "attention output with NaN past kv_len")
    if wl.topb:
        mass = run.mass.cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(mass))
        G.assert_close(mass, ref["mass"], "mass with NaN past kv_len")


@pytest.mark.parametrize("name", ["small_ragged_b5", "small_splitk_h1024", "small_d64_rows150",
                                  "llada8b_b1_l768", "llada8b_verify_b8"])
def test_unfused_ablation_is_bitwise_equal(name):
    """flash_cache_step_unfused (projection -> fp32 Y in HBM -> rotary ->
    staging -> scatter) gives bitwise the fused step's Q, slot mapping and cache
    contents: the same projection kernels and rounding helper, only the traffic
    differs.  Covers the split-K path (with and without a split reduction) and
    the tiled path."""
    _banner(f"unfused ablation vs fused: {name}")
    fd = _fd()
    dev = "cuda:0"
    wl = synth.WORKLOADS[name]()
    outs = []
    for fn in (fd.flash_cache_step, fd.flash_cache_step_unfused):
        run = G.GpuRun(wl, dev)
        q, sm = fn(run.cache, run.x, run.w, run.cu, run.pos, run.slots, wl.rope_base)
        torch.cuda.synchronize()
        outs.append((G.bits_of(q), sm.cpu().numpy(), G.bits_of(run.cache.k_cache),
                     G.bits_of(run.cache.v_cache)))
    for what, a_, b_ in zip(("q", "slot mapping", "K cache", "V cache"), outs[0], outs[1]):
        assert np.array_equal(a_, b_), what


@pytest.mark.parametrize("case", ["d64_b16_h16", "d128_b8_h32_views"])
def test_second_pass_mass_path(case):
    """Caches past 1024 keys with enough sequences x heads for one workgroup
    per unit: the mass comes from a second, last-first pass over K in the same
    workgroup.  Ragged lengths (not multiples of the block size), two row tiles
    in some sequences, two-view sequences; element-wise against the oracle,
    and bitwise equal on eight reruns."""
    import kv_cache_attention_flash_amd as fd
    fd.load()
    g = np.random.default_rng(31 if case.startswith("d64") else 32)
    specs = []
    if case == "d64_b16_h16":
        for b in range(16):
            L = int(g.integers(1030, 2200))
            w = int(g.integers(8, 49))
            w0 = int(g.integers(0, L - w))
            pool = [p for p in range(L) if not (w0 <= p < w0 + w)]
            nt = int(g.integers(0, 41))
            tr = tuple(sorted(int(p) for p in g.choice(pool, size=nt, replace=False)))
            specs.append(SeqSpec(kv_len=L, window=(w0, w), tracked=tr))
        wl = synth.build("reread_d64", 26, 256, 16, 64, 64, 1.0e4, specs, topb=16)
    else:
        for b in range(8):
            L = int(g.integers(1100, 1800))
            if b % 3 == 0:
                ctx = L - 16
                w0 = int(g.integers(0, ctx - 16))
                specs.append(SeqSpec(kv_len=L, window=(w0, 16), tracked=(), draft_start=ctx))
            else:
                w0 = int(g.integers(32, L - 32))
                tr = tuple(sorted(int(p) for p in g.choice(w0, 32, replace=False)))
                specs.append(SeqSpec(kv_len=L, window=(w0, 32), tracked=tr))
        wl = synth.build("reread_d128", 27, 512, 32, 128, 32, 5.0e5, specs, topb=32)
    run = G.GpuRun(wl, "cuda:0")
    path = fd.attention_path(wl.batch, wl.rows, wl.num_heads, wl.head_dim, wl.max_kv_len,
                             run.max_rows, wl.max_kv_len)
    _banner(f"second-pass mass {case}: lengths {wl.kv_len.tolist()}, path {path}")
    assert path == "split_mass_reread"
    run.step()
    a_out, a_mass = run.out.clone(), run.mass.clone()
    full_check(wl, run=run)
    for rep in range(8):  # the mass pass's row-group sums cross a barrier every tile
        o2, m2 = fd.scheduled_attention(run.cache, run.q, run.cu, run.kv_len, wl.max_kv_len,
                                        run.max_rows, views=run.views, want_mass=True)
        torch.cuda.synchronize()
        assert torch.equal(o2, a_out) and torch.equal(m2, a_mass), rep
