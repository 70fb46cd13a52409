"""GPU parity on seeded random small shapes: every path the library picks by
shape, against the CPU oracle with the same bar as the fixed workloads.

Each case draws the head count and size, the hidden size (a multiple of 128:
256-multiples take the split-K projection at up to 64 rows, the others the
tiled one), the block size, a batch of 1-7 sequences with ragged cache
lengths, windows and tracked rows (some sequences two-view), and a top-B
budget (zero leaves out the mass, which moves attention to the split path).
The rows total crosses 64 in some cases, so both projection kernels and both
attention paths occur.

A second family draws long caches (up to 3500 slots, lengths on and next to
the 1024-key split boundaries) with the mass always asked for: attention then
takes the split path whose splits exchange their row statistics (more than
one split per sequence), with up to 88 rows per sequence (two row tiles),
both head sizes, block sizes up to 256 and two-view sequences.
"""

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from tests.test_parity_gpu import full_check  # noqa: E402

CASES = 64


def random_workload(seed):
    """Even seeds: at most ~64 rows and hidden sizes the split-K projection
    takes; odd seeds: larger batches and any hidden size."""
    g = np.random.default_rng(1000 + seed)
    small = seed % 2 == 0
    heads = int(g.choice([1, 2, 3, 4, 6]))
    dim = int(g.choice([64, 128]))
    hid = int(g.choice([256, 512, 1024] if small else [128, 256, 384, 512, 1024]))
    bs = int(g.choice([32, 64, 128]))
    batch = int(g.integers(1, 4 if small else 8))
    wmax, tmax = (16, 8) if small else (32, 16)
    two_view = g.random() < 0.3
    specs = []
    for _ in range(batch):
        if two_view and g.random() < 0.7:
            w = int(g.integers(1, wmax + 1))
            ctx = int(g.integers(w, 260))
            w0 = int(g.integers(0, ctx - w + 1))
            pool = [p for p in range(ctx) if not (w0 <= p < w0 + w)]
            nt = min(int(g.integers(0, tmax // 2 + 1)), len(pool))
            tr = tuple(sorted(int(p) for p in g.choice(pool, size=nt, replace=False))) if nt else ()
            specs.append(synth.SeqSpec(kv_len=ctx + w, window=(w0, w), tracked=tr,
                                       draft_start=ctx))
        else:
            length = int(g.integers(1, 400))
            w = int(g.integers(0, min(wmax, length) + 1))
            w0 = int(g.integers(0, length - w + 1))
            pool = [p for p in range(length) if not (w0 <= p < w0 + w)]
            nt = min(int(g.integers(0, tmax + 1)), len(pool))
            tr = tuple(sorted(int(p) for p in g.choice(pool, size=nt, replace=False))) if nt else ()
            specs.append(synth.SeqSpec(kv_len=length, window=(w0, w), tracked=tr))
    topb = int(g.choice([0, 0, 4, 8, 16]))
    return synth.build(f"random_{seed}", 60 + seed, hid, heads, dim, bs, 1.0e4, specs, topb=topb)


@pytest.mark.parametrize("seed", range(CASES))
def test_random_shape(seed):
    wl = random_workload(seed)
    if wl.rows == 0:
        pytest.skip("no active rows drawn")
    print(f"[random] seed {seed}: rows {wl.rows}, batch {wl.batch}, {wl.num_heads}x{wl.head_dim}, "
          f"hidden {wl.hid}, block {wl.block_size}, topb {wl.topb}, "
          f"views {wl.views is not None}", flush=True)
    full_check(wl)


LONG_CASES = 24


def random_long_workload(seed):
    g = np.random.default_rng(5000 + seed)
    heads = int(g.choice([1, 2, 3, 4]))
    dim = int(g.choice([64, 128]))
    hid = int(g.choice([256, 384, 512]))
    bs = int(g.choice([32, 64, 128, 256]))
    batch = int(g.integers(1, 5))
    two_view = g.random() < 0.3
    specs = []
    for _ in range(batch):
        if g.random() < 0.3:
            length = int(g.choice([1024, 1025, 2047, 2048, 2049, 3072]))
        else:
            length = int(g.integers(700, 3501))
        if two_view and g.random() < 0.6:
            w = int(g.integers(1, 33))
            ctx = length - w
            w0 = int(g.integers(0, ctx - w + 1))
            pool = [p for p in range(ctx) if not (w0 <= p < w0 + w)]
            nt = int(g.integers(0, 17))
            tr = tuple(sorted(int(p) for p in g.choice(pool, size=nt, replace=False))) if nt else ()
            specs.append(synth.SeqSpec(kv_len=length, window=(w0, w), tracked=tr,
                                       draft_start=ctx))
        else:
            w = int(g.integers(0, 49))
            w0 = int(g.integers(0, length - w + 1))
            pool = [p for p in range(length) if not (w0 <= p < w0 + w)]
            nt = int(g.integers(0, 41))
            tr = tuple(sorted(int(p) for p in g.choice(pool, size=nt, replace=False))) if nt else ()
            specs.append(synth.SeqSpec(kv_len=length, window=(w0, w), tracked=tr))
    topb = int(g.choice([4, 8, 16, 32]))
    return synth.build(f"random_long_{seed}", 200 + seed, hid, heads, dim, bs, 1.0e4, specs,
                       topb=topb)


@pytest.mark.parametrize("seed", range(LONG_CASES))
def test_random_long_cache(seed):
    wl = random_long_workload(seed)
    if wl.rows == 0:
        pytest.skip("no active rows drawn")
    print(f"[random-long] seed {seed}: rows {wl.rows}, batch {wl.batch}, "
          f"{wl.num_heads}x{wl.head_dim}, hidden {wl.hid}, block {wl.block_size}, "
          f"lengths {wl.kv_len.tolist()}, topb {wl.topb}, views {wl.views is not None}",
          flush=True)
    full_check(wl)


REREAD_CASES = 6


def random_reread_workload(seed):
    """Enough sequences x heads for one workgroup per (sequence, row tile,
    head) unit (>= 256) and caches past 1024 keys: attention takes the split
    path whose workgroups read K a second time for the mass.  Block sizes 32
    to 256, both head sizes, ragged lengths (some on a tile boundary), one or
    two row tiles per sequence, some two-view sequences."""
    g = np.random.default_rng(7000 + seed)
    dim = int(g.choice([64, 128]))
    heads = int(g.choice([16, 32]))
    batch = 256 // heads + int(g.integers(0, 3))
    bs = int(g.choice([32, 64, 128, 256]))
    specs = []
    for _ in range(batch):
        length = int(g.choice([1056, 2048])) if g.random() < 0.25 else int(g.integers(1030, 2300))
        if g.random() < 0.25:
            w = int(g.integers(1, 33))
            ctx = length - w
            w0 = int(g.integers(0, ctx - w + 1))
            specs.append(synth.SeqSpec(kv_len=length, window=(w0, w), tracked=(), draft_start=ctx))
        else:
            w = int(g.integers(1, 49))
            w0 = int(g.integers(0, length - w + 1))
            pool = [p for p in range(length) if not (w0 <= p < w0 + w)]
            nt = int(g.integers(0, 41))
            tr = tuple(sorted(int(p) for p in g.choice(pool, size=nt, replace=False))) if nt else ()
            specs.append(synth.SeqSpec(kv_len=length, window=(w0, w), tracked=tr))
    topb = int(g.choice([8, 16, 32]))
    return synth.build(f"random_reread_{seed}", 300 + seed, 256, heads, dim, bs, 1.0e4, specs,
                       topb=topb)


@pytest.mark.parametrize("seed", range(REREAD_CASES))
def test_random_second_pass_mass(seed):
    import kv_cache_attention_flash_amd as fd
    fd.load()
    wl = random_reread_workload(seed)
    path = fd.attention_path(wl.batch, wl.rows, wl.num_heads, wl.head_dim, wl.max_kv_len,
                             int(np.diff(wl.cu_rows).max()), wl.max_kv_len)
    print(f"[random-reread] seed {seed}: rows {wl.rows}, batch {wl.batch}, "
          f"{wl.num_heads}x{wl.head_dim}, block {wl.block_size}, "
          f"lengths {wl.kv_len.min()}..{wl.kv_len.max()}, topb {wl.topb}, path {path}",
          flush=True)
    assert path == "split_mass_reread"
    full_check(wl)
