"""The allocation-free attention entry point (scheduled_attention_static)
against scheduled_attention through the C ABI: bitwise the same outputs and
mass on two calls in a row that share the library's static scratch buffer,
the second with a smaller input; sizes past the buffer are refused before
anything is launched."""

import numpy as np
import pytest

import synth
from synth import SeqSpec

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from tests import gpu_util as G  # noqa: E402

DEV = "cuda:0"


def _fd():
    import kv_cache_attention_flash_amd as fd
    fd.load()
    return fd


def _long_batch():
    """Four sequences past 1024 keys: splits that exchange row statistics
    through counters and partials in the scratch buffer."""
    g = np.random.default_rng(41)
    specs = [SeqSpec(kv_len=4096 - 53 * b, window=(int(g.integers(32, 3000)), 32),
                     tracked=tuple(sorted(int(p) for p in g.choice(32, 32, replace=False))))
             for b in range(4)]
    return synth.build("static_long_b4", 28, 512, 8, 128, 32, 5.0e5, specs, topb=32)


def _compare(fd, wl, want_mass=True):
    run = G.GpuRun(wl, DEV)
    q, _ = fd.flash_cache_step(run.cache, run.x, run.w, run.cu, run.pos, run.slots, wl.rope_base)
    o_ref, m_ref = fd.scheduled_attention(run.cache, q, run.cu, run.kv_len, wl.max_kv_len,
                                          run.max_rows, views=run.views, want_mass=want_mass)
    out = torch.full_like(o_ref, 3.0)
    mass = torch.full_like(m_ref, 3.0) if want_mass else None
    torch.cuda.synchronize()
    fd.scheduled_attention_static(run.cache, q, run.cu, run.kv_len, wl.max_kv_len, run.max_rows,
                                  out, mass=mass, views=run.views)
    torch.cuda.synchronize()
    assert torch.equal(out, o_ref), wl.name
    if want_mass:
        assert torch.equal(mass, m_ref), wl.name
    path = fd.attention_path(wl.batch, wl.rows, wl.num_heads, wl.head_dim, wl.max_kv_len,
                             run.max_rows, wl.max_kv_len if want_mass else 0)
    print(f"[no-alloc] {wl.name}: path {path}, bitwise equal", flush=True)
    return path


def test_static_scratch_matches_the_workspace_call_twice():
    fd = _fd()
    first = _compare(fd, _long_batch())
    assert first == "split_mass_exchange"
    # a smaller input next, on the buffer the first call left behind
    second = _compare(fd, synth.small_long())
    assert second == "split_mass_exchange"
    _compare(fd, synth.small_ragged())                    # row-group path
    _compare(fd, synth.small_verify(), want_mass=False)   # split path with merges


def test_sizes_past_the_buffer_are_refused():
    fd = _fd()
    wl = synth.small_ragged()
    run = G.GpuRun(wl, DEV)
    batch, h, d, L = 64, 64, 128, 4096  # the mass partials alone need 64 MiB
    need = fd.attention_workspace_bytes(batch, batch * 64, h, d, L, 64, L)
    assert need > fd.static_scratch_bytes()
    cache = fd.PagedKVCache(torch.zeros((8, h, 32, d), dtype=torch.bfloat16, device=DEV),
                            torch.zeros((8, h, 32, d), dtype=torch.bfloat16, device=DEV),
                            torch.zeros((batch, L // 32), dtype=torch.int32, device=DEV))
    q = torch.zeros((batch * 64, h, d), dtype=torch.bfloat16, device=DEV)
    out = torch.full((batch * 64, h, d), 5.0, dtype=torch.float32, device=DEV)
    mass = torch.full((batch, L), 5.0, dtype=torch.float32, device=DEV)
    cu = torch.arange(0, batch * 64 + 1, 64, dtype=torch.int32, device=DEV)
    kv = torch.full((batch,), L, dtype=torch.int32, device=DEV)
    with pytest.raises(fd.FdlError) as e:
        fd.scheduled_attention_static(cache, q, cu, kv, L, 64, out, mass=mass)
    assert e.value.status == 5, str(e.value)
    torch.cuda.synchronize()
    assert bool((out == 5.0).all()) and bool((mass == 5.0).all())
    del run
