"""GPU parity: the HIP path (through the C ABI) against the CPU oracle, on the
same seeded inputs.

Integers (slot mapping, tracking-set indices, accepted lengths) must match
bit-exactly; floats (Q, written K/V, attention output, attention mass) within
max|d| <= 2e-2 * max|ref| and rel-L2 <= 5e-3.  Tracking-set indices are exact
against the oracle's selection rule applied to the GPU's own fp32 mass, and
certified against a staged oracle (fp64 attention from the GPU's stored bf16
Q/K/V): any differing index must be a near-tie.
"""

import numpy as np
import pytest

import oracle as O
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _dev():
    import kv_cache_attention_flash_amd as fd
    fd.load()
    return "cuda:0"


from tests import gpu_util as G  # noqa: E402


def _banner(msg):
    print(f"[parity] {msg}", flush=True)


def full_check(wl, run=None, seqs=None, staged=True, check_untouched=True):
    """Run the GPU step (unless given) and compare everything with the oracle."""
    dev = _dev()
    init_k, init_v = wl.k_cache, wl.v_cache
    run = run or G.GpuRun(wl, dev).step()
    ref = G.oracle_step(wl, seqs=seqs)
    rows = ref["rows"]
    sm = run.slot_mapping.cpu().numpy()
    assert np.array_equal(sm[rows], ref["slot_mapping"]), "slot mapping"
    q_bits = G.bits_of(run.q)
    G.assert_close(O.bf16_bits_to_f64(q_bits[rows]), O.bf16_bits_to_f64(ref["q"]), "Q")
    k_bits = G.bits_of(run.cache.k_cache)
    v_bits = G.bits_of(run.cache.v_cache)
    G.compare_cache(wl, ref, k_bits, v_bits, init_k, init_v,
                    seqs=None if check_untouched else "skip")
    out = run.out.cpu().numpy()
    G.assert_close(out[rows], ref["out"], "attention output")
    seq_ids = np.arange(wl.batch) if seqs is None else np.asarray(seqs)
    if wl.topb:
        mass = run.mass.cpu().numpy().astype(np.float64)
        idx = run.idx.cpu().numpy()
        G.assert_close(mass[seq_ids], ref["mass"], "attention mass")
        for b in range(wl.batch):  # exact against the rule applied to the GPU's own mass
            L = int(wl.kv_len[b])
            assert np.array_equal(idx[b], O.top_b(mass[b], L, wl.topb)), f"top-B seq {b}"
            assert np.all(mass[b, L:] == 0.0)
    if staged:
        sub = ref["sub"]
        o_s, probs = O.attention(q_bits[rows], k_bits, v_bits, sub["bt"], wl.block_size, sub["cu"],
                                 sub["kv_len"], views=sub["views"], want_probs=True)
        G.assert_close(out[rows], o_s, "attention output vs staged oracle")
        if wl.topb:
            m_s = O.attention_mass(probs, wl.max_kv_len)
            G.assert_close(mass[seq_ids], m_s, "mass vs staged oracle")
            err = np.max(np.abs(mass[seq_ids] - m_s)) / np.max(m_s)
            assert err < 1e-5, f"mass vs staged oracle rel err {err:.2e}"
            near = G.certify_topb(idx[seq_ids], m_s, sub["kv_len"], wl.topb, wl.name)
            _banner(f"{wl.name}: staged mass err {err:.2e}, certified near-ties {near}")
    return run, ref


SMALL = ["tiny_h256_l128", "small_ragged_b5", "small_verify_b3", "small_d64_rows150",
         "small_splitk_h1024", "small_long_l1500"]


@pytest.mark.parametrize("name", SMALL)
def test_small_workloads_elementwise(name):
    _banner(name)
    wl = synth.WORKLOADS[name]()
    run, _ = full_check(wl)
    if wl.verify is not None:
        _check_verify(wl.verify)


def _check_verify(v):
    import kv_cache_attention_flash_amd as fd
    dev = _dev()
    d, m, c = (torch.from_numpy(a).to(dev) for a in (v["draft"], v["mask"], v["conf"]))
    got = fd.verify_accept(d, m, c, float(v["threshold"])).cpu().numpy()
    want = [O.accept_length(v["draft"][b], v["mask"][b], v["conf"][b], v["threshold"])
            for b in range(len(v["draft"]))]
    assert list(got) == want


def test_llada8b_b1_full():
    _banner("llada8b_b1_l768 (hidden 4096, 32x128, batch 1, cache 768, 64 rows)")
    full_check(synth.llada8b_b1())


def test_llada8b_ragged_b32_full():
    """Batch 32, ragged lengths, refresh and update stages: every sequence
    element-wise against the oracle (Q, written K/V, untouched cache bytes,
    output, mass, top-B), plus the staged-oracle certification."""
    _banner("llada8b_ragged_b32 (batch 32, cache 512..1024, 2048 rows), all sequences")
    wl = synth.llada8b_ragged_b32()
    run, _ = full_check(wl)
    mass = run.mass.cpu().numpy().astype(np.float64)
    rows_per_seq = np.diff(wl.cu_rows)
    for b in range(wl.batch):  # the mass of a sequence sums to heads x rows
        s = mass[b].sum()
        assert abs(s - wl.num_heads * rows_per_seq[b]) <= 2e-5 * wl.num_heads * rows_per_seq[b], b


@pytest.mark.parametrize("name", ["llada8b_b1_l768", "small_ragged_b5", "small_splitk_h1024",
                                  "small_d64_rows150"])
def test_unfused_ablation_against_the_oracle(name):
    """flash_cache_step_unfused (projection -> fp32 Y in HBM -> rotary and
    rounding -> staging -> cache scatter) followed by attention, compared with
    the oracle like the fused step: the batch-1 layer (split-K projection), a
    ragged batch, a split reduction and the tiled projection."""
    _banner(f"unfused ablation vs oracle: {name}")
    wl = synth.WORKLOADS[name]()
    run = G.GpuRun(wl, _dev()).step(unfused=True)
    full_check(wl, run=run)


def test_llada8b_verify_b8_full():
    _banner("llada8b_verify_b8 (two-view, batch 8, 512 rows)")
    wl = synth.llada8b_verify_b8()
    full_check(wl)
    _check_verify(wl.verify)


@pytest.mark.slow
def test_llada8b_stack32_sampled():
    """32 layers of the step at batch 16, cache 4096: properties on every layer
    (mass sums, top-B, a second attention call bitwise equal), element-wise
    oracle comparison on sampled layers and sequences."""
    import kv_cache_attention_flash_amd as fd
    dev = _dev()
    wl = synth.llada8b_stack32_layout()
    cu, pos, slots = G.i32(wl.cu_rows, dev), G.i32(wl.positions, dev), G.i32(wl.slots, dev)
    kv_len, bt = G.i32(wl.kv_len, dev), G.i32(wl.block_table, dev)
    sample_layers = {0, 31}
    for layer in range(wl.layers):
        x, w, k, v = synth.stack_layer_tensors(wl, layer, dev)
        if layer in sample_layers:
            init = (G.bits_of(x), G.bits_of(w), G.bits_of(k), G.bits_of(v))
        cache = fd.PagedKVCache(k, v, bt)
        q, sm = fd.flash_cache_step(cache, x, w, cu, pos, slots, wl.rope_base)
        out, mass = fd.scheduled_attention(cache, q, cu, kv_len, 4096, 64, want_mass=True)
        out2, mass2 = fd.scheduled_attention(cache, q, cu, kv_len, 4096, 64, want_mass=True)
        assert torch.equal(out2, out) and torch.equal(mass2, mass), layer  # deterministic
        del out2, mass2
        idx = fd.track_topb(mass, kv_len, 32)
        m = mass.cpu().numpy().astype(np.float64)
        ix = idx.cpu().numpy()
        for b in range(wl.batch):
            assert abs(m[b].sum() - 32 * 64) <= 2e-5 * 32 * 64, (layer, b)
            assert np.array_equal(ix[b], O.top_b(m[b], 4096, 32)), (layer, b)
        if layer in sample_layers:
            _banner(f"stack layer {layer}: oracle on sequences 0 and 15")
            wl.x, wl.w, wl.k_cache, wl.v_cache = init
            run = type("R", (), {})()
            run.slot_mapping, run.q, run.out, run.mass, run.idx = sm, q, out, mass, idx
            run.cache = cache
            full_check(wl, run=run, seqs=[0, 15], check_untouched=False)
            wl.x = wl.w = wl.k_cache = wl.v_cache = None
        del x, w, k, v, cache, q, out, mass, idx
        torch.cuda.empty_cache()
