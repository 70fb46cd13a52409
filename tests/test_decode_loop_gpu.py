"""GPU parity of the multi-step decoding loop: the device planner and hidden-row
gather against the oracle's planning rules (bit-exact), the row-capacity
contract of the projection and attention calls (rows past cu_rows[batch] are
inactive), and whole loops checked step by step against the oracle fed the
GPU's own state at the start of each step (so a near-tie in one step's top-B
set cannot make the two trajectories drift apart), plus the free-running
oracle trajectory, whose plans must match the GPU's for as long as its top-B
sets do (where they first differ is reported).
"""

import numpy as np
import pytest

import oracle as O
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from tests import gpu_util as G  # noqa: E402


def _fd():
    import kv_cache_attention_flash_amd as fd
    fd.load()
    return fd


def _banner(msg):
    print(f"[loop] {msg}", flush=True)


DEV = "cuda:0"


def _random_plan_case(g, batch, topb):
    w = int(g.integers(1, 41))
    bs = int(g.choice([4, 32]))
    k = int(g.integers(0, 5))
    step = int(g.integers(0, 4))
    kv_len = g.integers(0, 200, batch).astype(np.int32)
    front = (g.integers(-3, 204, batch)).astype(np.int32)
    acc = g.integers(-3, 50, batch).astype(np.int32)
    if topb:
        tracked = np.sort(g.integers(-1, 210, (batch, topb)), axis=1).astype(np.int32)
        mix = g.random(batch) < 0.25  # some rows unsorted with repeats
        tracked[mix] = g.integers(-1, 210, (int(mix.sum()), topb))
    else:
        tracked = np.zeros((batch, 0), np.int32)
    return w, bs, k, step, kv_len, front, acc, tracked


def _run_plan(fd, w, bs, k, step, kv_len, front, acc, tracked):
    batch, topb = tracked.shape
    cap = batch * (w + topb)
    fr = G.i32(front, DEV)
    pos = torch.full((max(cap, 1),), -7, dtype=torch.int32, device=DEV)
    slots = torch.full((max(cap, 1),), -7, dtype=torch.int32, device=DEV)
    cu, pos, slots, stage = fd.decode_plan(G.i32(kv_len, DEV), fr,
                                           G.i32(tracked, DEV) if topb else None,
                                           G.i32(acc, DEV), step, w, bs, k, positions_out=pos,
                                           slots_out=slots)
    torch.cuda.synchronize()
    return fr.cpu().numpy(), stage.cpu().numpy()[:batch], cu.cpu().numpy(), pos.cpu().numpy(), \
        slots.cpu().numpy()


def test_plan_matches_oracle_random():
    fd = _fd()
    g = np.random.default_rng(100)
    cases = 0
    for batch, topb in [(1, 8), (3, 0), (17, 32), (64, 64), (65, 70), (300, 16), (1000, 5)]:
        for _ in range(6):
            w, bs, k, step, kv_len, front, acc, tracked = _random_plan_case(g, batch, topb)
            _banner(f"plan batch {batch} topb {topb} W {w} bs {bs} K {k} step {step}")
            f, stage, cu, pos, slots = _run_plan(fd, w, bs, k, step, kv_len, front, acc, tracked)
            rf, rstage, rcu, rpos, rslots = O.plan_step(step, kv_len, w, bs, k, tracked, acc, front)
            assert np.array_equal(f, rf), "frontier"
            assert np.array_equal(stage, rstage), "stage"
            assert np.array_equal(cu, rcu), "cu_rows"
            n = int(rcu[-1])
            assert np.array_equal(pos[:n], rpos) and np.array_equal(slots[:n], rslots), "rows"
            assert np.all(pos[n:] == -7) and np.all(slots[n:] == -7), "rows past the plan written"
            cases += 1
    _banner(f"{cases} random plans bit-exact")


def test_plan_largest_batch():
    fd = _fd()
    g = np.random.default_rng(101)
    w, bs, k, step, kv_len, front, acc, tracked = _random_plan_case(g, 4096, 4)
    got = _run_plan(fd, w, bs, k, step, kv_len, front, acc, tracked)
    ref = O.plan_step(step, kv_len, w, bs, k, tracked, acc, front)
    n = int(ref[2][-1])
    for a, b, what in zip(got[:3], ref[:3], ("frontier", "stage", "cu_rows")):
        assert np.array_equal(a, b), what
    assert np.array_equal(got[3][:n], ref[3])


def test_gather_matches_oracle():
    fd = _fd()
    g = np.random.default_rng(102)
    batch, max_len, hid, w, topb = 5, 90, 264, 12, 6
    com = g.integers(0, 65536, (batch, max_len, hid)).astype(np.uint16)
    msk = g.integers(0, 65536, (batch, max_len, hid)).astype(np.uint16)
    kv_len = g.integers(0, max_len + 1, batch).astype(np.int32)
    front = g.integers(0, max_len + 1, batch).astype(np.int32)
    tracked = np.sort(g.integers(-1, max_len, (batch, topb)), axis=1).astype(np.int32)
    acc = g.integers(0, 8, batch).astype(np.int32)
    fr = G.i32(front, DEV)
    cu, pos, slots, _ = fd.decode_plan(G.i32(kv_len, DEV), fr, G.i32(tracked, DEV),
                                       G.i32(acc, DEV), 1, w, 8, 2)
    cap = batch * (w + topb)
    x = torch.full((cap, hid), 3.0, dtype=torch.bfloat16, device=DEV)
    fd.gather_hidden(cu, pos, fr, G.bf16_tensor(com, DEV), G.bf16_tensor(msk, DEV), x_out=x)
    torch.cuda.synchronize()
    cu_h, pos_h, f_h = cu.cpu().numpy(), pos.cpu().numpy(), fr.cpu().numpy()
    n = int(cu_h[-1])
    ref = O.hidden_rows(com, msk, cu_h, pos_h[:n], f_h)
    xb = G.bits_of(x)
    assert np.array_equal(xb[:n], ref)
    assert np.all(xb[n:] == G.bits_of(torch.tensor([3.0], dtype=torch.bfloat16))[0])
    _banner(f"gather: {n} rows bit-exact, {cap - n} inactive rows untouched")


# --- the row-capacity contract of the per-step calls --------------------------------


@pytest.mark.parametrize("name,extra", [("small_splitk_h1024", 9), ("small_ragged_b5", 37),
                                        ("small_d64_rows150", 70)])
@pytest.mark.parametrize("unfused", [False, True])
def test_projection_inactive_rows(name, extra, unfused):
    """Rows past cu_rows[batch] are neither read nor written; active rows are
    bitwise those of a call sized exactly."""
    fd = _fd()
    wl = synth.WORKLOADS[name]()
    _banner(f"capacity {name} +{extra} rows unfused={unfused}")
    fn = fd.flash_cache_step_unfused if unfused else fd.flash_cache_step
    r = wl.rows
    exact = G.GpuRun(wl, DEV)
    q1, sm1 = fn(exact.cache, exact.x, exact.w, exact.cu, exact.pos, exact.slots, wl.rope_base)
    cap = G.GpuRun(wl, DEV)
    g = np.random.default_rng(5)
    xpad = np.concatenate([wl.x, g.integers(0, 65536, (extra, wl.hid)).astype(np.uint16)])
    # in-range slot 0 / position 0 in the tail: a wrong read would be visible
    pos = torch.cat([cap.pos, torch.zeros(extra, dtype=torch.int32, device=DEV)])
    slots = torch.cat([cap.slots, torch.zeros(extra, dtype=torch.int32, device=DEV)])
    q2 = torch.full((r + extra, wl.num_heads, wl.head_dim), 5.0, dtype=torch.bfloat16, device=DEV)
    sm2 = torch.full((r + extra,), -9, dtype=torch.int64, device=DEV)
    fn(cap.cache, G.bf16_tensor(xpad, DEV), cap.w, cap.cu, pos, slots, wl.rope_base, q_out=q2,
       slot_mapping_out=sm2)
    torch.cuda.synchronize()
    assert np.array_equal(G.bits_of(q2[:r]), G.bits_of(q1))
    assert np.all(G.bits_of(q2[r:]) == G.bits_of(torch.tensor([5.0], dtype=torch.bfloat16))[0])
    assert torch.equal(sm2[:r], sm1) and bool((sm2[r:] == -9).all())
    assert torch.equal(cap.cache.k_cache, exact.cache.k_cache)
    assert torch.equal(cap.cache.v_cache, exact.cache.v_cache)


@pytest.mark.parametrize("name", ["small_ragged_b5", "small_long_l1500", "llada8b_b1_l768"])
@pytest.mark.parametrize("mass", [False, True])
def test_attention_inactive_rows(name, mass):
    """Attention over a row capacity: active rows bitwise equal to the exact
    call, inactive output rows untouched (split merge and row-group paths)."""
    fd = _fd()
    wl = synth.WORKLOADS[name]()
    _banner(f"attention capacity {name} mass={mass}")
    run = G.GpuRun(wl, DEV)
    q, _ = fd.flash_cache_step(run.cache, run.x, run.w, run.cu, run.pos, run.slots, wl.rope_base)
    r, extra = wl.rows, 29
    o1, m1 = fd.scheduled_attention(run.cache, q, run.cu, run.kv_len, wl.max_kv_len, run.max_rows,
                                    want_mass=mass)
    qpad = torch.cat([q, torch.zeros((extra,) + tuple(q.shape[1:]), dtype=q.dtype, device=DEV)])
    o2 = torch.full((r + extra, wl.num_heads, wl.head_dim), 7.0, dtype=torch.float32, device=DEV)
    _, m2 = fd.scheduled_attention(run.cache, qpad, run.cu, run.kv_len, wl.max_kv_len,
                                   run.max_rows, out=o2, want_mass=mass)
    torch.cuda.synchronize()
    assert torch.equal(o2[:r], o1)
    assert bool((o2[r:] == 7.0).all())
    if mass:
        assert torch.equal(m1, m2)


# --- whole loops ------------------------------------------------------------------------


class LoopRun:
    def __init__(self, wl):
        fd = _fd()
        self.wl = wl
        w, k, v, hc, hm = synth.loop_tensors(wl, DEV)
        self.cache = fd.PagedKVCache(k, v, G.i32(wl.block_table, DEV))
        self.kv_len = G.i32(wl.kv_len, DEV)
        sc = wl.scan
        scan = (G.i32(sc["draft"], DEV), G.i32(sc["mask"], DEV),
                torch.from_numpy(sc["conf"]).to(DEV), sc["threshold"])
        self.loop = fd.DecodeLoop(self.cache, w, hc, hm, self.kv_len, G.i32(wl.frontier0, DEV),
                                  G.i32(wl.tracked0, DEV), wl.window_len, wl.rope_base,
                                  wl.refresh_period, wl.max_len, scan=scan)
        self.hc, self.hm, self.w = hc, hm, w

    def host_state(self):
        lp = self.loop
        return (lp.frontier.cpu().numpy(), lp.tracked.cpu().numpy(), lp.accept.cpu().numpy())


def _check_step(wl, t, lp, state, kc, vc, w_bits, hc_bits, hm_bits, sample_seqs=None):
    """Step t of the GPU loop against the oracle from the GPU's state before it."""
    front, tracked, acc = state
    rf, rstage, rcu, rpos, rslots = O.plan_step(t, wl.kv_len, wl.window_len, wl.block_size,
                                                wl.refresh_period, tracked, acc, front)
    cu = lp.cu_rows.cpu().numpy()
    n = int(rcu[-1])
    assert np.array_equal(lp.frontier.cpu().numpy(), rf), f"step {t}: frontier"
    assert np.array_equal(lp.stage.cpu().numpy(), rstage), f"step {t}: stage"
    assert np.array_equal(cu, rcu), f"step {t}: cu_rows"
    assert np.array_equal(lp.positions.cpu().numpy()[:n], rpos), f"step {t}: positions"
    assert np.array_equal(lp.slots.cpu().numpy()[:n], rslots), f"step {t}: slots"
    x_bits = G.bits_of(lp.x)[:n]
    x_ref = O.hidden_rows(hc_bits, hm_bits, rcu, rpos, rf)
    assert np.array_equal(x_bits, x_ref), f"step {t}: hidden rows"
    seqs = np.arange(wl.batch) if sample_seqs is None else np.asarray(sample_seqs)
    rows = np.concatenate([np.arange(rcu[b], rcu[b + 1]) for b in seqs]).astype(np.int64)
    scu = np.cumsum([0] + [int(rcu[b + 1] - rcu[b]) for b in seqs]).astype(np.int32)
    ref = O.decode_step(x_ref[rows], w_bits, wl.num_heads, wl.head_dim, rpos[rows], wl.rope_base,
                        scu, rslots[rows], wl.block_table[seqs], wl.block_size, kc, vc,
                        wl.kv_len[seqs], topb=wl.topb, mass_stride=wl.max_len)
    assert np.array_equal(lp.slot_mapping.cpu().numpy()[rows], ref["slot_mapping"])
    q_bits = G.bits_of(lp.q)
    G.assert_close(O.bf16_bits_to_f64(q_bits[rows]), O.bf16_bits_to_f64(ref["q"]), f"step {t}: Q")
    k_bits, v_bits = G.bits_of(lp.cache.k_cache), G.bits_of(lp.cache.v_cache)
    G.compare_cache(wl, ref, k_bits, v_bits, kc, vc,
                    seqs=None if sample_seqs is None else "sampled")
    out = lp.out.cpu().numpy()
    G.assert_close(out[rows], ref["out"], f"step {t}: attention output")
    mass = lp.mass.cpu().numpy().astype(np.float64)
    G.assert_close(mass[seqs], ref["mass"], f"step {t}: mass")
    idx = lp.tracked.cpu().numpy()
    for b in range(wl.batch):
        L = int(wl.kv_len[b])
        assert np.array_equal(idx[b], O.top_b(mass[b], L, wl.topb)), f"step {t}: top-B seq {b}"
        assert np.all(mass[b, L:] == 0.0)
        nrows = int(rcu[b + 1] - rcu[b])
        assert abs(mass[b, :L].sum() - wl.num_heads * nrows) <= 1e-5 * max(1, wl.num_heads * nrows)
    # staged oracle (fp64 attention on the GPU's stored bf16 Q, K, V): any
    # index where the sets differ must be a near-tie
    o_s, probs = O.attention(q_bits[rows], k_bits, v_bits, wl.block_table[seqs], wl.block_size,
                             scu, wl.kv_len[seqs], want_probs=True)
    m_s = O.attention_mass(probs, wl.max_len)
    near = G.certify_topb(idx[seqs], m_s, wl.kv_len[seqs], wl.topb, f"{wl.name} step {t}")
    sc = wl.scan
    acc_ref = np.array([O.accept_length(sc["draft"][t][b], sc["mask"][t][b], sc["conf"][t][b],
                                        sc["threshold"]) for b in range(wl.batch)], np.int32)
    assert np.array_equal(lp.accept.cpu().numpy(), acc_ref), f"step {t}: accept lengths"
    return n, near, rstage, k_bits, v_bits


@pytest.mark.parametrize("name", ["small_loop_b4", "small_loop_d128"])
def test_loop_step_by_step(name):
    wl = synth.LOOP_WORKLOADS[name]()
    run = LoopRun(wl)
    lp = run.loop
    kc, vc = wl.k_cache, wl.v_cache
    plans = []
    stages_seen = set()
    for t in range(wl.steps):
        state = run.host_state()
        lp.step(t)
        torch.cuda.synchronize()
        n, near, stage, kc, vc = _check_step(wl, t, lp, state, kc, vc, wl.w, wl.hidden_committed,
                                             wl.hidden_masked)
        stages_seen |= set(int(s) for s in stage)
        plans.append((lp.cu_rows.cpu().numpy(), lp.positions.cpu().numpy()[:n],
                      lp.tracked.cpu().numpy(), lp.frontier.cpu().numpy()))
        _banner(f"{name} step {t}: {n} rows, stages {stage.tolist()}, near-ties {near}")
    assert stages_seen == {O.STAGE_UPDATE, O.STAGE_REFRESH, O.STAGE_DONE}
    # The free-running oracle (its own fp64 projection, its own cache) takes
    # the same plans for as long as its top-B sets agree with the GPU's; where
    # they first differ is reported, as the independent oracle's top-B is a
    # statistic (its bf16 Q/K round differently now and then), not a gate.
    sc = wl.scan
    recs, _, _ = O.decode_loop(wl.steps, wl.w, wl.num_heads, wl.head_dim, wl.rope_base,
                               wl.block_table, wl.block_size, wl.k_cache, wl.v_cache, wl.kv_len,
                               wl.hidden_committed, wl.hidden_masked, wl.frontier0, wl.tracked0,
                               wl.window_len, wl.topb, wl.refresh_period, sc["draft"],
                               sc["mask"], sc["conf"], sc["threshold"], mass_stride=wl.max_len)
    for t, (rec, (cu, pos, idx, front)) in enumerate(zip(recs, plans)):
        assert np.array_equal(rec["cu_rows"], cu) and np.array_equal(rec["positions"], pos)
        assert np.array_equal(rec["frontier"], front)
        if not np.array_equal(rec["topb"], idx):
            diff = int(sum(len(set(a.tolist()) ^ set(b.tolist())) for a, b in zip(rec["topb"], idx)))
            _banner(f"{name}: free-running top-B sets first differ at step {t} ({diff} indices)")
            break
    else:
        _banner(f"{name}: free-running oracle trajectory identical over {wl.steps} steps")


def test_loop_full_size_b32():
    """The batch-32 layer as a 16-step loop: every step's plan, hidden rows,
    top-B sets, mass sums and accept lengths against the oracle; at steps 0,
    7 and 15 the outputs of four sequences against the oracle in full."""
    wl = synth.LOOP_WORKLOADS["llada8b_loop_b32"]()
    run = LoopRun(wl)
    lp = run.loop
    hc_bits, hm_bits = G.bits_of(run.hc), G.bits_of(run.hm)
    w_bits = G.bits_of(run.w)
    rows_total = 0
    for t in range(wl.steps):
        state = run.host_state()
        full = t in (0, 7, 15)
        if full:
            kc, vc = G.bits_of(lp.cache.k_cache), G.bits_of(lp.cache.v_cache)
        lp.step(t)
        torch.cuda.synchronize()
        if full:
            n, near, stage, _, _ = _check_step(wl, t, lp, state, kc, vc, w_bits, hc_bits,
                                               hm_bits, sample_seqs=[0, 9, 22, 31])
            _banner(f"full-size step {t}: {n} rows checked in full for 4 sequences, "
                    f"near-ties {near}")
        else:
            front, tracked, acc = state
            rf, rstage, rcu, rpos, _ = O.plan_step(t, wl.kv_len, wl.window_len, wl.block_size,
                                                   wl.refresh_period, tracked, acc, front)
            n = int(rcu[-1])
            assert np.array_equal(lp.frontier.cpu().numpy(), rf)
            assert np.array_equal(lp.cu_rows.cpu().numpy(), rcu)
            assert np.array_equal(lp.positions.cpu().numpy()[:n], rpos)
            x_ref = O.hidden_rows(hc_bits, hm_bits, rcu, rpos, rf)
            assert np.array_equal(G.bits_of(lp.x)[:n], x_ref)
            mass = lp.mass.cpu().numpy().astype(np.float64)
            idx = lp.tracked.cpu().numpy()
            for b in range(wl.batch):
                L = int(wl.kv_len[b])
                assert np.array_equal(idx[b], O.top_b(mass[b], L, wl.topb))
                nr = int(rcu[b + 1] - rcu[b])
                assert abs(mass[b, :L].sum() - wl.num_heads * nr) <= 1e-5 * wl.num_heads * max(nr, 1)
            sc = wl.scan
            acc_ref = [O.accept_length(sc["draft"][t][b], sc["mask"][t][b], sc["conf"][t][b],
                                       sc["threshold"]) for b in range(wl.batch)]
            assert lp.accept.cpu().numpy().tolist() == acc_ref
            _banner(f"full-size step {t}: {n} rows, plan/hidden/top-B/accept exact")
        rows_total += n
    _banner(f"full-size loop: {rows_total} active rows over {wl.steps} steps")
