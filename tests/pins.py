"""Pins of the CPU oracle: checks against closed forms, invariants, hand-worked
fixtures and brute force.  Each pin returns None or raises AssertionError, so the
mutation test can plant a mistake in the oracle and show that some pin fails.

Page key: [P4] "Flash-dLLM: I/O-Aware KV Caching and Parallel Decoding for Fast,
Memory-Efficient Diffusion LLMs" (ai4snews.wisdomeyes.cn summary), paragraphs 1-5.
"""

import json
import math
import os

import numpy as np

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def bits(x):
    """Exact fp64 -> bf16 bits for values known to be representable (test helper)."""
    b = (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(O.bf16_bits_to_f64(b), np.asarray(x, np.float64)), "not bf16-exact"
    return b


# --- bf16 codec -------------------------------------------------------------

def pin_bf16_midpoints():
    """Round-to-nearest-even at exact halfway points (storage format of the cache)."""
    one = 1.0
    cases = {one + 2.0 ** -8: 1.0,                      # halfway, even neighbour below
             one + 3 * 2.0 ** -8: one + 2.0 ** -6,      # halfway, even neighbour above
             one + 2.0 ** -8 + 2.0 ** -30: one + 2.0 ** -7,  # just above halfway
             -(one + 2.0 ** -8): -1.0,
             0.0: 0.0,
             3.0: 3.0}
    for x, want in cases.items():
        got = O.bf16_bits_to_f64(O.f64_to_bf16_bits(np.array([x])))[0]
        assert got == want, (x, got, want)
    big = O.f64_to_bf16_bits(np.array([3.5e38, -3.5e38]))
    assert np.all(np.isinf(O.bf16_bits_to_f64(big)))


def pin_bf16_vs_torch(n=20000, seed=0):
    """fp32 inputs: direct fp64->bf16 rounding equals torch's fp32->bf16 cast (RNE)."""
    import torch
    g = np.random.default_rng(seed)
    a = np.concatenate([g.standard_normal(n).astype(np.float32) * np.float32(10.0) ** g.integers(-30, 30, n).astype(np.float32),
                        np.array([1e-40, -1e-40, 1.1754944e-38, 3.3e38, 0.0, -0.0, 1.0], np.float32)])
    a = a[np.isfinite(a)]
    want = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = O.f64_to_bf16_bits(a.astype(np.float64))
    assert np.array_equal(got, want), np.flatnonzero(got != want)[:5]


# --- QKV projection ---------------------------------------------------------

def pin_gemm_integer_exact(seed=1):
    """Small-integer inputs: the product is exact; compare with a Python-int triple loop."""
    g = np.random.default_rng(seed)
    r, hid, n = 5, 12, 9
    xi = g.integers(-2, 3, (r, hid))
    wi = g.integers(-2, 3, (n, hid))
    y = O.qkv_projection(bits(xi.astype(np.float64)), bits(wi.astype(np.float64)))
    for i in range(r):
        for j in range(n):
            acc = 0
            for k in range(hid):
                acc += int(xi[i, k]) * int(wi[j, k])
            assert y[i, j] == acc, (i, j, y[i, j], acc)


# --- rotary embedding --------------------------------------------------------

def pin_rope_closed_form():
    """D=4, base b: e0 at position p -> (cos p, 0, sin p, 0) and
    e1 -> (0, cos(p b^-1/2), 0, sin(p b^-1/2)) (half-split pairs; an interleaved
    convention would give (cos p, sin p, 0, 0))."""
    base = 10000.0
    for p in (0, 1, 7, 1000):
        e = np.zeros((2, 1, 4))
        e[0, 0, 0] = 1.0
        e[1, 0, 1] = 1.0
        out = O.rope_rotate(e, np.array([p, p]), base)
        a1 = p * base ** -0.5
        assert np.allclose(out[0, 0], [math.cos(p), 0, math.sin(p), 0], atol=1e-12), out[0, 0]
        assert np.allclose(out[1, 0], [0, math.cos(a1), 0, math.sin(a1)], atol=1e-12), out[1, 0]


def pin_rope_invariants(seed=2):
    """Per-pair norms preserved; <R_m q, R_n k> depends only on m - n; p = 0 is the identity."""
    g = np.random.default_rng(seed)
    d = 128
    q = g.standard_normal((1, 1, d))
    k = g.standard_normal((1, 1, d))
    for base in (1e4, 5e5):
        r = O.rope_rotate(q, np.array([3]), base)
        half = d // 2
        n0 = q[..., :half] ** 2 + q[..., half:] ** 2
        n1 = r[..., :half] ** 2 + r[..., half:] ** 2
        assert np.allclose(n0, n1, rtol=1e-12, atol=1e-12)
        m, n = 37, 5
        ref = np.sum(O.rope_rotate(q, np.array([m]), base) * O.rope_rotate(k, np.array([n]), base))
        for t in (1, 100, 3000):
            sh = np.sum(O.rope_rotate(q, np.array([m + t]), base) * O.rope_rotate(k, np.array([n + t]), base))
            assert abs(sh - ref) < 1e-9 * (1 + abs(ref)), (t, sh, ref)
        assert np.array_equal(O.rope_rotate(q, np.array([0]), base), q)


# --- cache write ---------------------------------------------------------------

def pin_slot_map_hand():
    gd = golden("slot_map.json")
    ps = O.physical_slots(np.array(gd["cu_rows"]), np.array(gd["slots"]),
                          np.array(gd["block_table"]), gd["block_size"])
    assert list(ps) == gd["expect_physical"], ps


def _tiny_step(seed, h=2, d=8, hid=16, bs=4, lens=(10, 7), perm=None, rows=None):
    g = np.random.default_rng(seed)
    nblk = [-(-L // bs) for L in lens]
    nb = sum(nblk)
    perm = np.arange(nb) if perm is None else np.asarray(perm)
    bt = np.zeros((len(lens), max(nblk)), np.int32)
    off = 0
    for b, n in enumerate(nblk):
        bt[b, :n] = perm[off:off + n]
        off += n
    rows = rows or [[2, 3, 0], [6]]
    cu = np.cumsum([0] + [len(r) for r in rows]).astype(np.int32)
    slots = np.array([s for r in rows for s in r], np.int32)
    pos = slots.copy()
    x = bits(np.round(g.standard_normal((len(slots), hid)) * 4) / 4)
    w = bits(np.round(g.standard_normal((3 * h * d, hid)) * 8) / 64)
    kc = bits(np.round(g.standard_normal((nb, h, bs, d)) * 4) / 4)
    vc = bits(np.round(g.standard_normal((nb, h, bs, d)) * 4) / 4)
    return dict(x=x, w=w, h=h, d=d, pos=pos, cu=cu, slots=slots, bt=bt, bs=bs, kc=kc, vc=vc,
                kv_len=np.array(lens, np.int32))


def pin_cache_write_invariants():
    """Only the active slots change; written V equals the unrotated projection
    rounded to bf16; logical results do not depend on the physical block order."""
    t = _tiny_step(3)
    q, kc, vc, ps = O.flash_cache_step(t["x"], t["w"], t["h"], t["d"], t["pos"], 1e4, t["cu"],
                                       t["slots"], t["bt"], t["bs"], t["kc"], t["vc"])
    hd = t["h"] * t["d"]
    flat_old = t["kc"].transpose(0, 2, 1, 3).reshape(-1, hd)
    flat_new = kc.transpose(0, 2, 1, 3).reshape(-1, hd)
    untouched = np.setdiff1d(np.arange(flat_old.shape[0]), ps)
    assert np.array_equal(flat_old[untouched], flat_new[untouched])
    vflat = vc.transpose(0, 2, 1, 3).reshape(-1, hd)
    y = O.bf16_bits_to_f64(t["x"]) @ O.bf16_bits_to_f64(t["w"]).T
    assert np.array_equal(vflat[ps], O.f64_to_bf16_bits(y[:, 2 * hd:]))  # V is stored unrotated
    kflat = flat_new[ps]
    moved = t["pos"] != 0
    assert not np.array_equal(kflat[moved], O.f64_to_bf16_bits(y[moved, hd:2 * hd]))  # K is rotated
    # block permutation invariance of everything logical
    t2 = _tiny_step(3, perm=[4, 2, 0, 3, 1])
    blocks_old = t["bt"]
    kc2 = np.zeros_like(t2["kc"])
    vc2 = np.zeros_like(t2["vc"])
    for b in range(2):
        for i in range(-(-int(t["kv_len"][b]) // t["bs"])):
            kc2[t2["bt"][b, i]] = t["kc"][blocks_old[b, i]]
            vc2[t2["bt"][b, i]] = t["vc"][blocks_old[b, i]]
    r1 = O.decode_step(t["x"], t["w"], t["h"], t["d"], t["pos"], 1e4, t["cu"], t["slots"], t["bt"],
                       t["bs"], t["kc"], t["vc"], t["kv_len"], topb=3)
    r2 = O.decode_step(t["x"], t["w"], t["h"], t["d"], t["pos"], 1e4, t["cu"], t["slots"], t2["bt"],
                       t["bs"], kc2, vc2, t["kv_len"], topb=3)
    assert np.array_equal(r1["out"], r2["out"]) and np.array_equal(r1["topb"], r2["topb"])
    assert np.array_equal(r1["mass"], r2["mass"]) and np.array_equal(r1["q"], r2["q"])


# --- attention -------------------------------------------------------------------

def _one_seq_cache(kmat, vmat, bs=4):
    """Pack [L, D] keys/values of one head into a 1-head paged cache with identity table."""
    L, d = kmat.shape
    nb = -(-L // bs)
    kc = np.zeros((nb, 1, bs, d), np.uint16)
    vc = np.zeros((nb, 1, bs, d), np.uint16)
    kp = np.zeros((nb * bs, d))
    vp = np.zeros((nb * bs, d))
    kp[:L] = kmat
    vp[:L] = vmat
    kc[:, 0] = bits(kp).reshape(nb, bs, d)
    vc[:, 0] = bits(vp).reshape(nb, bs, d)
    return kc, vc, np.arange(nb, dtype=np.int32)[None]


def pin_attention_closed_forms(seed=4):
    g = np.random.default_rng(seed)
    d, L = 4, 7
    kmat = np.round(g.standard_normal((L, d)) * 8) / 8
    vmat = np.round(g.standard_normal((L, d)) * 8) / 8
    kc, vc, bt = _one_seq_cache(kmat, vmat)
    # q = 0: uniform weights -> O = mean of V
    q = np.zeros((1, 1, d), np.uint16)
    o = O.attention(q, kc, vc, bt, 4, np.array([0, 1]), np.array([L]))
    assert np.allclose(o[0, 0], vmat.mean(0), atol=1e-15)
    # single visible key -> O = v_0
    o = O.attention(bits(np.ones((1, 1, d))), kc, vc, bt, 4, np.array([0, 1]), np.array([1]))
    assert np.array_equal(o[0, 0], vmat[0])
    # two keys whose scaled scores differ by ln 3 -> weights 3/4 and 1/4
    s = math.log(3.0)
    k2 = np.zeros((2, d))
    k2[0, 0] = 1.0
    v2 = np.zeros((2, d))
    v2[0, 1] = 1.0
    v2[1, 2] = 1.0
    kc2, vc2, bt2 = _one_seq_cache(k2, v2)
    qv = np.zeros((1, 1, d))
    qv[0, 0, 0] = 2.0  # q.k0 = 2, q.k1 = 0; scale = s/2 makes the gap ln 3
    o = O.attention(bits(qv), kc2, vc2, bt2, 4, np.array([0, 1]), np.array([2]), scale=s / 2)
    assert abs(o[0, 0, 1] - 0.75) < 1e-14 and abs(o[0, 0, 2] - 0.25) < 1e-14, o
    # default scale is 1/sqrt(D): q.k gap of ln(3)*sqrt(D) gives 3/4 too
    qd = np.zeros((1, 1, d))
    qd[0, 0, 0] = 2.0
    o = O.attention(bits(qd), kc2, vc2, bt2, 4, np.array([0, 1]), np.array([2]))
    w0 = 1.0 / (1.0 + math.exp(-2.0 / math.sqrt(d)))
    assert abs(o[0, 0, 1] - w0) < 1e-14, (o, w0)


def pin_softmax_rows_sum_to_one(seed=5):
    t = _tiny_step(seed)
    q, kc, vc, _ = O.flash_cache_step(t["x"], t["w"], t["h"], t["d"], t["pos"], 1e4, t["cu"],
                                      t["slots"], t["bt"], t["bs"], t["kc"], t["vc"])
    _, probs = O.attention(q, kc, vc, t["bt"], t["bs"], t["cu"], t["kv_len"], want_probs=True)
    for p in probs:
        assert np.allclose(p.sum(-1), 1.0, rtol=0, atol=1e-12)
        assert np.all(p >= 0)


def pin_attention_brute_force(seed=6):
    """Pure-Python loops over an explicit mask matrix on a tiny two-view case."""
    g = np.random.default_rng(seed)
    d, h, bs = 4, 2, 4
    view = (1, 2, 4)
    L = 6
    nb = 2
    kc = bits(np.round(g.standard_normal((nb, h, bs, d)) * 4) / 4)
    vc = bits(np.round(g.standard_normal((nb, h, bs, d)) * 4) / 4)
    bt = np.array([[1, 0]], np.int32)
    q = bits(np.round(g.standard_normal((4, h, d)) * 4) / 4)
    o = O.attention(q, kc, vc, bt, bs, np.array([0, 4]), np.array([L]), views=np.array([view]))
    vis = golden("two_view_mask.json")["expect"]
    qf, kf, vf = (O.bf16_bits_to_f64(a) for a in (q, kc, vc))
    for hh in range(h):
        for r in range(4):
            sc, vals = [], []
            for j in range(L):
                if not vis[r][j]:
                    continue
                blk, off = int(bt[0, j // bs]), j % bs
                sc.append(sum(qf[r, hh, c] * kf[blk, hh, off, c] for c in range(d)) / math.sqrt(d))
                vals.append([vf[blk, hh, off, c] for c in range(d)])
            mx = max(sc)
            ws = [math.exp(s - mx) for s in sc]
            z = sum(ws)
            want = [sum(ws[i] * vals[i][c] for i in range(len(ws))) / z for c in range(d)]
            assert np.allclose(o[r, hh], want, rtol=1e-12, atol=1e-12), (hh, r)


def pin_two_view_mask_hand():
    gd = golden("two_view_mask.json")
    vis = O.visibility_mask(gd["rows"], gd["kv_len"], gd["view"])
    assert np.array_equal(vis.astype(int), np.array(gd["expect"])), vis.astype(int)


def pin_two_view_closed_forms(seed=7):
    """q = 0: draft row i -> (sum_ctx v + sum_{i'<=i} v_draft)/(|ctx|+i+1);
    mask row i -> (sum_ctx v + sum_window v)/(|ctx|+W).  Perturbing one view's
    keys/values leaves the other view's outputs bit-identical; perturbing draft
    key j leaves draft rows i < j bit-identical."""
    g = np.random.default_rng(seed)
    d, w0, wl, d0 = 4, 3, 3, 8
    L = d0 + wl
    vmat = np.round(g.standard_normal((L, d)) * 8) / 8
    kmat = np.round(g.standard_normal((L, d)) * 8) / 8
    kc, vc, bt = _one_seq_cache(kmat, vmat)
    view = np.array([[w0, wl, d0]])
    cu = np.array([0, 2 * wl])
    q0 = np.zeros((2 * wl, 1, d), np.uint16)
    o = O.attention(q0, kc, vc, bt, 4, cu, np.array([L]), views=view)
    ctx = [j for j in range(d0) if not (w0 <= j < w0 + wl)]
    for i in range(wl):
        want = (vmat[ctx].sum(0) + vmat[d0:d0 + i + 1].sum(0)) / (len(ctx) + i + 1)
        assert np.allclose(o[i, 0], want, atol=1e-14), i
        want = (vmat[ctx].sum(0) + vmat[w0:w0 + wl].sum(0)) / (len(ctx) + wl)
        assert np.allclose(o[wl + i, 0], want, atol=1e-14), i
    q = bits(np.round(g.standard_normal((2 * wl, 1, d)) * 4) / 4)
    base = O.attention(q, kc, vc, bt, 4, cu, np.array([L]), views=view)
    k2, v2 = kmat.copy(), vmat.copy()
    k2[d0:] += 1.0
    v2[d0:] -= 2.0
    kcp, vcp, _ = _one_seq_cache(k2, v2)
    pert = O.attention(q, kcp, vcp, bt, 4, cu, np.array([L]), views=view)
    assert np.array_equal(pert[wl:], base[wl:])       # mask view blind to draft keys
    assert not np.array_equal(pert[:wl], base[:wl])
    k3, v3 = kmat.copy(), vmat.copy()
    k3[w0:w0 + wl] += 1.0
    v3[w0:w0 + wl] -= 2.0
    kcp, vcp, _ = _one_seq_cache(k3, v3)
    pert = O.attention(q, kcp, vcp, bt, 4, cu, np.array([L]), views=view)
    assert np.array_equal(pert[:wl], base[:wl])       # draft view blind to window (mask-view) keys
    k4, v4 = kmat.copy(), vmat.copy()
    k4[d0 + 2] += 1.0
    v4[d0 + 2] -= 2.0
    kcp, vcp, _ = _one_seq_cache(k4, v4)
    pert = O.attention(q, kcp, vcp, bt, 4, cu, np.array([L]), views=view)
    assert np.array_equal(pert[:2], base[:2])         # causal inside the draft view
    assert not np.array_equal(pert[2], base[2])


# --- attention mass and top-B -----------------------------------------------

def pin_mass_sum_and_uniform(seed=8):
    """sum_j m_b[j] = H * R_b; with q = 0 every visible key has equal mass, so the
    tie rule makes top-B = {0..B-1}."""
    t = _tiny_step(seed, h=3)
    q, kc, vc, _ = O.flash_cache_step(t["x"], t["w"], t["h"], t["d"], t["pos"], 1e4, t["cu"],
                                      t["slots"], t["bt"], t["bs"], t["kc"], t["vc"])
    _, probs = O.attention(q, kc, vc, t["bt"], t["bs"], t["cu"], t["kv_len"], want_probs=True)
    mass = O.attention_mass(probs)
    for b in range(2):
        rb = t["cu"][b + 1] - t["cu"][b]
        assert abs(mass[b].sum() - 3 * rb) < 1e-12 * 3 * rb
    q0 = np.zeros_like(q)
    _, probs = O.attention(q0, kc, vc, t["bt"], t["bs"], t["cu"], t["kv_len"], want_probs=True)
    mass = O.attention_mass(probs)
    for b in range(2):
        L = int(t["kv_len"][b])
        assert np.all(mass[b, :L] == mass[b, 0])
        assert list(O.top_b(mass[b], L, 4)) == [0, 1, 2, 3]


def pin_top_b_crafted():
    m = np.array([0.5, 2.0, 2.0, 0.1, 3.0, 2.0, 0.0])
    assert list(O.top_b(m, 7, 3)) == [1, 2, 4]          # ties at 2.0 -> lower indices win
    assert list(O.top_b(m, 7, 1)) == [4]
    assert list(O.top_b(m, 7, 7)) == [0, 1, 2, 3, 4, 5, 6]
    assert list(O.top_b(m, 3, 5)) == [0, 1, 2, -1, -1]   # kv_len < B pads with -1
    assert list(O.top_b(m, 6, 4)) == [1, 2, 4, 5]
    assert list(O.top_b(np.array([1.0, 0.0, 5.0]), 2, 1)) == [0]  # keys past kv_len never count
    assert list(O.top_b(np.zeros(5), 5, 2)) == [0, 1]


def pin_top_b_brute(seed=9):
    g = np.random.default_rng(seed)
    for _ in range(50):
        n = int(g.integers(1, 40))
        b = int(g.integers(1, 12))
        m = g.integers(0, 5, n).astype(np.float64) / 4  # many ties
        best = sorted(range(n), key=lambda j: (-m[j], j))[:b]
        want = sorted(best) + [-1] * (b - len(best))
        assert list(O.top_b(m, n, b)) == want


# --- accept scan -----------------------------------------------------------------

def pin_accept_hand():
    gd = golden("accept_hand.json")
    thr = np.float32(gd["threshold"])
    for c in gd["cases"]:
        conf = [thr if v == "0.9f" else np.float32(v) for v in c["conf"]]
        got = O.accept_length(c["draft"], c["mask"], conf, thr)
        assert got == c["expect"], (c, got)


# --- multi-step loop: planning, hidden rows, state carried between steps ------------

def pin_decode_plan_hand():
    """Hand-worked three-step plan of four sequences (refresh and update
    stages, finished sequences, capped and negative accept lengths, tracked
    entries inside the window, past the length, repeated)."""
    gd = golden("decode_plan_hand.json")
    f = np.array(gd["frontier0"], np.int32)
    for t, st in enumerate(gd["steps"]):
        f, stage, cu, pos, slots = O.plan_step(t, gd["kv_len"], gd["window_len"],
                                               gd["block_size"], gd["refresh_period"],
                                               st["tracked"], st["accept"], f)
        assert list(f) == st["frontier"], (t, list(f))
        assert list(stage) == st["stage"], (t, list(stage))
        assert list(cu) == st["cu_rows"], (t, list(cu))
        assert list(pos) == st["positions"], (t, list(pos))
        assert list(slots) == st["positions"], (t, "slot = position")


def _plan_invariants(t, kv_len, w, bs, k, tracked, accept, f_in, plan):
    f, stage, cu, pos, slots = plan
    assert cu[0] == 0 and np.all(np.diff(cu) >= 0) and cu[-1] == len(pos)
    assert np.array_equal(pos, slots)
    for b, length in enumerate(kv_len):
        f0 = min(max(int(f_in[b]), 0), length)
        if t == 0 or f0 >= length:
            assert f[b] == f0
        else:
            assert f[b] == min(length, f0 + max(1, min(max(int(accept[b]), 0), w)))
        rows = [int(p) for p in pos[cu[b]:cu[b + 1]]]
        if f[b] >= length:
            assert rows == [] and stage[b] == O.STAGE_DONE
            continue
        refresh = k > 0 and (t + b) % k == 0
        assert stage[b] == (O.STAGE_REFRESH if refresh else O.STAGE_UPDATE)
        w0 = rows[0]
        assert w0 == ((f[b] // bs) * bs if refresh else f[b])
        nwin = min(w0 + w, length) - w0
        assert rows[:nwin] == list(range(w0, w0 + nwin))
        tr = rows[nwin:]
        assert all(0 <= p < length and not (w0 <= p < w0 + nwin) for p in tr)
        assert tr == sorted(set(tr)) and len(rows) == len(set(rows))
        assert len(rows) <= w + len(tracked[b])
        # every valid tracked entry outside the window, ascending input, is a row
        srt = sorted(set(int(p) for p in tracked[b]))
        want = [p for p in srt if 0 <= p < length and not (w0 <= p < w0 + nwin)]
        if list(tracked[b]) == srt:
            assert tr == want


def pin_decode_plan_invariants(seed=10):
    """Random states: window placement, commit rule, finished sequences and
    tracked-row filtering hold for every sequence."""
    g = np.random.default_rng(seed)
    for _ in range(200):
        batch = int(g.integers(1, 7))
        bs = int(g.choice([4, 8, 32]))
        w = int(g.integers(1, 12))
        nb = int(g.integers(1, 6))
        k = int(g.integers(0, 4))
        t = int(g.integers(0, 5))
        kv_len = [int(v) for v in g.integers(0, 40, batch)]
        f_in = g.integers(-2, 45, batch)
        accept = g.integers(-3, 15, batch)
        tracked = np.sort(g.integers(-1, 45, (batch, nb)), axis=1)
        if g.random() < 0.3:
            tracked = g.integers(-1, 45, (batch, nb))
        plan = O.plan_step(t, kv_len, w, bs, k, tracked, accept, f_in)
        _plan_invariants(t, kv_len, w, bs, k, tracked, accept, f_in, plan)


def pin_hidden_rows_marker():
    """Each row takes the committed-token table's row when its position lies
    below the frontier, the masked-token table's row otherwise."""
    batch, max_len, hid = 3, 10, 4
    com = np.zeros((batch, max_len, hid), np.uint16)
    msk = np.zeros((batch, max_len, hid), np.uint16)
    for b in range(batch):
        for p in range(max_len):
            com[b, p] = [b, p, 0, 7]
            msk[b, p] = [b, p, 1, 7]
    cu = np.array([0, 3, 3, 5], np.int32)
    pos = np.array([4, 5, 1, 9, 0], np.int32)
    front = [5, 0, 9]
    x = O.hidden_rows(com, msk, cu, pos, front)
    want = [[0, 4, 0, 7], [0, 5, 1, 7], [0, 1, 0, 7], [2, 9, 1, 7], [2, 0, 0, 7]]
    assert x.tolist() == want, x.tolist()


def _tiny_loop_inputs(seed, steps=3):
    g = np.random.default_rng(seed)
    h, d, bs, hid, w, nb = 2, 4, 4, 8, 4, 3
    kv_len = np.array([14, 9, 6], np.int32)
    nblk = [-(-int(n) // bs) for n in kv_len]
    perm = g.permutation(sum(nblk))
    bt = np.zeros((3, max(nblk)), np.int32)
    o = 0
    for b, n in enumerate(nblk):
        bt[b, :n] = perm[o:o + n]
        o += n
    def rnd(shape, scale=1.0):
        return O.f64_to_bf16_bits(g.standard_normal(shape) * scale)
    kc = rnd((sum(nblk), h, bs, d))
    vc = rnd((sum(nblk), h, bs, d))
    wq = rnd((3 * h * d, hid), 0.3)
    com = rnd((3, 14, hid))
    msk = rnd((3, 14, hid))
    draft = g.integers(0, 5, (steps, 3, w)).astype(np.int32)
    mask = np.where(g.random((steps, 3, w)) < 0.8, draft, draft + 1).astype(np.int32)
    conf = g.random((steps, 3, w)).astype(np.float32)
    return dict(w_bits=wq, num_heads=h, head_dim=d, rope_base=100.0, block_table=bt,
                block_size=bs, k_cache_bits=kc, v_cache_bits=vc, kv_len=kv_len,
                hidden_committed=com, hidden_masked=msk, frontier0=np.array([3, 2, 6], np.int32),
                tracked0=np.array([[0, 1, 9], [0, 5, 8], [0, 1, 2]], np.int32), window_len=w,
                topb=nb, refresh_period=2, draft=draft, mask=mask, conf=conf,
                threshold=np.float32(0.5))


def pin_decode_loop_carries_state(seed=11):
    """The loop's step t sees the cache as written by steps 0..t (recomposed
    here from the single-step functions), takes step t-1's top-B set and
    accept lengths into its plan, and its masses sum to heads x rows."""
    a = _tiny_loop_inputs(seed)
    recs, kc_end, vc_end = O.decode_loop(3, **a)
    kc, vc = a["k_cache_bits"], a["v_cache_bits"]
    f = a["frontier0"]
    tracked, accept = a["tracked0"], np.zeros(3, np.int32)
    for t, rec in enumerate(recs):
        f, stage, cu, pos, slots = O.plan_step(t, a["kv_len"], a["window_len"], a["block_size"],
                                               a["refresh_period"], tracked, accept, f)
        assert np.array_equal(cu, rec["cu_rows"]) and np.array_equal(pos, rec["positions"])
        x = O.hidden_rows(a["hidden_committed"], a["hidden_masked"], cu, pos, f)
        q, kc, vc, _ = O.flash_cache_step(x, a["w_bits"], 2, 4, pos, a["rope_base"], cu, slots,
                                          a["block_table"], 4, kc, vc)
        o = O.attention(q, kc, vc, a["block_table"], 4, cu, a["kv_len"])
        assert np.array_equal(o, rec["out"]), t
        for b in range(3):
            nrows = int(cu[b + 1] - cu[b])
            s = rec["mass"][b].sum()
            assert abs(s - 2 * nrows) <= 1e-12 * max(1.0, 2 * nrows), (t, b, s)
        tracked = rec["topb"]
        accept = np.array([O.accept_length(a["draft"][t][b], a["mask"][t][b], a["conf"][t][b],
                                           a["threshold"]) for b in range(3)], np.int32)
        assert np.array_equal(accept, rec["accept"])
    assert np.array_equal(kc, kc_end) and np.array_equal(vc, vc_end)


def pin_decode_loop_closed_form_frontier(seed=12):
    """With every scan position passing, each step commits the whole window
    (W tokens) until the sequence is finished: f_t = min(L, f_0 + W t)."""
    a = _tiny_loop_inputs(seed, steps=4)
    a["mask"] = a["draft"].copy()
    a["conf"] = np.ones_like(a["conf"])
    recs, _, _ = O.decode_loop(4, **a)
    for t, rec in enumerate(recs):
        want = np.minimum(a["kv_len"], a["frontier0"] + a["window_len"] * t)
        assert np.array_equal(rec["frontier"], want), (t, rec["frontier"], want)
        done = want >= a["kv_len"]
        assert np.array_equal(np.diff(rec["cu_rows"])[done], np.zeros(int(done.sum())))


# --- mask-view confidence producer (LM head) ----------------------------------------

def _one_hot_head(columns):
    """Hidden rows e_0 and a weight whose column 0 holds each row's logits: the
    logits of row r are exactly columns[r] (bf16-exact values)."""
    cols = np.asarray(columns, np.float64)  # [rows, vocab]
    rows, vocab = cols.shape
    hid = rows + 2
    w = np.zeros((vocab, hid))
    h = np.zeros((rows, hid))
    for r in range(rows):
        w[:, r] = cols[r]
        h[r, r] = 1.0
    return bits(h), bits(w)


def pin_lm_head_hand():
    """Hand-worked tokens and confidences: a dominant logit, tied maxima (lower
    id), uniform logits (1/V), logits past exp's range, the maximum last."""
    gd = golden("lm_head_hand.json")
    for c in gd["cases"]:
        h, w = _one_hot_head([c["logits"]])
        tok, conf, _ = O.lm_head_confidence(h, w)
        want = eval(c["conf"], {"__builtins__": {}}, {"exp": math.exp})
        assert int(tok[0]) == c["token"], (c, tok)
        assert abs(conf[0] - want) <= 1e-12 * want, (c, conf[0], want)


def pin_lm_head_brute(seed=13):
    """Tiny random heads against pure-Python logits, argmax and softmax."""
    g = np.random.default_rng(seed)
    for _ in range(20):
        rows, vocab, hid = int(g.integers(1, 5)), int(g.integers(1, 9)), int(g.integers(1, 6))
        h = bits(np.round(g.standard_normal((rows, hid)) * 8) / 8)
        w = bits(np.round(g.standard_normal((vocab, hid)) * 8) / 8)
        tok, conf, _ = O.lm_head_confidence(h, w)
        hf, wf = O.bf16_bits_to_f64(h), O.bf16_bits_to_f64(w)
        for r in range(rows):
            z = [sum(float(hf[r, k]) * float(wf[v, k]) for k in range(hid)) for v in range(vocab)]
            best = max(range(vocab), key=lambda v: (z[v], -v))
            p = math.exp(z[best]) / sum(math.exp(zv) for zv in z)
            assert int(tok[r]) == best and abs(conf[r] - p) <= 1e-12, (r, z, tok[r], conf[r], p)


def pin_verify_chain_hand():
    """Draft tokens from the draft rows, tokens and confidences from the mask
    rows, then the accept scan (hand-worked in the fixture)."""
    gd = golden("lm_head_hand.json")["chain"]
    # vocab 4; logits built so the argmax and the confidence are known:
    # confidence c for token t with the other three logits at 0 needs
    # exp(a) / (3 + exp(a)) = c, i.e. a = ln(3c / (1 - c)); rounded to bf16 the
    # probability moves a little but stays on the same side of 0.5.
    def row(t, c):
        a = math.log(3 * c / (1 - c))
        z = [0.0] * 4
        z[t] = float(O.bf16_bits_to_f64(O.f64_to_bf16_bits(a)))
        return z
    draft = [row(1, 0.9), row(2, 0.9), row(0, 0.9), row(3, 0.9), row(3, 0.9), row(1, 0.9)]
    mask = [row(1, 0.8), row(2, 0.6), row(1, 0.9), row(3, 0.9), row(3, 0.4), row(1, 0.9)]
    hd, w_d = _one_hot_head(draft)
    hm, w_m = _one_hot_head(mask)
    # one head for both views: stack the two weights' columns
    w = np.concatenate([O.bf16_bits_to_f64(w_d), O.bf16_bits_to_f64(w_m)], axis=1)
    hdd = np.concatenate([O.bf16_bits_to_f64(hd), np.zeros_like(O.bf16_bits_to_f64(hm))], axis=1)
    hmm = np.concatenate([np.zeros_like(O.bf16_bits_to_f64(hd)), O.bf16_bits_to_f64(hm)], axis=1)
    dtok, mtok, conf, acc = O.verify_chain(bits(hdd), bits(hmm), bits(w), 2, 3,
                                           np.float32(gd["threshold"]))
    assert dtok.tolist() == [[1, 2, 0], [3, 3, 1]], dtok
    assert mtok.tolist() == [[1, 2, 1], [3, 3, 1]], mtok
    assert acc.tolist() == gd["expect_accept"], acc


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
