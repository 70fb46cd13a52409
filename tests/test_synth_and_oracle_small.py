"""Synthetic workloads are deterministic and well-formed; the oracle runs on the
small ones and satisfies its invariants there.  No GPU."""

import numpy as np
import pytest

import oracle as O
import synth

SMALL = ["tiny_h256_l128", "small_ragged_b5", "small_verify_b3", "small_d64_rows150",
         "small_splitk_h1024", "small_long_l1500"]


def _check_layout(wl):
    cu = wl.cu_rows
    assert cu[0] == 0 and np.all(np.diff(cu) >= 0) and cu[-1] == len(wl.positions) == len(wl.slots)
    for b in range(wl.batch):
        s = wl.slots[cu[b]:cu[b + 1]]
        assert len(np.unique(s)) == len(s), "duplicate slot inside a sequence"
        assert np.all(s >= 0) and np.all(s < wl.kv_len[b])
        nblk = -(-int(wl.kv_len[b]) // wl.block_size)
        assert nblk <= wl.max_blocks
        if wl.views is not None and wl.views[b, 1] > 0:
            w0, w, d0 = wl.views[b]
            assert w0 + w <= d0 and d0 + w <= wl.kv_len[b]
    used = np.concatenate([wl.block_table[b, :-(-int(wl.kv_len[b]) // wl.block_size)]
                           for b in range(wl.batch)])
    assert len(np.unique(used)) == len(used) and used.max() < wl.num_blocks


@pytest.mark.parametrize("name", sorted(synth.WORKLOADS))
def test_layout_only(name):
    wl = synth.WORKLOADS[name](materialize=False)
    _check_layout(wl)


def test_stack_layout():
    wl = synth.llada8b_stack32_layout()
    _check_layout(wl)
    assert wl.rows == 1024 and wl.batch == 16 and wl.num_blocks == 2048


def test_full_size_shapes():
    assert synth.llada8b_b1(materialize=False).rows == 64
    assert synth.llada8b_ragged_b32(materialize=False).rows == 2048
    v = synth.llada8b_verify_b8(materialize=False)
    assert v.rows == 512 and v.num_blocks == 264 and v.verify["draft"].shape == (8 + 6, 32)


@pytest.mark.parametrize("name", SMALL)
def test_deterministic_and_oracle_invariants(name):
    a = synth.WORKLOADS[name]()
    b = synth.WORKLOADS[name]()
    for f in ("x", "w", "k_cache", "v_cache", "block_table", "positions"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    res = O.decode_step(a.x, a.w, a.num_heads, a.head_dim, a.positions, a.rope_base, a.cu_rows,
                        a.slots, a.block_table, a.block_size, a.k_cache, a.v_cache, a.kv_len,
                        views=a.views, topb=a.topb)
    for bb in range(a.batch):
        rb = a.cu_rows[bb + 1] - a.cu_rows[bb]
        assert abs(res["mass"][bb].sum() - a.num_heads * rb) <= 1e-9 * max(1, a.num_heads * rb)
        sel = res["topb"][bb]
        assert np.all(np.diff(sel[sel >= 0]) > 0)


def test_verify_scan_statistics():
    v = synth.verify_scan_inputs(4, 4000, 32, crafted=False)
    agree = np.mean(v["draft"] == v["mask"])
    assert 0.68 < agree < 0.72
    lens = [O.accept_length(d, m, c, v["threshold"]) for d, m, c in zip(v["draft"], v["mask"], v["conf"])]
    # per-position pass rate 0.7 * 0.1: E[len] = sum_k 0.07^k ~ 0.0753, P(len = 0) = 0.93
    assert abs(np.mean(lens) - 0.0753) < 0.02
    assert abs(np.mean(np.array(lens) == 0) - 0.93) < 0.015


def test_verify_crafted_rows():
    v = synth.verify_scan_inputs(4, 2, 32)
    d, m, c, t = v["draft"][2:], v["mask"][2:], v["conf"][2:], v["threshold"]
    got = [O.accept_length(d[i], m[i], c[i], t) for i in range(len(d))]
    assert got == [32, 5, 0, 31, 32, 9]
