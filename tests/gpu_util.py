"""Helpers for the GPU parity tests: upload a synthetic workload, run the HIP path
through the C ABI, and compare with the CPU oracle.

Tolerances (floating point): max|d| <= 2e-2 * max|ref| and rel-L2 <= 5e-3 for
bf16-in / fp32-accumulate outputs and the written K/V.  Integers: bit-exact.
"""

from __future__ import annotations

import numpy as np
import torch

import kv_cache_attention_flash_amd as fd
import oracle as O

TOL_MAX = 2e-2
TOL_L2 = 5e-3


def bf16_tensor(bits: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def bits_of(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def i32(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)


def assert_close(got, ref, what):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    if ref.size == 0:
        return
    scale = np.max(np.abs(ref))
    err = np.max(np.abs(got - ref))
    l2 = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)
    assert err <= TOL_MAX * scale + 1e-30, f"{what}: max|d| {err:.3e} > {TOL_MAX} * {scale:.3e}"
    assert l2 <= TOL_L2, f"{what}: rel-L2 {l2:.3e} > {TOL_L2}"
    return err / max(scale, 1e-300), l2


class GpuRun:
    """A workload resident on the GPU and the outputs of one step."""

    def __init__(self, wl, dev="cuda:0", x=None, w=None, k=None, v=None, block_table=None):
        self.wl = wl
        self.dev = dev
        self.x = x if x is not None else bf16_tensor(wl.x, dev)
        self.w = w if w is not None else bf16_tensor(wl.w, dev)
        kc = k if k is not None else bf16_tensor(wl.k_cache, dev)
        vc = v if v is not None else bf16_tensor(wl.v_cache, dev)
        bt = block_table if block_table is not None else wl.block_table
        self.cache = fd.PagedKVCache(kc, vc, i32(bt, dev))
        self.cu = i32(wl.cu_rows, dev)
        self.pos = i32(wl.positions, dev)
        self.slots = i32(wl.slots, dev)
        self.kv_len = i32(wl.kv_len, dev)
        self.views = i32(wl.views, dev) if wl.views is not None else None
        rows_per_seq = np.diff(wl.cu_rows)
        self.max_rows = int(rows_per_seq.max()) if len(rows_per_seq) else 0

    def step(self, topb=None, stream=None, unfused=False):
        """flash_cache_step (or, with ``unfused``, its three-launch ablation
        flash_cache_step_unfused) -> scheduled_attention (+ mass) -> track_topb."""
        wl = self.wl
        topb = wl.topb if topb is None else topb
        fc = fd.flash_cache_step_unfused if unfused else fd.flash_cache_step
        q, sm = fc(self.cache, self.x, self.w, self.cu, self.pos, self.slots, wl.rope_base,
                   stream=stream)
        out, mass = fd.scheduled_attention(self.cache, q, self.cu, self.kv_len, wl.max_kv_len,
                                           self.max_rows, views=self.views,
                                           want_mass=bool(topb), stream=stream)
        idx = fd.track_topb(mass, self.kv_len, topb, stream=stream) if topb else None
        torch.cuda.synchronize()
        self.q, self.slot_mapping, self.out, self.mass, self.idx = q, sm, out, mass, idx
        return self


def oracle_step(wl, topb=None, seqs=None, k_cache=None, v_cache=None):
    """Independent oracle for all sequences, or for the subset ``seqs`` (rows of
    those sequences only; their cache blocks are disjoint from the others)."""
    topb = wl.topb if topb is None else topb
    kc = wl.k_cache if k_cache is None else k_cache
    vc = wl.v_cache if v_cache is None else v_cache
    if seqs is None:
        sub = dict(x=wl.x, positions=wl.positions, slots=wl.slots, cu=wl.cu_rows,
                   bt=wl.block_table, kv_len=wl.kv_len, views=wl.views)
        rows = np.arange(wl.rows)
    else:
        rows = np.concatenate([np.arange(wl.cu_rows[b], wl.cu_rows[b + 1]) for b in seqs])
        cu = np.cumsum([0] + [wl.cu_rows[b + 1] - wl.cu_rows[b] for b in seqs]).astype(np.int32)
        sub = dict(x=wl.x[rows], positions=wl.positions[rows], slots=wl.slots[rows], cu=cu,
                   bt=wl.block_table[seqs], kv_len=wl.kv_len[seqs],
                   views=None if wl.views is None else wl.views[seqs])
    res = O.decode_step(sub["x"], wl.w, wl.num_heads, wl.head_dim, sub["positions"], wl.rope_base,
                        sub["cu"], sub["slots"], sub["bt"], wl.block_size, kc, vc, sub["kv_len"],
                        views=sub["views"], topb=topb, mass_stride=wl.max_kv_len)
    res["rows"] = rows
    res["sub"] = sub
    return res


def written_mask(wl, slot_mapping, num_blocks):
    m = np.zeros(num_blocks * wl.block_size, dtype=bool)
    m[np.asarray(slot_mapping, dtype=np.int64)] = True
    return m.reshape(num_blocks, wl.block_size)


def compare_cache(wl, ref_res, gpu_k_bits, gpu_v_bits, init_k, init_v, seqs=None):
    """Written K/V within tolerance of the oracle; every other byte unchanged."""
    ps = ref_res["slot_mapping"]
    blk, off = ps // wl.block_size, ps % wl.block_size
    assert_close(O.bf16_bits_to_f64(gpu_k_bits[blk, :, off, :]),
                 O.bf16_bits_to_f64(ref_res["k_cache"][blk, :, off, :]), "written K")
    assert_close(O.bf16_bits_to_f64(gpu_v_bits[blk, :, off, :]),
                 O.bf16_bits_to_f64(ref_res["v_cache"][blk, :, off, :]), "written V")
    if seqs is None:
        wm = written_mask(wl, ps, gpu_k_bits.shape[0])
        keep = ~wm  # [num_blocks, bs]
        assert np.array_equal(gpu_k_bits.transpose(0, 2, 1, 3)[keep],
                              init_k.transpose(0, 2, 1, 3)[keep]), "K bytes outside active slots changed"
        assert np.array_equal(gpu_v_bits.transpose(0, 2, 1, 3)[keep],
                              init_v.transpose(0, 2, 1, 3)[keep]), "V bytes outside active slots changed"


def certify_topb(gpu_idx, staged_mass, kv_len, topb, what):
    """Every index where the GPU's set differs from the staged oracle's must be a
    near-tie: |m(i) - m(j)| <= 1e-5 * max m.  Returns the number of near-ties."""
    near = 0
    for b in range(len(kv_len)):
        ref = O.top_b(staged_mass[b], int(kv_len[b]), topb)
        got = gpu_idx[b]
        if np.array_equal(ref, got):
            continue
        a = set(int(v) for v in got if v >= 0)
        r = set(int(v) for v in ref if v >= 0)
        only_g, only_r = sorted(a - r), sorted(r - a)
        assert len(only_g) == len(only_r), (what, b)
        m = staged_mass[b]
        tol = 1e-5 * float(np.max(m[:int(kv_len[b])]))
        for i, j in zip(only_g, only_r):
            assert abs(m[i] - m[j]) <= tol, (what, b, i, j, m[i], m[j], tol)
            near += 1
    return near
