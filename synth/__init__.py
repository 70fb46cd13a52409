"""Seeded synthetic inputs for the per-layer Flash-dLLM decode step.

This module only draws inputs: random hidden states, weights and cache contents,
row layouts and block tables.  It holds none of the method's arithmetic, so both
the GPU library's tests/benchmark and the CPU oracle can take their inputs from
it without sharing any computation.

Recipe: every stream is ``numpy.random.default_rng([workload_id, layer, stream])``
with streams 0 X, 1 W, 2 K cache, 3 V cache, 4 window/tracked positions,
5 block permutation, 6 lengths, 8 draft tokens, 9 agreement, 10 replacement
tokens, 11 confidences, 12 and 13 the committed- and masked-token hidden-state
tables of a multi-step loop (whose per-step scan draws use the step as the
``layer`` key), 14 the LM-head weight, 15 the mask rows' final hidden states,
16 the draft rows' perturbation.  Real values are drawn as standard normals in fp32
(the weight scaled by 0.02 in fp32) and rounded to bf16 by torch's CPU cast.
The large 32-layer stack draws its tensors on the GPU with torch's seeded
generator instead (host generation of ~19 G values would take minutes); those
tensors are copied back to the host when the oracle needs them.

Shapes follow the pages' LLaDA-8B-class decode settings: hidden 4096, 32 heads x
128, rotary base 500000, paged cache with block size 32.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

STREAM_X, STREAM_W, STREAM_K, STREAM_V, STREAM_POS, STREAM_PERM, STREAM_LEN = 0, 1, 2, 3, 4, 5, 6
STREAM_DRAFT, STREAM_AGREE, STREAM_REPL, STREAM_CONF = 8, 9, 10, 11
STREAM_HID_COMMITTED, STREAM_HID_MASKED = 12, 13
STREAM_LM_W, STREAM_LM_H, STREAM_LM_NOISE = 14, 15, 16


def rng(workload_id: int, layer: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([int(workload_id), int(layer), int(stream)])


def to_bf16_bits(a_f32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns via torch's CPU cast (round to nearest even)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a_f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def normal_bf16(workload_id, layer, stream, shape, scale=1.0) -> np.ndarray:
    g = rng(workload_id, layer, stream)
    a = g.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        a *= np.float32(scale)
    return to_bf16_bits(a)


@dataclasses.dataclass
class SeqSpec:
    """Active rows of one sequence.

    Plain sequence: ``window`` = (w0, W) window rows at positions w0..w0+W-1,
    then ``tracked`` rows (ascending positions); every row's cache slot equals
    its position.  Two-view sequence (``draft_start`` = d0 set): W draft rows at
    positions w0+i writing slots d0+i, then W mask rows at positions w0+i
    writing slots w0+i, then tracked rows.
    """
    kv_len: int
    window: tuple = (0, 0)
    tracked: tuple = ()
    draft_start: Optional[int] = None


@dataclasses.dataclass
class Workload:
    name: str
    workload_id: int
    hid: int
    num_heads: int
    head_dim: int
    block_size: int
    rope_base: float
    kv_len: np.ndarray        # int32 [batch]
    cu_rows: np.ndarray       # int32 [batch+1]
    positions: np.ndarray     # int32 [R]
    slots: np.ndarray         # int32 [R]
    block_table: np.ndarray   # int32 [batch, max_blocks]
    num_blocks: int
    views: Optional[np.ndarray]  # int32 [batch, 3] or None
    topb: int                 # 0: no mass / tracking-set selection
    layers: int = 1
    x: Optional[np.ndarray] = None        # bf16 bits [R, hid]
    w: Optional[np.ndarray] = None        # bf16 bits [3HD, hid]
    k_cache: Optional[np.ndarray] = None  # bf16 bits [num_blocks, H, bs, D]
    v_cache: Optional[np.ndarray] = None
    verify: Optional[dict] = None         # draft, mask, conf (fp32), threshold (fp32)

    @property
    def batch(self) -> int:
        return len(self.kv_len)

    @property
    def rows(self) -> int:
        return int(self.cu_rows[-1])

    @property
    def max_blocks(self) -> int:
        return self.block_table.shape[1]

    @property
    def max_kv_len(self) -> int:
        return int(self.kv_len.max()) if len(self.kv_len) else 0


def layout(workload_id: int, specs, block_size: int, layer: int = 0):
    """Row arrays, two-view descriptors and a seeded permuted block table."""
    batch = len(specs)
    cu = [0]
    pos, slots = [], []
    views = np.zeros((batch, 3), np.int32)
    any_view = False
    for b, s in enumerate(specs):
        w0, wl = s.window
        if s.draft_start is not None:
            any_view = True
            views[b] = (w0, wl, s.draft_start)
            pos += [w0 + i for i in range(wl)]
            slots += [s.draft_start + i for i in range(wl)]
            pos += [w0 + i for i in range(wl)]
            slots += [w0 + i for i in range(wl)]
        else:
            pos += [w0 + i for i in range(wl)]
            slots += [w0 + i for i in range(wl)]
        tr = sorted(int(t) for t in s.tracked)
        pos += tr
        slots += tr
        cu.append(len(pos))
    kv_len = np.array([s.kv_len for s in specs], np.int32)
    nblk = [-(-int(s.kv_len) // block_size) for s in specs]
    num_blocks = int(sum(nblk))
    max_blocks = max(nblk + [1])
    perm = rng(workload_id, layer, STREAM_PERM).permutation(max(num_blocks, 1))
    bt = np.zeros((batch, max_blocks), np.int32)  # unused entries: 0 (never read)
    off = 0
    for b, n in enumerate(nblk):
        bt[b, :n] = perm[off:off + n]
        off += n
    return (kv_len, np.array(cu, np.int32), np.array(pos, np.int32),
            np.array(slots, np.int32), bt, max(num_blocks, 1),
            views if any_view else None)


def build(name, workload_id, hid, num_heads, head_dim, block_size, rope_base, specs,
          topb, layer=0, layers=1, materialize=True) -> Workload:
    kv_len, cu, pos, slots, bt, nb, views = layout(workload_id, specs, block_size, layer)
    wl = Workload(name, workload_id, hid, num_heads, head_dim, block_size, rope_base,
                  kv_len, cu, pos, slots, bt, nb, views, topb, layers)
    if materialize:
        fill_layer(wl, layer)
    return wl


def fill_layer(wl: Workload, layer: int) -> Workload:
    """Draw X, W and the two cache pools of one layer on the host."""
    r, hd = wl.rows, wl.num_heads * wl.head_dim
    wid = wl.workload_id
    wl.x = normal_bf16(wid, layer, STREAM_X, (r, wl.hid))
    wl.w = normal_bf16(wid, layer, STREAM_W, (3 * hd, wl.hid), scale=0.02)
    shape = (wl.num_blocks, wl.num_heads, wl.block_size, wl.head_dim)
    wl.k_cache = normal_bf16(wid, layer, STREAM_K, shape)
    wl.v_cache = normal_bf16(wid, layer, STREAM_V, shape)
    return wl


def distinct(g: np.random.Generator, lo: int, hi: int, n: int):
    """n distinct integers from [lo, hi), ascending."""
    n = min(n, hi - lo)
    return tuple(sorted(int(v) for v in g.choice(np.arange(lo, hi), size=n, replace=False)))


# ---------------------------------------------------------------------------
# The five decode-step workloads
# ---------------------------------------------------------------------------


def tiny_h256(materialize=True) -> Workload:
    """hidden 256, 4 heads x 64, one sequence, cache 128 (64 prompt + 64
    generated), window 64..79, 8 tracked from 0..63, base 1e4, top-8."""
    g = rng(1, 0, STREAM_POS)
    spec = SeqSpec(kv_len=128, window=(64, 16), tracked=distinct(g, 0, 64, 8))
    return build("tiny_h256_l128", 1, 256, 4, 64, 32, 1.0e4, [spec], topb=8,
                 materialize=materialize)


def llada8b_b1(materialize=True) -> Workload:
    """LLaDA-8B-class layer, batch 1: hidden 4096, 32 x 128, cache 768
    (256 prompt + 512 generated), window 256..287 + 32 tracked from [0, 256),
    64 active rows, base 5e5; the tracking set (32) is re-selected."""
    g = rng(2, 0, STREAM_POS)
    spec = SeqSpec(kv_len=768, window=(256, 32), tracked=distinct(g, 0, 256, 32))
    return build("llada8b_b1_l768", 2, 4096, 32, 128, 32, 5.0e5, [spec], topb=32,
                 materialize=materialize)


def llada8b_ragged_b32(materialize=True) -> Workload:
    """Same layer, batch 32, cache lengths U{512..1024}; even sequences in the
    refresh stage (block-aligned 32-row window), odd ones in the update stage
    (window at any offset); 32 tracked rows each; top-32 per sequence."""
    gl = rng(3, 0, STREAM_LEN)
    gp = rng(3, 0, STREAM_POS)
    specs = []
    for b in range(32):
        length = int(gl.integers(512, 1025))
        if b % 2 == 0:
            w0 = 32 * int(gp.integers(1, length // 32))
        else:
            w0 = int(gp.integers(32, length - 32 + 1))
        specs.append(SeqSpec(kv_len=length, window=(w0, 32),
                             tracked=distinct(gp, 0, w0, 32)))
    return build("llada8b_ragged_b32", 3, 4096, 32, 128, 32, 5.0e5, specs, topb=32,
                 materialize=materialize)


def verify_scan_inputs(workload_id: int, batch: int, window: int, crafted=True):
    """Draft tokens, mask-view argmax tokens (about 70 % agreement) and fp32
    confidences U(0,1) for the accept scan, threshold 0.9f; plus crafted rows
    that exercise long prefixes, which the random draws almost never do."""
    v = 1 << 20
    draft = rng(workload_id, 0, STREAM_DRAFT).integers(0, v, size=(batch, window)).astype(np.int32)
    agree = rng(workload_id, 0, STREAM_AGREE).random(size=(batch, window)) < 0.7
    repl = rng(workload_id, 0, STREAM_REPL).integers(0, v - 1, size=(batch, window))
    mask = np.where(agree, draft, (draft.astype(np.int64) + 1 + repl) % v).astype(np.int32)
    conf = rng(workload_id, 0, STREAM_CONF).random(size=(batch, window), dtype=np.float32)
    thr = np.float32(0.9)
    if crafted:
        rows_d, rows_m, rows_c = [], [], []
        base_d = np.arange(window, dtype=np.int32) * 7 + 11
        hi = np.full(window, 0.95, np.float32)
        # all accepted
        rows_d.append(base_d); rows_m.append(base_d.copy()); rows_c.append(hi.copy())
        # confidence exactly at the threshold at position 5 (strict comparison stops there)
        c = hi.copy(); c[min(5, window - 1)] = thr
        rows_d.append(base_d); rows_m.append(base_d.copy()); rows_c.append(c)
        # first position disagrees
        m = base_d.copy(); m[0] += 1
        rows_d.append(base_d); rows_m.append(m); rows_c.append(hi.copy())
        # disagreement at the last position
        m = base_d.copy(); m[-1] += 1
        rows_d.append(base_d); rows_m.append(m); rows_c.append(hi.copy())
        # the next float above the threshold passes
        c = hi.copy(); c[:] = np.nextafter(thr, np.float32(1.0))
        rows_d.append(base_d); rows_m.append(base_d.copy()); rows_c.append(c)
        # a NaN confidence fails
        c = hi.copy(); c[min(9, window - 1)] = np.float32(np.nan)
        rows_d.append(base_d); rows_m.append(base_d.copy()); rows_c.append(c)
        draft = np.concatenate([draft, np.stack(rows_d)])
        mask = np.concatenate([mask, np.stack(rows_m)])
        conf = np.concatenate([conf, np.stack(rows_c)])
    return dict(draft=np.ascontiguousarray(draft), mask=np.ascontiguousarray(mask),
                conf=np.ascontiguousarray(conf), threshold=thr)


def llada8b_verify_b8(materialize=True) -> Workload:
    """Two-view verify step: batch 8, context 1024 plus one draft block
    (33 blocks per sequence), block-aligned window of 32; 32 draft rows and
    32 mask rows per sequence at the same positions; then the accept scan."""
    gp = rng(4, 0, STREAM_POS)
    specs = []
    for _ in range(8):
        w0 = 32 * int(gp.integers(1, 32))
        specs.append(SeqSpec(kv_len=1024 + 32, window=(w0, 32), draft_start=1024))
    wl = build("llada8b_verify_b8", 4, 4096, 32, 128, 32, 5.0e5, specs, topb=0,
               materialize=materialize)
    wl.verify = verify_scan_inputs(4, 8, 32)
    return wl


def llada8b_stack32_layout() -> Workload:
    """32-layer stack, batch 16, cache 4096 per sequence: window of 32 at
    w0 ~ U{32..4064} (shared by all layers) + 32 tracked from [0, w0); top-32
    re-selected per layer.  Tensors are drawn per layer on the GPU
    (``stack_layer_tensors``)."""
    gp = rng(5, 0, STREAM_POS)
    specs = []
    for _ in range(16):
        w0 = int(gp.integers(32, 4064 + 1))
        specs.append(SeqSpec(kv_len=4096, window=(w0, 32), tracked=distinct(gp, 0, w0, 32)))
    return build("llada8b_stack32_b16_l4096", 5, 4096, 32, 128, 32, 5.0e5, specs, topb=32,
                 layers=32, materialize=False)


def stack_layer_tensors(wl: Workload, layer: int, device):
    """Draw one layer's X, W, K and V pools as torch bf16 tensors on ``device``
    with torch's seeded generator (seed = workload*1e6 + layer*100 + stream)."""
    import torch
    hd = wl.num_heads * wl.head_dim
    shapes = {STREAM_X: ((wl.rows, wl.hid), 1.0), STREAM_W: ((3 * hd, wl.hid), 0.02),
              STREAM_K: ((wl.num_blocks, wl.num_heads, wl.block_size, wl.head_dim), 1.0),
              STREAM_V: ((wl.num_blocks, wl.num_heads, wl.block_size, wl.head_dim), 1.0)}
    out = {}
    for stream, (shape, scale) in shapes.items():
        g = torch.Generator(device=device)
        g.manual_seed(wl.workload_id * 1_000_000 + layer * 100 + stream)
        t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        if scale != 1.0:
            t.mul_(scale)
        out[stream] = t.to(torch.bfloat16)
        del t
    return out[STREAM_X], out[STREAM_W], out[STREAM_K], out[STREAM_V]


# ---------------------------------------------------------------------------
# Small workloads for element-wise parity: several tiles and ragged tails
# ---------------------------------------------------------------------------


def small_ragged(materialize=True) -> Workload:
    """hidden 512, 4 x 128, batch 5 with lengths that are not multiples of the
    block size, refresh and update windows, varying tracked counts, top-8."""
    g = rng(11, 0, STREAM_POS)
    lens = [200, 77, 33, 160, 96]
    specs = []
    for b, length in enumerate(lens):
        if b % 2 == 0:
            w0 = 32 * int(g.integers(0, max(1, length // 32)))
            wl = min(32, length - w0)
        else:
            w0 = int(g.integers(0, length - 16 + 1))
            wl = 16
        nt = int(g.integers(0, 13))
        pool = [p for p in range(length) if not (w0 <= p < w0 + wl)]
        tr = tuple(sorted(int(p) for p in g.choice(pool, size=min(nt, len(pool)), replace=False)))
        specs.append(SeqSpec(kv_len=length, window=(w0, wl), tracked=tr))
    return build("small_ragged_b5", 11, 512, 4, 128, 32, 5.0e5, specs, topb=8,
                 materialize=materialize)


def small_verify(materialize=True) -> Workload:
    """Two-view step at small size: hidden 256, 2 x 64, batch 3, contexts of
    different lengths, windows of 16 at block- and non-block-aligned offsets."""
    specs = [SeqSpec(kv_len=96 + 16, window=(32, 16), draft_start=96),
             SeqSpec(kv_len=150 + 16, window=(70, 16), draft_start=150),
             SeqSpec(kv_len=64 + 16, window=(0, 16), draft_start=64)]
    wl = build("small_verify_b3", 12, 256, 2, 64, 32, 1.0e4, specs, topb=8,
               materialize=materialize)
    wl.verify = verify_scan_inputs(12, 3, 16)
    return wl


def small_d64_many_rows(materialize=True) -> Workload:
    """head_dim 64, batch 2, one sequence with 150 active rows (more than one row
    tile) and a long cache, one with 1 row; hidden 384."""
    g = rng(13, 0, STREAM_POS)
    specs = [SeqSpec(kv_len=300, window=(100, 64), tracked=distinct(g, 0, 100, 86)),
             SeqSpec(kv_len=45, window=(44, 1))]
    return build("small_d64_rows150", 13, 384, 6, 64, 32, 1.0e4, specs, topb=16,
                 materialize=materialize)


def small_splitk(materialize=True) -> Workload:
    """Few rows (40) on a narrow layer (hidden 1024, 2 x 128) so the projection
    splits its reduction across workgroups; batch 2, lengths 96 and 70."""
    g = rng(14, 0, STREAM_POS)
    specs = [SeqSpec(kv_len=96, window=(64, 16), tracked=distinct(g, 0, 64, 8)),
             SeqSpec(kv_len=70, window=(40, 8), tracked=distinct(g, 0, 40, 8))]
    return build("small_splitk_h1024", 14, 1024, 2, 128, 32, 1.0e4, specs, topb=8,
                 materialize=materialize)


def small_long(materialize=True) -> Workload:
    """Caches past 1024 keys on a narrow layer (hidden 256, 2 x 64): batch 2,
    lengths 1500 and 1100 (not multiples of the block size), 24 rows each,
    top-8."""
    g = rng(15, 0, STREAM_POS)
    specs = [SeqSpec(kv_len=1500, window=(1200, 16), tracked=distinct(g, 0, 1200, 8)),
             SeqSpec(kv_len=1100, window=(1050, 16), tracked=distinct(g, 0, 1050, 8))]
    return build("small_long_l1500", 15, 256, 2, 64, 32, 1.0e4, specs, topb=8,
                 materialize=materialize)


# ---------------------------------------------------------------------------
# Multi-step loop workloads
# ---------------------------------------------------------------------------


@dataclasses.dataclass
class LoopWorkload:
    """Initial state and inputs of a multi-step decoding loop of one layer.

    ``frontier0`` [batch] is each sequence's first uncommitted position,
    ``tracked0`` [batch, topb] the initial tracking set (ascending, -1 padded).
    Hidden states come from two tables bf16 [batch, max_len, hid]: a
    committed-token row and a masked-token row per position.  ``scan`` holds
    each step's accept-scan inputs, [steps, batch, W] draft and mask-view
    tokens and fp32 confidences, and the threshold 0.9f.
    """
    name: str
    workload_id: int
    hid: int
    num_heads: int
    head_dim: int
    block_size: int
    rope_base: float
    kv_len: np.ndarray
    block_table: np.ndarray
    num_blocks: int
    frontier0: np.ndarray
    tracked0: np.ndarray
    window_len: int
    topb: int
    refresh_period: int
    steps: int
    scan: dict
    w: Optional[np.ndarray] = None
    k_cache: Optional[np.ndarray] = None
    v_cache: Optional[np.ndarray] = None
    hidden_committed: Optional[np.ndarray] = None
    hidden_masked: Optional[np.ndarray] = None

    @property
    def batch(self) -> int:
        return len(self.kv_len)

    @property
    def max_len(self) -> int:
        return int(self.kv_len.max())


def loop_scan_inputs(workload_id: int, steps: int, batch: int, window: int):
    """Per-step accept-scan inputs: draft tokens U{0..2^20-1}; the mask-view
    argmax agrees with probability 0.98 (else a different token); confidences
    0.885 + 0.115 U(0,1) in fp32; threshold 0.9f.  A position then passes with
    probability about 0.85, so about 5.7 tokens are accepted per step, the
    figure the pages report for Flash-Verify."""
    v = 1 << 20
    shape = (batch, window)
    draft, mask, conf = [], [], []
    for t in range(steps):
        d = rng(workload_id, t, STREAM_DRAFT).integers(0, v, size=shape).astype(np.int32)
        agree = rng(workload_id, t, STREAM_AGREE).random(size=shape) < 0.98
        repl = rng(workload_id, t, STREAM_REPL).integers(0, v - 1, size=shape)
        m = np.where(agree, d, (d.astype(np.int64) + 1 + repl) % v).astype(np.int32)
        u = rng(workload_id, t, STREAM_CONF).random(size=shape, dtype=np.float32)
        c = (np.float32(0.885) + np.float32(0.115) * u).astype(np.float32)
        draft.append(d); mask.append(m); conf.append(c)
    return dict(draft=np.stack(draft), mask=np.stack(mask), conf=np.stack(conf),
                threshold=np.float32(0.9))


def build_loop(name, workload_id, hid, num_heads, head_dim, block_size, rope_base, kv_len,
               frontier0, tracked0, window_len, topb, refresh_period, steps,
               materialize=True) -> LoopWorkload:
    specs = [SeqSpec(kv_len=int(n)) for n in kv_len]
    kvl, _, _, _, bt, nb, _ = layout(workload_id, specs, block_size)
    tr = np.full((len(kv_len), topb), -1, np.int32)
    for b, t in enumerate(tracked0):
        t = sorted(int(v) for v in t)[:topb]
        tr[b, :len(t)] = t
    wl = LoopWorkload(name, workload_id, hid, num_heads, head_dim, block_size, rope_base, kvl,
                      bt, nb, np.array(frontier0, np.int32), tr, window_len, topb,
                      refresh_period, steps,
                      loop_scan_inputs(workload_id, steps, len(kv_len), window_len))
    if materialize:
        hd = num_heads * head_dim
        wl.w = normal_bf16(workload_id, 0, STREAM_W, (3 * hd, hid), scale=0.02)
        shape = (nb, num_heads, block_size, head_dim)
        wl.k_cache = normal_bf16(workload_id, 0, STREAM_K, shape)
        wl.v_cache = normal_bf16(workload_id, 0, STREAM_V, shape)
        tshape = (len(kv_len), wl.max_len, hid)
        wl.hidden_committed = normal_bf16(workload_id, 0, STREAM_HID_COMMITTED, tshape)
        wl.hidden_masked = normal_bf16(workload_id, 0, STREAM_HID_MASKED, tshape)
    return wl


def small_loop_b4(materialize=True) -> LoopWorkload:
    """Loop on a narrow layer (hidden 256, 2 x 64): batch 4, cache lengths
    150, 77, 40, 200; one sequence finished from the start, one finishing
    within two steps; window 16, budget 8, refresh every third step, 6 steps."""
    g = rng(21, 0, STREAM_POS)
    f0 = [60, 70, 40, 100]
    tracked = [distinct(g, 0, f, 8) for f in f0]
    return build_loop("small_loop_b4", 21, 256, 2, 64, 32, 1.0e4, [150, 77, 40, 200], f0,
                      tracked, 16, 8, 3, 6, materialize)


def small_loop_d128(materialize=True) -> LoopWorkload:
    """Loop with head_dim 128 (hidden 512, 4 x 128): batch 3, lengths 300, 129,
    64, one sequence starting at position 0 with an empty tracking set, one
    finishing within the run; window 32, budget 16, refresh every other step,
    5 steps."""
    g = rng(22, 0, STREAM_POS)
    f0 = [40, 118, 0]
    tracked = [distinct(g, 0, f, 16) for f in f0]
    return build_loop("small_loop_d128", 22, 512, 4, 128, 32, 5.0e5, [300, 129, 64], f0,
                      tracked, 32, 16, 2, 5, materialize)


def llada8b_loop_b32(materialize=False, steps=16) -> LoopWorkload:
    """The batch-32 ragged layer (hidden 4096, 32 x 128, lengths U{512..1024})
    run as a loop (16 steps unless ``steps`` says otherwise): each sequence
    starts at its window start with its
    32 tracked rows; window 32, budget 32, refresh every fourth step (stages
    staggered across the batch).  Tensors are drawn on the GPU
    (``loop_tensors``)."""
    base = llada8b_ragged_b32(materialize=False)
    f0, tracked = [], []
    cu = base.cu_rows
    for b in range(base.batch):
        rows = base.positions[cu[b]:cu[b + 1]]
        f0.append(int(rows[0]))
        tracked.append([int(p) for p in rows[32:]])
    return build_loop("llada8b_loop_b32", 23, 4096, 32, 128, 32, 5.0e5,
                      [int(n) for n in base.kv_len], f0, tracked, 32, 32, 4, steps, materialize)


def loop_tensors(wl: LoopWorkload, device):
    """torch bf16 tensors of a loop workload on ``device``: host draws when the
    workload is materialized, else torch's seeded generator on the device
    (seed = workload*1e6 + stream) for W, the cache pools and both tables."""
    import torch
    if wl.w is not None:
        def dev(a):
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
        return (dev(wl.w), dev(wl.k_cache), dev(wl.v_cache), dev(wl.hidden_committed),
                dev(wl.hidden_masked))
    hd = wl.num_heads * wl.head_dim
    cshape = (wl.num_blocks, wl.num_heads, wl.block_size, wl.head_dim)
    tshape = (wl.batch, wl.max_len, wl.hid)
    out = []
    for stream, shape, scale in ((STREAM_W, (3 * hd, wl.hid), 0.02), (STREAM_K, cshape, 1.0),
                                 (STREAM_V, cshape, 1.0), (STREAM_HID_COMMITTED, tshape, 1.0),
                                 (STREAM_HID_MASKED, tshape, 1.0)):
        g = torch.Generator(device=device)
        g.manual_seed(wl.workload_id * 1_000_000 + stream)
        t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        if scale != 1.0:
            t.mul_(scale)
        out.append(t.to(torch.bfloat16))
        del t
    return tuple(out)


# ---------------------------------------------------------------------------
# Mask-view confidence producer workloads (LM head)
# ---------------------------------------------------------------------------


@dataclasses.dataclass
class LmHeadWorkload:
    """Final hidden states of the window rows of a two-view step and an LM head.

    ``h_mask`` bf16 [batch*window, hid] are the mask rows; the draft rows
    ``h_draft`` are the same states plus ``noise`` x N(0,1) (drawn in fp32,
    then rounded), so the two views mostly agree.  ``w`` bf16 [vocab, hid] is
    N(0,1) x ``w_std``: with w_std = 16 / sqrt(hid) the logits have standard
    deviation about 16; over the 126464-token vocabulary the top token's
    probability then spreads over (0, 1) with a median near 0.87, so the 0.9f
    threshold splits the positions (a draft noise of 0.1 leaves about 3 in 4
    argmaxes unchanged).
    """
    name: str
    workload_id: int
    hid: int
    vocab: int
    batch: int
    window: int
    w_std: float
    noise: float
    threshold: np.float32 = np.float32(0.9)
    w: Optional[np.ndarray] = None
    h_mask: Optional[np.ndarray] = None
    h_draft: Optional[np.ndarray] = None

    @property
    def rows(self) -> int:
        return self.batch * self.window


def build_lm_head(name, workload_id, hid, vocab, batch, window, materialize=True):
    wl = LmHeadWorkload(name, workload_id, hid, vocab, batch, window,
                        w_std=16.0 / float(np.sqrt(hid)), noise=0.1)
    if materialize:
        wl.w = normal_bf16(workload_id, 0, STREAM_LM_W, (vocab, hid), scale=wl.w_std)
        base = rng(workload_id, 0, STREAM_LM_H).standard_normal((wl.rows, hid), dtype=np.float32)
        noise = rng(workload_id, 0, STREAM_LM_NOISE).standard_normal((wl.rows, hid),
                                                                     dtype=np.float32)
        wl.h_mask = to_bf16_bits(base)
        wl.h_draft = to_bf16_bits(base + np.float32(wl.noise) * noise)
    return wl


def tiny_lm_head(materialize=True) -> LmHeadWorkload:
    """Vocabulary 77 (less than one column tile), hidden 64, 2 sequences x 3 rows."""
    return build_lm_head("tiny_lmhead_v77", 31, 64, 77, 2, 3, materialize)


def small_lm_head(materialize=True) -> LmHeadWorkload:
    """Vocabulary 1000 (a ragged last column tile), hidden 256, 3 sequences x
    16 window rows (48 draft + 48 mask rows: a ragged row tile)."""
    return build_lm_head("small_lmhead_v1000", 32, 256, 1000, 3, 16, materialize)


def llada8b_lm_head_b8(materialize=False) -> LmHeadWorkload:
    """The two-view batch-8 step's window rows through an LLaDA-8B-class head:
    vocabulary 126464, hidden 4096, 8 sequences x 32 rows per view (256 draft
    + 256 mask rows).  Tensors are drawn on the GPU (``lm_head_tensors``)."""
    return build_lm_head("llada8b_lmhead_b8", 33, 4096, 126464, 8, 32, materialize)


def lm_head_tensors(wl: LmHeadWorkload, device):
    """(w, h_draft, h_mask) as torch bf16 tensors on ``device``: host draws when
    materialized, else torch's seeded generator on the device (seed =
    workload*1e6 + stream), the draft rows being the mask rows plus the noise."""
    import torch
    if wl.w is not None:
        def dev(a):
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
        return dev(wl.w), dev(wl.h_draft), dev(wl.h_mask)

    def draw(stream, shape):
        g = torch.Generator(device=device)
        g.manual_seed(wl.workload_id * 1_000_000 + stream)
        return torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    w = draw(STREAM_LM_W, (wl.vocab, wl.hid)).mul_(wl.w_std).to(torch.bfloat16)
    base = draw(STREAM_LM_H, (wl.rows, wl.hid))
    noise = draw(STREAM_LM_NOISE, (wl.rows, wl.hid))
    h_mask = base.to(torch.bfloat16)
    h_draft = base.add_(noise.mul_(wl.noise)).to(torch.bfloat16)
    return w, h_draft, h_mask


LM_HEAD_WORKLOADS = {
    "tiny_lmhead_v77": tiny_lm_head,
    "small_lmhead_v1000": small_lm_head,
    "llada8b_lmhead_b8": llada8b_lm_head_b8,
}


LOOP_WORKLOADS = {
    "small_loop_b4": small_loop_b4,
    "small_loop_d128": small_loop_d128,
    "llada8b_loop_b32": llada8b_loop_b32,
}


WORKLOADS = {
    "tiny_h256_l128": tiny_h256,
    "llada8b_b1_l768": llada8b_b1,
    "llada8b_ragged_b32": llada8b_ragged_b32,
    "llada8b_verify_b8": llada8b_verify_b8,
    "small_ragged_b5": small_ragged,
    "small_verify_b3": small_verify,
    "small_d64_rows150": small_d64_many_rows,
    "small_splitk_h1024": small_splitk,
    "small_long_l1500": small_long,
}
