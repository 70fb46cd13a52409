"""fp64 reference of one Flash-dLLM decoding step (test infrastructure only).

Conventions shared with the tests (none of them comes from the GPU library):

* bf16 tensors are numpy ``uint16`` arrays holding the raw bf16 bit patterns.
* ``x``      bf16 [R, hid]           hidden states of the active rows.
* ``w``      bf16 [3*H*D, hid]       the QKV weight as an ``nn.Linear`` weight:
  output feature n = row n; features [0,HD) are Q, [HD,2HD) K, [2HD,3HD) V, and
  head h owns features h*D .. h*D+D-1 inside each of the three groups.
* ``k_cache`` / ``v_cache`` bf16 [num_blocks, H, block_size, D] paged pools.
* ``block_table`` int32 [batch, max_blocks]: logical block -> physical block.
* ``cu_rows`` int32 [batch+1]: rows of sequence b are cu_rows[b]..cu_rows[b+1]-1.
* ``positions`` / ``slots`` int32 [R]: rotary position and logical cache slot of
  each active row.
* ``views`` int32 [batch, 3] = (window_start w0, window_len W, draft_slot_start
  d0), W == 0 meaning a plain (bidirectional) sequence; or None.

Page keys: [P4] = "Flash-dLLM: I/O-Aware KV Caching and Parallel Decoding for
Fast, Memory-Efficient Diffusion LLMs" (ai4snews.wisdomeyes.cn summary),
paragraphs 1-5.
"""

from __future__ import annotations

import math

import numpy as np

# ---------------------------------------------------------------------------
# bf16 codec (the storage format of Q, K, V and of the cache).
# ---------------------------------------------------------------------------

_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Widen bf16 bit patterns to float64 exactly (bf16 is the top half of fp32)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x) -> np.ndarray:
    """Round float64 values to bf16 with round-to-nearest-even, straight from fp64.

    bf16 keeps 8 significant bits and fp32's exponent range.  A finite x with
    x = m * 2**e, 0.5 <= |m| < 1, is rounded to a multiple of the quantum
    2**(e-8) (2**-133 below the normal range), ties to even; results above the
    largest finite bf16 become infinities.  NaN maps to the canonical quiet NaN.
    """
    x = np.asarray(x, dtype=np.float64)
    nan = np.isnan(x)
    xs = np.where(nan, 0.0, x)
    _, e = np.frexp(xs)
    q_exp = np.maximum(e - 8, -133)
    r = np.rint(np.ldexp(xs, -q_exp))  # np.rint rounds halves to even
    y = np.ldexp(r, q_exp)
    y = np.where(np.abs(y) > _BF16_MAX, np.copysign(np.inf, xs), y)
    bits = (y.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    bits = np.where(nan, np.uint16(0x7FC0), bits)
    return bits.astype(np.uint16)


# ---------------------------------------------------------------------------
# Flash-Cache: QKV projection, rotary embedding, cache write  [P4 para 1]
# ---------------------------------------------------------------------------


def qkv_projection(x_bits, w_bits) -> np.ndarray:
    """Y = X . W^T in fp64 for the active rows only [P4 para 1, para 2].

    ``w`` is stored as [3HD, hid] (output feature major), so the matrix of the
    projection Y = X.W_qkv (hid x 3HD) is ``w.T``.  No bias (the pages name none).
    """
    x = bf16_bits_to_f64(x_bits)
    w = bf16_bits_to_f64(w_bits)
    return x @ w.T


def rope_rotate(x, positions, base: float) -> np.ndarray:
    """Rotary embedding at each row's true position [P4 para 1; P4 para 3 shared positions].

    Reading (the pages give no convention): half-split pairs (i, i + D/2),
    frequency theta_i = base**(-2i/D), angle a = p * theta_i, and
    (x_i, x_{i+D/2}) -> (x_i cos a - x_{i+D/2} sin a, x_{i+D/2} cos a + x_i sin a).
    ``x`` is [R, H, D]; ``positions`` [R] are absolute, 0-based.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    i = np.arange(half, dtype=np.float64)
    theta = float(base) ** (-2.0 * i / d)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * theta[None, :]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x1 = x[..., :half]
    x2 = x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def row_sequence(cu_rows) -> np.ndarray:
    """Sequence index of every active row, from the row offsets."""
    cu = np.asarray(cu_rows, dtype=np.int64)
    seq = np.zeros(int(cu[-1]), dtype=np.int64)
    for b in range(len(cu) - 1):
        seq[cu[b]:cu[b + 1]] = b
    return seq


def physical_slots(cu_rows, slots, block_table, block_size: int) -> np.ndarray:
    """Physical cache slot of each row through the block table [P4 para 1].

    Logical slot s of sequence b lives in physical block block_table[b][s // bs]
    at offset s % bs; its physical slot number is that block * bs + offset.
    """
    seq = row_sequence(cu_rows)
    s = np.asarray(slots, dtype=np.int64)
    bt = np.asarray(block_table, dtype=np.int64)
    return bt[seq, s // block_size] * block_size + s % block_size


def flash_cache_step(x_bits, w_bits, num_heads, head_dim, positions, rope_base,
                     cu_rows, slots, block_table, block_size, k_cache_bits,
                     v_cache_bits):
    """One Flash-Cache call: QKV for the active rows, RoPE on Q and K, bf16
    storage, and K/V written into the paged cache [P4 para 1].

    The fused kernel changes how many bytes move, not what is computed, so the
    reference is the plain composition of its steps.  Rounding points: Q, K and V
    are rounded to bf16 once, after the rotation (the cache stores bf16).
    Returns (q_bits [R,H,D], new k_cache, new v_cache, slot_mapping int64 [R]).
    Every cache byte outside the written slots is left unchanged.
    """
    h, d = int(num_heads), int(head_dim)
    hd = h * d
    y = qkv_projection(x_bits, w_bits)
    r = y.shape[0]
    q = y[:, :hd].reshape(r, h, d)
    k = y[:, hd:2 * hd].reshape(r, h, d)
    v = y[:, 2 * hd:3 * hd].reshape(r, h, d)
    q = rope_rotate(q, positions, rope_base)
    k = rope_rotate(k, positions, rope_base)
    q_bits = f64_to_bf16_bits(q)
    k_bits = f64_to_bf16_bits(k)
    v_bits = f64_to_bf16_bits(v)
    ps = physical_slots(cu_rows, slots, block_table, block_size)
    if len(np.unique(ps)) != len(ps):
        raise ValueError("two active rows map to the same cache slot")
    kc = np.array(k_cache_bits, dtype=np.uint16, copy=True)
    vc = np.array(v_cache_bits, dtype=np.uint16, copy=True)
    if r:
        kc[ps // block_size, :, ps % block_size, :] = k_bits
        vc[ps // block_size, :, ps % block_size, :] = v_bits
    return q_bits, kc, vc, ps


# ---------------------------------------------------------------------------
# Scheduled attention with the two-view mask  [P4 para 1, para 3]
# ---------------------------------------------------------------------------


def visibility_mask(n_rows: int, kv_len: int, view=None) -> np.ndarray:
    """Which cached keys each row of one sequence may attend to.

    Plain sequence (no view, or window length 0): every row sees every slot in
    [0, kv_len) (bidirectional decoding of a masked diffusion model).

    Two-view sequence [P4 para 3] with view (w0, W, d0): the window's own cache
    slots w0..w0+W-1 hold the mask view; the draft view's keys sit in slots
    d0..d0+W-1 at the same rotary positions.  Rows 0..W-1 are the draft rows,
    rows W.. are mask rows.  Context = slots j < d0 outside the window.
      draft row i sees context and draft slots d0..d0+i (causal inside the view);
      a mask row sees context and the whole window, i.e. every j < d0.
    Neither view sees the other's keys.
    """
    j = np.arange(kv_len)
    if view is None or int(view[1]) == 0:
        return np.ones((n_rows, kv_len), dtype=bool)
    w0, wl, d0 = (int(v) for v in view)
    context = (j < d0) & ~((j >= w0) & (j < w0 + wl))
    vis = np.zeros((n_rows, kv_len), dtype=bool)
    for t in range(n_rows):
        if t < wl:
            vis[t] = context | ((j >= d0) & (j <= d0 + t))
        else:
            vis[t] = j < d0
    return vis


def gather_sequence_kv(cache_bits, block_table_row, kv_len: int, block_size: int):
    """Logical [H, kv_len, D] view of one sequence's keys or values (fp64)."""
    nblk = -(-int(kv_len) // block_size)
    blocks = np.asarray(block_table_row[:nblk], dtype=np.int64)
    c = bf16_bits_to_f64(np.asarray(cache_bits)[blocks])  # [nblk, H, bs, D]
    nb, h, bs, d = c.shape
    return c.transpose(1, 0, 2, 3).reshape(h, nb * bs, d)[:, :kv_len]


def attention(q_bits, k_cache_bits, v_cache_bits, block_table, block_size,
              cu_rows, kv_len, views=None, scale=None, want_probs=False):
    """Softmax attention of every active row over its sequence's cached keys.

    For sequence b, head h and row r: s_j = (q_r . k_j) * scale over the visible
    set (``visibility_mask``), P = softmax(s) with the maximum subtracted, and
    O_r = sum_j P_j v_j [P4 para 1 scheduled attention; P4 para 3 two views].
    scale defaults to 1/sqrt(D).  A row with no visible key gets O = 0.
    Returns O fp64 [R, H, D] and, if asked, the per-sequence P arrays
    [H, R_b, L_b] (zero where a key is not visible).
    """
    q = bf16_bits_to_f64(q_bits)
    r_total, h, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    cu = np.asarray(cu_rows, dtype=np.int64)
    lens = np.asarray(kv_len, dtype=np.int64)
    out = np.zeros((r_total, h, d))
    probs = []
    for b in range(len(lens)):
        r0, r1, length = int(cu[b]), int(cu[b + 1]), int(lens[b])
        view = None if views is None else np.asarray(views)[b]
        if r1 == r0:
            probs.append(np.zeros((h, 0, length)))
            continue
        kk = gather_sequence_kv(k_cache_bits, block_table[b], length, block_size)
        vv = gather_sequence_kv(v_cache_bits, block_table[b], length, block_size)
        vis = visibility_mask(r1 - r0, length, view)[None]  # [1, Rb, L]
        qb = q[r0:r1].transpose(1, 0, 2)  # [H, Rb, D]
        s = (qb @ kk.transpose(0, 2, 1)) * scale  # [H, Rb, L]
        s = np.where(vis, s, -np.inf)
        m = np.max(s, axis=-1, keepdims=True) if length else np.zeros(s.shape[:-1] + (1,))
        m = np.where(np.isfinite(m), m, 0.0)
        e = np.where(vis, np.exp(s - m), 0.0)
        z = e.sum(axis=-1, keepdims=True)
        p = np.divide(e, z, out=np.zeros_like(e), where=z > 0)
        out[r0:r1] = (p @ vv).transpose(1, 0, 2)
        probs.append(p)
    return (out, probs) if want_probs else out


def attention_mass(probs, mass_stride=None) -> np.ndarray:
    """Attention mass per cached key: m_b[j] = sum over heads and query rows of
    P[b, h, r, j] [P4 para 2 "most-attended tokens"].

    Summed, not averaged (same ranking, no rounding-made ties).  Returns
    fp64 [batch, mass_stride], zero past each sequence's length.
    """
    lens = [p.shape[-1] for p in probs]
    stride = max(lens + [0]) if mass_stride is None else int(mass_stride)
    m = np.zeros((len(probs), stride))
    for b, p in enumerate(probs):
        m[b, :p.shape[-1]] = p.sum(axis=(0, 1))
    return m


def top_b(mass_row, kv_len: int, b: int) -> np.ndarray:
    """The B most-attended keys of one sequence [P4 para 2 tracking budget].

    Keys j < kv_len are ranked by mass, larger first, equal masses broken
    towards the lower index; the first B of that order are returned as a set in
    ascending index order, padded with -1 when kv_len < B.
    """
    n = int(kv_len)
    m = np.asarray(mass_row, dtype=np.float64)[:n]
    idx = np.arange(n)
    order = np.lexsort((idx, -m))  # primary: mass descending; secondary: index ascending
    chosen = np.sort(order[:b])
    out = np.full(b, -1, dtype=np.int32)
    out[:len(chosen)] = chosen
    return out


# ---------------------------------------------------------------------------
# Flash-Verify acceptance  [P4 para 3]
# ---------------------------------------------------------------------------


def accept_length(draft_tok, mask_tok, conf, threshold) -> int:
    """Accepted prefix length of one sequence [P4 para 3].

    Positions are examined in causal order; position k is accepted when the
    draft token equals the mask-view argmax and the mask-view confidence
    exceeds the threshold (strictly).  The scan stops at the first position
    that fails.  Confidences and the threshold are compared as given (fp32
    values widened exactly).
    """
    k = 0
    n = len(draft_tok)
    while k < n and int(draft_tok[k]) == int(mask_tok[k]) and float(conf[k]) > float(threshold):
        k += 1
    return k


# ---------------------------------------------------------------------------
# The whole per-layer step
# ---------------------------------------------------------------------------


def decode_step(x_bits, w_bits, num_heads, head_dim, positions, rope_base, cu_rows,
                slots, block_table, block_size, k_cache_bits, v_cache_bits, kv_len,
                views=None, topb=0, mass_stride=None):
    """Flash-Cache, then scheduled attention on the updated cache, then (when
    topb > 0) the attention mass and the next tracking set [P4 paras 1-3].

    Order within the step: attention sees the freshly written K/V at the active
    slots and the old cache everywhere else.
    """
    q_bits, kc, vc, ps = flash_cache_step(
        x_bits, w_bits, num_heads, head_dim, positions, rope_base, cu_rows, slots,
        block_table, block_size, k_cache_bits, v_cache_bits)
    o, probs = attention(q_bits, kc, vc, block_table, block_size, cu_rows, kv_len,
                         views=views, want_probs=True)
    res = dict(q=q_bits, k_cache=kc, v_cache=vc, slot_mapping=ps, out=o)
    if topb:
        mass = attention_mass(probs, mass_stride)
        res["mass"] = mass
        res["topb"] = np.stack([top_b(mass[b], int(kv_len[b]), topb)
                                for b in range(len(kv_len))]) if len(kv_len) else \
            np.zeros((0, topb), np.int32)
    return res
