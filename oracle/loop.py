"""fp64 reference of a multi-step, weight-free decoding loop around the per-layer
step (test infrastructure only).

The pages describe the loop only in outline [P4 para 1: caching and update
stages alternate within a batch, so the sequences' lengths diverge and a
block table schedules them; P4 para 2: each step's query rows are a sliding
unmasking window plus a fixed budget of the most-attended tokens, re-selected
as decoding goes on; P4 para 3: a position is committed when the two views
agree and the mask-view confidence exceeds the threshold, in causal order].
The reading taken here, step by step (the design notes list it too):

* State per sequence b: the frontier f_b, the first position not yet
  committed (0 <= f_b <= L_b); the cache length L_b is fixed (a diffusion LM
  decodes a canvas of fixed length).
* Step t > 0 first commits the previous step's accepted prefix:
  f_b += max(1, min(accept_b, W)), capped at L_b.  At least one token per step
  is the caller's progress policy (the pages state none); at most the
  window's W tokens can be accepted.  Step 0 commits nothing.
* A sequence with f_b = L_b is finished and has no rows.
* Stage: the caching (refresh) stage when the refresh period K > 0 and
  (t + b) mod K = 0, else the update stage; the offset by b staggers the
  stages so both occur in one batch step.  Refresh: the window starts at the
  block boundary at or below f_b.  Update: the window starts at f_b.  Either
  way it is [w0, min(w0 + W, L_b)).
* Tracked rows: the previous step's top-B set (the caller's initial set at
  t = 0), keeping an entry when it lies in [0, L_b), outside the window and
  above every entry kept before it (a top-B set is ascending; this also
  drops repeats).  Window positions are recomputed anyway, so an entry inside
  the window is not a second row.
* Rows of a sequence: the window positions ascending, then the kept tracked
  positions; each row's cache slot is its position.
* Hidden state of a row at position p: a committed-token row when p < f_b,
  else a masked-token row (two synthetic tables, as no model supplies them).
* Then the per-layer step (reference.decode_step), the top-B selection of
  its mass and the accept scan of this step's (synthetic) draft and
  mask-view tokens and confidences.
"""

from __future__ import annotations

import numpy as np

from . import reference as R

STAGE_UPDATE, STAGE_REFRESH, STAGE_DONE = 0, 1, 2


def plan_step(step, kv_len, window_len, block_size, refresh_period, tracked, accept_len,
              frontier):
    """Rows of one loop step (the planning rules in the module docstring).

    Returns (frontier [batch] after this step's commit, stage [batch],
    cu_rows [batch+1], positions [R], slots [R]), all int32.
    """
    batch = len(kv_len)
    w = int(window_len)
    new_f = np.zeros(batch, np.int32)
    stage = np.zeros(batch, np.int32)
    cu = [0]
    rows = []
    for b in range(batch):
        length = max(0, int(kv_len[b]))
        f = min(max(int(frontier[b]), 0), length)
        if step > 0 and f < length:
            acc = min(max(int(accept_len[b]), 0), w)
            f = min(length, f + max(1, acc))
        new_f[b] = f
        if f >= length:
            stage[b] = STAGE_DONE
            cu.append(len(rows))
            continue
        refresh = refresh_period > 0 and (step + b) % refresh_period == 0
        stage[b] = STAGE_REFRESH if refresh else STAGE_UPDATE
        w0 = (f // block_size) * block_size if refresh else f
        w1 = min(w0 + w, length)
        rows.extend(range(w0, w1))
        last = -1
        for t in tracked[b]:
            t = int(t)
            if t < 0 or t >= length or w0 <= t < w1 or t <= last:
                continue
            rows.append(t)
            last = t
        cu.append(len(rows))
    pos = np.array(rows, np.int32)
    return new_f, stage, np.array(cu, np.int32), pos, pos.copy()


def hidden_rows(hidden_committed, hidden_masked, cu_rows, positions, frontier):
    """Hidden-state rows of the step: the committed-token row of (b, p) when
    p < f_b, else the masked-token row (tables bf16 [batch, max_len, hid])."""
    cu = np.asarray(cu_rows)
    out = np.zeros((int(cu[-1]), hidden_committed.shape[-1]), np.uint16)
    for b in range(len(cu) - 1):
        for r in range(int(cu[b]), int(cu[b + 1])):
            p = int(positions[r])
            src = hidden_committed if p < int(frontier[b]) else hidden_masked
            out[r] = src[b, p]
    return out


def decode_loop(steps, w_bits, num_heads, head_dim, rope_base, block_table, block_size,
                k_cache_bits, v_cache_bits, kv_len, hidden_committed, hidden_masked, frontier0,
                tracked0, window_len, topb, refresh_period, draft, mask, conf, threshold,
                mass_stride=None):
    """Run ``steps`` loop steps in fp64 and return one record per step.

    ``draft`` / ``mask`` / ``conf`` are [steps, batch, W] scan inputs.  A
    record holds the plan (frontier, stage, cu_rows, positions), the step's
    outputs (q, out, mass, topb, slot_mapping) and the accept lengths; the
    cache evolves from step to step.
    """
    kc = np.array(k_cache_bits, copy=True)
    vc = np.array(v_cache_bits, copy=True)
    batch = len(kv_len)
    frontier = np.asarray(frontier0, np.int32).copy()
    tracked = np.asarray(tracked0, np.int32).copy()
    accept = np.zeros(batch, np.int32)
    stride = int(max(kv_len)) if mass_stride is None else int(mass_stride)
    records = []
    for t in range(steps):
        frontier, stage, cu, pos, slots = plan_step(t, kv_len, window_len, block_size,
                                                    refresh_period, tracked, accept, frontier)
        x = hidden_rows(hidden_committed, hidden_masked, cu, pos, frontier)
        res = R.decode_step(x, w_bits, num_heads, head_dim, pos, rope_base, cu, slots,
                            block_table, block_size, kc, vc, kv_len, topb=topb,
                            mass_stride=stride)
        kc, vc = res["k_cache"], res["v_cache"]
        tracked = np.asarray(res["topb"], np.int32)
        accept = np.array([R.accept_length(draft[t][b], mask[t][b], conf[t][b], threshold)
                           for b in range(batch)], np.int32)
        records.append(dict(frontier=frontier.copy(), stage=stage, cu_rows=cu, positions=pos,
                            x=x, q=res["q"], out=res["out"], mass=res["mass"],
                            topb=tracked.copy(), slot_mapping=res["slot_mapping"],
                            accept=accept.copy()))
    return records, kc, vc
