"""Plant plausible mistakes in the CPU oracle and check that at least one pin
catches each.  The mistakes live only in this process (monkeypatched), on the CPU."""

import numpy as np
import pytest

import oracle
import oracle.lm_head as LH
import oracle.loop as LP
import oracle.reference as R
from tests import pins

_orig = {name: getattr(R, name) for name in dir(R) if callable(getattr(R, name))}
_orig_loop = {name: getattr(LP, name) for name in ("plan_step", "hidden_rows", "decode_loop")}
_orig_lm = {name: getattr(LH, name) for name in ("lm_head_confidence", "verify_chain")}


def _truncating_bf16(x):
    x = np.asarray(x, dtype=np.float64)
    return (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _gemm_dropped_term(x_bits, w_bits):
    x = R.bf16_bits_to_f64(x_bits)
    w = R.bf16_bits_to_f64(w_bits)
    return x[:, :-1] @ w[:, :-1].T


def _rope_variant(kind):
    def rope(x, positions, base):
        x = np.asarray(x, dtype=np.float64)
        d = x.shape[-1]
        half = d // 2
        i = np.arange(half, dtype=np.float64)
        theta = float(base) ** ((-1.0 if kind == "theta" else -2.0) * i / d)
        ang = np.asarray(positions, dtype=np.float64)[:, None] * theta[None, :]
        c = np.cos(ang)[:, None, :]
        s = np.sin(ang)[:, None, :]
        if kind == "interleaved":
            x1, x2 = x[..., 0::2], x[..., 1::2]
            out = np.empty_like(x)
            out[..., 0::2] = x1 * c - x2 * s
            out[..., 1::2] = x2 * c + x1 * s
            return out
        x1, x2 = x[..., :half], x[..., half:]
        sign = -1.0 if kind == "sign" else 1.0
        return np.concatenate([x1 * c - sign * x2 * s, x2 * c + sign * x1 * s], axis=-1)
    return rope


def _slots_wrong_offset(cu_rows, slots, block_table, block_size):
    seq = R.row_sequence(cu_rows)
    s = np.asarray(slots, dtype=np.int64)
    bt = np.asarray(block_table, dtype=np.int64)
    return bt[seq, s // block_size] * block_size + s // block_size


def _attention_no_scale(*a, **k):
    k["scale"] = 1.0 if k.get("scale") is None else k["scale"]
    return _orig["attention"](*a, **k)


def _vis_variant(kind):
    def vis(n_rows, kv_len, view=None):
        m = _orig["visibility_mask"](n_rows, kv_len, view)
        if view is None or int(view[1]) == 0:
            return m
        w0, wl, d0 = (int(v) for v in view)
        j = np.arange(kv_len)
        for t in range(min(wl, n_rows)):
            if kind == "leak":
                m[t] |= (j >= w0) & (j < w0 + wl)
            elif kind == "noncausal":
                m[t] |= (j >= d0) & (j < d0 + wl)
        return m
    return vis


def _mass_mean(probs, mass_stride=None):
    m = _orig["attention_mass"](probs, mass_stride)
    for b, p in enumerate(probs):
        if p.shape[1]:
            m[b] /= p.shape[0] * p.shape[1]
    return m


def _topb_variant(kind):
    def topb(mass_row, kv_len, b):
        n = int(kv_len)
        m = np.asarray(mass_row, dtype=np.float64)[:n]
        idx = np.arange(n)
        if kind == "hi_ties":
            order = np.lexsort((-idx, -m))
            chosen = np.sort(order[:b])
        else:  # kept in mass order
            order = np.lexsort((idx, -m))
            chosen = order[:b]
        out = np.full(b, -1, dtype=np.int32)
        out[:len(chosen)] = chosen
        return out
    return topb


def _accept_variant(kind):
    def acc(draft, mask, conf, thr):
        if kind == "ge":
            k = 0
            while k < len(draft) and int(draft[k]) == int(mask[k]) and float(conf[k]) >= float(thr):
                k += 1
            return k
        return sum(1 for k in range(len(draft))
                   if int(draft[k]) == int(mask[k]) and float(conf[k]) > float(thr))
    return acc


def _fcs_rotating_v(x_bits, w_bits, num_heads, head_dim, positions, rope_base, cu_rows, slots,
                    block_table, block_size, k_cache_bits, v_cache_bits):
    h, d = int(num_heads), int(head_dim)
    hd = h * d
    y = R.qkv_projection(x_bits, w_bits)
    r = y.shape[0]
    q = R.rope_rotate(y[:, :hd].reshape(r, h, d), positions, rope_base)
    k = R.rope_rotate(y[:, hd:2 * hd].reshape(r, h, d), positions, rope_base)
    v = R.rope_rotate(y[:, 2 * hd:].reshape(r, h, d), positions, rope_base)
    ps = R.physical_slots(cu_rows, slots, block_table, block_size)
    kc = np.array(k_cache_bits, copy=True)
    vc = np.array(v_cache_bits, copy=True)
    kc[ps // block_size, :, ps % block_size, :] = R.f64_to_bf16_bits(k)
    vc[ps // block_size, :, ps % block_size, :] = R.f64_to_bf16_bits(v)
    return R.f64_to_bf16_bits(q), kc, vc, ps


def _plan_variant(kind):
    def plan(step, kv_len, window_len, block_size, refresh_period, tracked, accept_len, frontier):
        batch = len(kv_len)
        w = int(window_len)
        new_f = np.zeros(batch, np.int32)
        stage = np.zeros(batch, np.int32)
        cu, rows = [0], []
        for b in range(batch):
            length = max(0, int(kv_len[b]))
            f = min(max(int(frontier[b]), 0), length)
            if step > 0 and f < length:
                acc = max(int(accept_len[b]), 0)
                if kind != "no_cap":
                    acc = min(acc, w)
                f = min(length, f + (acc if kind == "no_min_commit" else max(1, acc)))
            new_f[b] = f
            if f >= length:
                stage[b] = 2
                cu.append(len(rows))
                continue
            refresh = refresh_period > 0 and (step + b) % refresh_period == 0
            stage[b] = 1 if refresh else 0
            w0 = (f // block_size) * block_size if refresh and kind != "unaligned" else f
            w1 = min(w0 + w, length)
            rows.extend(range(w0, w1))
            last = -1
            for t in tracked[b]:
                t = int(t)
                inside = w0 <= t < w1 and kind != "window_dupes"
                if t < 0 or t >= length or inside or t <= last:
                    continue
                rows.append(t)
                last = t
            cu.append(len(rows))
        pos = np.array(rows, np.int32)
        return new_f, stage, np.array(cu, np.int32), pos, pos.copy()
    return plan


def _hidden_le(hidden_committed, hidden_masked, cu_rows, positions, frontier):
    cu = np.asarray(cu_rows)
    out = np.zeros((int(cu[-1]), hidden_committed.shape[-1]), np.uint16)
    for b in range(len(cu) - 1):
        for r in range(int(cu[b]), int(cu[b + 1])):
            p = int(positions[r])
            out[r] = (hidden_committed if p <= int(frontier[b]) else hidden_masked)[b, p]
    return out


def _loop_variant(kind):
    def loop(steps, w_bits, num_heads, head_dim, rope_base, block_table, block_size,
             k_cache_bits, v_cache_bits, kv_len, hidden_committed, hidden_masked, frontier0,
             tracked0, window_len, topb, refresh_period, draft, mask, conf, threshold,
             mass_stride=None):
        kc0, vc0 = k_cache_bits, v_cache_bits
        kc, vc = kc0, vc0
        frontier = np.asarray(frontier0, np.int32).copy()
        tracked = np.asarray(tracked0, np.int32).copy()
        accept = np.zeros(len(kv_len), np.int32)
        recs = []
        for t in range(steps):
            frontier, stage, cu, pos, slots = LP.plan_step(t, kv_len, window_len, block_size,
                                                           refresh_period, tracked, accept,
                                                           frontier)
            x = LP.hidden_rows(hidden_committed, hidden_masked, cu, pos, frontier)
            res = R.decode_step(x, w_bits, num_heads, head_dim, pos, rope_base, cu, slots,
                                block_table, block_size, kc, vc, kv_len, topb=topb,
                                mass_stride=int(max(kv_len)))
            if kind != "no_carry":
                kc, vc = res["k_cache"], res["v_cache"]
            if kind != "stale_tracked":
                tracked = np.asarray(res["topb"], np.int32)
            accept = np.array([R.accept_length(draft[t][b], mask[t][b], conf[t][b], threshold)
                               for b in range(len(kv_len))], np.int32)
            recs.append(dict(frontier=frontier.copy(), stage=stage, cu_rows=cu, positions=pos,
                             x=x, q=res["q"], out=res["out"], mass=res["mass"],
                             topb=np.asarray(res["topb"], np.int32), accept=accept.copy()))
        return recs, res["k_cache"], res["v_cache"]
    return loop


def _lm_variant(kind):
    def lm(h_bits, w_bits):
        z = R.bf16_bits_to_f64(h_bits) @ R.bf16_bits_to_f64(w_bits).T
        if kind == "hi_ties":
            tok = (z.shape[1] - 1 - np.argmax(z[:, ::-1], axis=1)).astype(np.int32)
        else:
            tok = np.argmax(z, axis=1).astype(np.int32)
        zmax = z[np.arange(z.shape[0]), tok]
        if kind == "no_shift":
            with np.errstate(over="ignore", invalid="ignore"):
                conf = np.exp(zmax) / np.exp(z).sum(axis=1)
        elif kind == "max_logit":
            conf = 1.0 / (1.0 + np.exp(-zmax))
        else:
            conf = 1.0 / np.exp(z - zmax[:, None]).sum(axis=1)
        return tok, conf, z
    return lm


def _chain_draft_conf(h_draft_bits, h_mask_bits, w_bits, batch, window, threshold):
    dtok, dconf, _ = LH.lm_head_confidence(h_draft_bits, w_bits)
    mtok, _, _ = LH.lm_head_confidence(h_mask_bits, w_bits)
    dtok, mtok, conf = (a.reshape(batch, window) for a in (dtok, mtok, dconf))
    acc = np.array([R.accept_length(dtok[b], mtok[b], conf[b], threshold) for b in range(batch)],
                   np.int32)
    return dtok, mtok, conf, acc


MUTANTS = {
    "bf16_truncates": ("f64_to_bf16_bits", _truncating_bf16),
    "gemm_drops_term": ("qkv_projection", _gemm_dropped_term),
    "rope_sign": ("rope_rotate", _rope_variant("sign")),
    "rope_interleaved": ("rope_rotate", _rope_variant("interleaved")),
    "rope_theta": ("rope_rotate", _rope_variant("theta")),
    "slot_offset": ("physical_slots", _slots_wrong_offset),
    "attention_unscaled": ("attention", _attention_no_scale),
    "view_leak": ("visibility_mask", _vis_variant("leak")),
    "view_noncausal": ("visibility_mask", _vis_variant("noncausal")),
    "mass_mean": ("attention_mass", _mass_mean),
    "topb_high_ties": ("top_b", _topb_variant("hi_ties")),
    "topb_mass_order": ("top_b", _topb_variant("order")),
    "accept_ge": ("accept_length", _accept_variant("ge")),
    "accept_no_stop": ("accept_length", _accept_variant("nostop")),
    "v_rotated": ("flash_cache_step", _fcs_rotating_v),
    "plan_no_min_commit": ("plan_step", _plan_variant("no_min_commit")),
    "plan_no_cap": ("plan_step", _plan_variant("no_cap")),
    "plan_window_dupes": ("plan_step", _plan_variant("window_dupes")),
    "plan_refresh_unaligned": ("plan_step", _plan_variant("unaligned")),
    "hidden_rows_le": ("hidden_rows", _hidden_le),
    "loop_no_carry": ("decode_loop", _loop_variant("no_carry")),
    "loop_stale_tracked": ("decode_loop", _loop_variant("stale_tracked")),
    "lm_head_high_ties": ("lm_head_confidence", _lm_variant("hi_ties")),
    "lm_head_unshifted_softmax": ("lm_head_confidence", _lm_variant("no_shift")),
    "lm_head_sigmoid_conf": ("lm_head_confidence", _lm_variant("max_logit")),
    "chain_draft_confidence": ("verify_chain", _chain_draft_conf),
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_some_pin_catches(mutant, monkeypatch):
    name, fn = MUTANTS[mutant]
    mod = LP if name in _orig_loop else LH if name in _orig_lm else R
    monkeypatch.setattr(mod, name, fn)
    if hasattr(oracle, name):
        monkeypatch.setattr(oracle, name, fn)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches mutant {mutant}"
