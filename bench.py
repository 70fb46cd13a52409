#!/usr/bin/env python3
"""Throughput of the per-layer Flash-dLLM decode step on one MI355X.

One step = flash_cache_step (QKV projection + rotary embedding + paged K/V write)
-> scheduled_attention (with the attention mass when the tracking set is
re-selected) -> track_topb (next tracking set) [-> verify_accept on the two-view
workload].  Default workload: the 32-layer stack of the LLaDA-8B-class layer
(hidden 4096, 32 heads x 128, rotary base 5e5) at batch 16 with a 4096-slot
cache per sequence, 64 active rows per sequence (window of 32 + 32 tracked),
the tracking set re-selected in every layer: the largest workload, and the one
that streams the whole ~34 GB cache plus 32 weights from HBM every step.
``--workload`` selects the single-layer shapes (batch 1, batch 32 ragged,
two-view batch 8); they are also parity cases of the tests.

Inputs are resident in HBM before timing.  A single-layer step's working set
(~116 MB at batch 1) would fit in the 256 MB last-level cache, so those
workloads rotate over independent copies of weights, hidden states and cache
until the rotation exceeds ~560 MB: every step streams its weight and cache
from HBM.  The stack needs no copies (38 GB per step).

Prints ONE JSON line (N = 1): metric, value (active query tokens/s per layer),
ms_per_step (all layers of a step), the roofline of the call that takes longer
(duration from HIP events recorded around each launch on its stream inside the
timed loop) and of the other call, the whole step's HBM fraction against its
algorithmic bytes, and the CPU oracle's throughput on a bounded sample of the
same workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "active query tokens/s per layer (fused QKV+RoPE+KV-write+attn); % HBM roofline"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA
PROFILE_DIR = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "kv_cache_attention_flash_amd", "csrc")
SOURCES = {"flash_cache_step": [os.path.join(CSRC, "flash_cache.hip")],
           "flash_cache_step_unfused": [os.path.join(CSRC, "flash_cache.hip")],
           "scheduled_attention": [os.path.join(CSRC, "attention.hip")]}
ROTATION_BYTES = 560e6

WORKLOADS = {
    "llada8b_b1_l768": "hidden 4096, 32x128 MHA, batch 1, cache 768 (256 prompt + 512 generated), "
                       "64 active rows (window 32 + 32 tracked), rope base 5e5, top-32 re-selection",
    "llada8b_ragged_b32": "hidden 4096, 32x128 MHA, batch 32, cache U{512..1024} (block size 32), "
                          "half refresh / half update stage, 64 active rows each (2048 total), top-32",
    "llada8b_verify_b8": "hidden 4096, 32x128 MHA, batch 8, context 1024 + one draft block, "
                         "32 draft + 32 mask rows per sequence (two-view mask), accept scan tau 0.9",
    "llada8b_stack32_b16_l4096": "32 independent layers of hidden 4096, 32x128 MHA, batch 16, "
                                 "cache 4096, 64 active rows each (1024 per layer), top-32 per layer",
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def flash_cache_bytes(wl) -> int:
    """Algorithmic HBM bytes of one flash_cache_step launch: the weight once,
    the active rows' hidden states and their written K and V (bf16).  Q's write
    is half of the Q round trip, which is not algorithmic (q_round_trip_bytes)."""
    hd = wl.num_heads * wl.head_dim
    return 2 * 3 * hd * wl.hid + wl.rows * (2 * wl.hid + 4 * hd)


def flash_cache_flops(wl) -> int:
    return 2 * wl.rows * wl.hid * 3 * wl.num_heads * wl.head_dim


def attention_bytes(wl) -> int:
    """Algorithmic bytes of scheduled_attention: every cached K and V slot of a
    sequence once per head, O out (fp32), the mass out (fp32) when asked.  Q's
    read is the other half of the Q round trip (not algorithmic)."""
    hd = wl.num_heads * wl.head_dim
    kv = int(sum(int(v) for v in wl.kv_len)) * hd * 2 * 2
    mass = 4 * int(sum(int(v) for v in wl.kv_len)) if wl.topb else 0
    return kv + wl.rows * hd * 4 + mass


def q_round_trip_bytes(wl) -> int:
    """Q written by flash_cache_step and read back by scheduled_attention (bf16):
    moved because the two are separate calls, not part of the algorithmic bytes."""
    return 4 * wl.rows * wl.num_heads * wl.head_dim


def step_bytes(wl) -> int:
    """Algorithmic bytes of one layer's step: W + R (2 hid + 4 HD + 4 HD) +
    4 HD sum(L) + 4 sum(L) [mass] -- the projection's and the attention's."""
    return flash_cache_bytes(wl) + attention_bytes(wl)


def visible_pairs(wl) -> int:
    """Sum over active rows of the number of slots the row attends to."""
    tot = 0
    for b in range(wl.batch):
        n = int(wl.cu_rows[b + 1] - wl.cu_rows[b])
        L = int(wl.kv_len[b])
        if wl.views is None or int(wl.views[b][1]) == 0:
            tot += n * L
            continue
        w0, W, d0 = (int(v) for v in wl.views[b])
        lim = min(d0, L)
        ctx = lim - max(0, min(w0 + W, lim) - w0)  # context outside the window
        for t in range(n):
            tot += ctx + min(t + 1, max(0, L - d0)) if t < W else lim
    return tot


def attention_flops(wl) -> int:
    return 4 * wl.num_heads * wl.head_dim * visible_pairs(wl)


def source_hash(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_file(call, workload):
    return os.path.join(PROFILE_DIR, f"{call}_{workload}_traffic.json")


def load_traffic(call, workload):
    """HBM bytes per launch from the committed rocprofv3 counter runs, only if
    they were taken on the current kernel source."""
    try:
        with open(traffic_file(call, workload)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != source_hash(SOURCES[call]):
        return None
    return t.get("bytes_per_launch")


class HipTimer:
    """HIP events created with hipEventDisableSystemFence: recording them does
    not write back and invalidate the caches, which would otherwise add a few
    microseconds to every bracketed launch (the HIP runtime documents the flag
    for timing).  Uses the HIP runtime torch has loaded (soname libamdhip64.so.7)."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = self.ct.c_void_p()
        rc = self.hip.hipEventCreateWithFlags(self.ct.byref(e), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed: {rc}")
        return e

    def record(self, e, stream_handle):
        rc = self.hip.hipEventRecord(e, self.ct.c_void_p(stream_handle))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed: {rc}")

    def ms(self, a, b) -> float:
        out = self.ct.c_float()
        rc = self.hip.hipEventElapsedTime(self.ct.byref(out), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return out.value


def _threads():
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        return 1


def sequence_subset(wl, seqs, x, k_cache, v_cache):
    """Inputs of the sequences ``seqs`` alone (their rows, block-table rows,
    lengths and views); the cache pools stay whole.  Selection only."""
    import numpy as np
    rows = np.concatenate([np.arange(wl.cu_rows[b], wl.cu_rows[b + 1]) for b in seqs])
    cu = np.cumsum([0] + [int(wl.cu_rows[b + 1] - wl.cu_rows[b]) for b in seqs]).astype(np.int32)
    return dict(rows=rows, x=x[rows], positions=wl.positions[rows], slots=wl.slots[rows], cu=cu,
                bt=wl.block_table[seqs], kv_len=wl.kv_len[seqs], k=k_cache, v=v_cache,
                views=None if wl.views is None else wl.views[seqs], seqs=list(seqs))


def cpu_baseline(wl, sub, w, budget_s, sample_desc):
    """The oracle as it stands, on a bounded sample of the workload, on this
    host's cores; tokens/s per layer = sampled active rows / oracle time."""
    import numpy as np
    import oracle as O
    times, res = [], None
    t_end = time.perf_counter() + budget_s
    while not times or time.perf_counter() < t_end:
        t0 = time.perf_counter()
        res = O.decode_step(sub["x"], w, wl.num_heads, wl.head_dim, sub["positions"], wl.rope_base,
                            sub["cu"], sub["slots"], sub["bt"], wl.block_size, sub["k"], sub["v"],
                            sub["kv_len"], views=sub["views"], topb=wl.topb,
                            mass_stride=wl.max_kv_len)
        times.append(time.perf_counter() - t0)
    mean = float(np.mean(times))
    n = len(sub["rows"])
    return ({"value": n / mean, "unit": "tokens/s/layer", "cores": int(_threads()),
             "kind": "oracle",
             "sample": f"{len(times)} oracle step(s) over {sample_desc} ({n} active rows, "
                       f"fp64 numpy, {mean:.2f} s each)"}, res)


def parity_against(res, sub, st, wl):
    """GPU outputs of the sampled sequences against the oracle: slot mapping,
    tracking set (the oracle's rule on the GPU's mass) and accepted lengths
    exact, output within the float tolerance."""
    import numpy as np
    import oracle as O
    rows = sub["rows"]
    ok = bool(np.array_equal(st.slot_mapping.cpu().numpy()[rows], res["slot_mapping"]))
    o = st.out.cpu().numpy().astype(np.float64)[rows]
    err = float(np.max(np.abs(o - res["out"])) / np.max(np.abs(res["out"])))
    ok &= err <= 2e-2
    if wl.topb:
        m = st.mass.cpu().numpy().astype(np.float64)
        idx = st.idx.cpu().numpy()
        for b in sub["seqs"]:
            ok &= bool(np.array_equal(idx[b], O.top_b(m[b], int(wl.kv_len[b]), wl.topb)))
    if wl.verify is not None:
        v = wl.verify
        want = [O.accept_length(v["draft"][b], v["mask"][b], v["conf"][b], v["threshold"])
                for b in range(wl.batch)]
        ok &= [int(a) for a in st.accept_len.cpu().numpy()] == want
    return {"ok": bool(ok), "out_max_rel_err": err, "sequences": len(sub["seqs"])}


def roofline_entry(call, wl, ms, workload):
    """Roofline of one library call from its measured average duration; the
    bound is HBM if the call's algorithmic flops per byte are below the ridge
    point (2.5 PFLOP/s / 8 TB/s = 312.5), else MFMA."""
    if call.startswith("flash_cache_step"):
        nbytes, flops = flash_cache_bytes(wl), flash_cache_flops(wl)
    else:
        nbytes, flops = attention_bytes(wl), attention_flops(wl)
    ridge = MFMA_BF16_PEAK_TFS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if flops / nbytes < ridge:
        achieved = nbytes / (ms / 1e3) / 1e9
        e = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        achieved = flops / (ms / 1e3) / 1e12
        e = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFS,
             "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFS, 4)}
    e["traffic"] = load_traffic(call, workload)
    e["kernel"] = call
    e["algorithmic_bytes"] = nbytes
    e["algorithmic_flops"] = flops
    e["avg_launch_us"] = round(ms * 1e3, 2)
    return e


LOOP_METRIC = "decode-loop steps/s (one layer, batch 32, every step planned on the device)"
LOOP_WORKLOAD = ("llada8b_loop_b32: hidden 4096, 32x128 MHA, batch 32, cache U{512..1024}; per "
                 "step decode_plan (window 32 + up to 32 tracked rows, refresh every 4th step "
                 "staggered across the batch, commit max(1, accepted)) -> gather_hidden -> "
                 "flash_cache_step -> scheduled_attention(+mass) -> track_topb -> verify_accept "
                 "(synthetic scan, ~5.7 accepted per step)")


def run_loop(args):
    """The multi-step loop: steps/s of the whole batch with every step planned
    on the device.  An untimed pass from the same initial state records each
    step's active rows and frontiers (copies that would otherwise sit inside
    the timed region); the timed pass then runs the same steps with nothing
    added, and its final frontiers must equal the untimed pass's."""
    import numpy as np
    import torch

    import kv_cache_attention_flash_amd as fd
    import synth

    steps_k = args.steps if args.steps is not None else 32
    warmup = args.warmup if args.warmup is not None else 4
    fd.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = synth.llada8b_loop_b32(steps=warmup + steps_k)
    w, k, v, hc, hm = synth.loop_tensors(wl, dev)
    k0, v0 = k.clone(), v.clone()

    def i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)

    sc = wl.scan
    scan = (i32(sc["draft"]), i32(sc["mask"]), torch.from_numpy(sc["conf"]).to(dev),
            float(sc["threshold"]))
    kv = i32(wl.kv_len)
    cache = fd.PagedKVCache(k, v, i32(wl.block_table))
    loop = fd.DecodeLoop(cache, w, hc, hm, kv, i32(wl.frontier0), i32(wl.tracked0),
                         wl.window_len, wl.rope_base, wl.refresh_period, wl.max_len, scan=scan)
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    log(f"loop {wl.name}: batch {wl.batch}, row capacity {loop.cap}, "
        f"{warmup} + {steps_k} steps, resident {torch.cuda.memory_allocated(dev) / 1e9:.2f} GB")

    def reset():
        k.copy_(k0)
        v.copy_(v0)
        loop.frontier.copy_(i32(wl.frontier0))
        loop.tracked.copy_(i32(wl.tracked0))
        loop.accept.zero_()
        torch.cuda.synchronize()

    rows, fronts = [], []
    for t in range(warmup + steps_k):
        loop.step(t, sh)
        rows.append(int(loop.cu_rows[-1].item()))
        fronts.append(loop.frontier.cpu().numpy().astype(np.int64))
    reset()
    for t in range(warmup):
        loop.step(t, sh)
    torch.cuda.synchronize()
    ht = HipTimer()
    # Pass 1: the steps as they run (nothing recorded between the calls).
    start, end = ht.event(), ht.event()
    ht.record(start, sh)
    for i in range(steps_k):
        loop.step(warmup + i, sh)
    ht.record(end, sh)
    torch.cuda.synchronize()
    total_ms = ht.ms(start, end)
    same = bool(np.array_equal(loop.frontier.cpu().numpy(), fronts[-1]))
    # Pass 2, from the same state: an event around every call for the
    # per-call durations (each record costs about a microsecond of GPU time).
    reset()
    for t in range(warmup):
        loop.step(t, sh)
    torch.cuda.synchronize()
    names = ["decode_plan", "gather_hidden", "flash_cache_step", "scheduled_attention",
             "track_topb", "verify_accept"]
    ev = [[ht.event() for _ in range(len(names) + 1)] for _ in range(steps_k)]
    start2, end2 = ht.event(), ht.event()
    ht.record(start2, sh)
    for i in range(steps_k):
        t, e = warmup + i, ev[i]
        ht.record(e[0], sh)
        loop.run_plan(t, sh)
        ht.record(e[1], sh)
        loop.run_gather(sh)
        ht.record(e[2], sh)
        loop.run_flash_cache(sh)
        ht.record(e[3], sh)
        loop.run_attention(sh)
        ht.record(e[4], sh)
        loop.run_topb(sh)
        ht.record(e[5], sh)
        loop.run_verify(t, sh)
        ht.record(e[6], sh)
    ht.record(end2, sh)
    torch.cuda.synchronize()
    instr_ms = ht.ms(start2, end2)
    same = same and bool(np.array_equal(loop.frontier.cpu().numpy(), fronts[-1]))
    per_call = {n: float(np.mean([ht.ms(e[j], e[j + 1]) for e in ev])) for j, n in enumerate(names)}
    timed_rows = rows[warmup:]
    committed = int(fronts[-1].sum() - fronts[warmup - 1].sum()) if warmup else \
        int(fronts[-1].sum() - wl.frontier0.astype(np.int64).sum())
    ms_per_step = total_ms / steps_k
    r_avg = float(np.mean(timed_rows))
    hd = wl.num_heads * wl.head_dim
    fc_flops = 2 * r_avg * wl.hid * 3 * hd
    fc_ms = per_call["flash_cache_step"]
    ridge = MFMA_BF16_PEAK_TFS * 1e12 / (HBM_PEAK_GBS * 1e9)
    fc_bytes = 2 * 3 * hd * wl.hid + r_avg * (2 * wl.hid + 2 * 3 * hd + 16)
    if fc_flops / fc_bytes >= ridge:
        ach = fc_flops / (fc_ms / 1e3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": MFMA_BF16_PEAK_TFS,
                "unit": "TFLOP/s", "frac": round(ach / MFMA_BF16_PEAK_TFS, 4)}
    else:
        ach = fc_bytes / (fc_ms / 1e3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4)}
    roof.update({"traffic": None, "kernel": "flash_cache_step (row capacity "
                 f"{loop.cap}, {r_avg:.0f} active rows on average)",
                 "algorithmic_flops": int(fc_flops), "avg_launch_us": round(fc_ms * 1e3, 2)})
    log(f"loop step {ms_per_step * 1e3:.1f} us; " +
        ", ".join(f"{n} {per_call[n] * 1e3:.1f} us" for n in names) +
        f"; frontiers reproduced: {same}")

    cpu = None
    if args.cpu_budget > 0:
        cpu = loop_cpu_baseline(wl, w, k0, v0, hc, hm, args.cpu_budget)
        log(f"cpu oracle loop {cpu['value']:.3f} steps/s")
    line = {
        "metric": LOOP_METRIC, "value": round(1e3 / ms_per_step, 1), "unit": "steps/s",
        "n_gpus": 1, "steps": steps_k, "warmup": warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": LOOP_WORKLOAD, "batch": wl.batch, "row_capacity": loop.cap,
                   "hidden": wl.hid, "heads": wl.num_heads, "head_dim": wl.head_dim},
        "active_rows_per_s": round(sum(timed_rows) / (total_ms / 1e3), 1),
        "committed_tokens_per_s": round(committed / (total_ms / 1e3), 1),
        "active_rows_per_step": round(r_avg, 1),
        "committed_tokens_per_step": round(committed / steps_k, 2),
        "roofline": roof,
        "cpu_baseline": cpu,
        "step_breakdown_us": {n: round(per_call[n] * 1e3, 2) for n in names},
        "ms_per_step_with_call_events": round(instr_ms / steps_k, 5),
        "frontiers_reproduced": same,
    }
    print(json.dumps(line), flush=True)


def loop_cpu_baseline(wl, w, k0, v0, hc, hm, budget_s):
    """The oracle loop over the whole batch from the same initial state, for
    one step (more if the budget allows a second): steps/s measured, not
    extrapolated (the oracle's per-step costs are not linear in the
    sequences: it widens the whole weight each step)."""
    import numpy as np
    import torch
    import oracle as O

    def host(t):
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    w_h, k_h, v_h, hc_h, hm_h = host(w), host(k0), host(v0), host(hc), host(hm)
    sc = wl.scan

    def run(n):
        t0 = time.perf_counter()
        O.decode_loop(n, w_h, wl.num_heads, wl.head_dim, wl.rope_base, wl.block_table,
                      wl.block_size, k_h, v_h, wl.kv_len, hc_h, hm_h, wl.frontier0, wl.tracked0,
                      wl.window_len, wl.topb, wl.refresh_period, sc["draft"], sc["mask"],
                      sc["conf"], sc["threshold"], mass_stride=wl.max_len)
        return time.perf_counter() - t0
    n_steps, el = 1, run(1)
    if 3 * el < budget_s:
        n_steps = min(wl.steps, int(budget_s / el))
        el = run(n_steps)
    return {"value": n_steps / el, "unit": "steps/s", "cores": int(_threads()), "kind": "oracle",
            "sample": f"oracle loop over the whole batch ({wl.batch} sequences) for {n_steps} "
                      f"step(s) from the same initial state ({el:.1f} s, fp64 numpy)"}


LM_METRIC = "mask-view confidence producer: scored rows/s (LM head + argmax + softmax confidence)"
LM_WORKLOAD = ("llada8b_lmhead_b8: the two-view batch-8 step's window rows (256 draft + 256 mask) "
               "through a 126464 x 4096 bf16 LM head; per row the argmax token and its softmax "
               "probability (logits never leave the chip), then verify_accept over 8 x 32")


def run_lm_head(args):
    """lm_head_confidence over the 512 window rows of the two-view batch-8 step
    (draft and mask views in one call) followed by the accept scan; duration
    from HIP events around each call on its stream."""
    import numpy as np
    import torch

    import kv_cache_attention_flash_amd as fd
    import synth

    steps_k = args.steps if args.steps is not None else 50
    warmup = args.warmup if args.warmup is not None else 5
    fd.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = synth.llada8b_lm_head_b8()
    w, hd, hm = synth.lm_head_tensors(wl, dev)
    h_all = torch.cat([hd, hm])
    rows = h_all.shape[0]
    tok = torch.empty((rows,), dtype=torch.int32, device=dev)
    conf = torch.empty((rows,), dtype=torch.float32, device=dev)
    acc = torch.empty((wl.batch,), dtype=torch.int32, device=dev)
    ws = torch.empty((fd.lm_head_workspace_bytes(rows, wl.vocab),), dtype=torch.uint8, device=dev)
    sh = torch.cuda.current_stream(dev).cuda_stream
    shape = (wl.batch, wl.window)
    dt, mt, mc = tok[:256].view(shape), tok[256:].view(shape), conf[256:].view(shape)

    def step():
        fd.lm_head_confidence(h_all, w, token_out=tok, conf_out=conf, workspace=ws, stream=sh)
        fd.verify_accept(dt, mt, mc, wl.threshold, out=acc, stream=sh)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ht = HipTimer()
    ev = [[ht.event() for _ in range(3)] for _ in range(steps_k)]
    start, end = ht.event(), ht.event()
    ht.record(start, sh)
    for e in ev:
        ht.record(e[0], sh)
        fd.lm_head_confidence(h_all, w, token_out=tok, conf_out=conf, workspace=ws, stream=sh)
        ht.record(e[1], sh)
        fd.verify_accept(dt, mt, mc, wl.threshold, out=acc, stream=sh)
        ht.record(e[2], sh)
    ht.record(end, sh)
    torch.cuda.synchronize()
    total_ms = ht.ms(start, end)
    lm_ms = float(np.mean([ht.ms(e[0], e[1]) for e in ev]))
    ver_ms = float(np.mean([ht.ms(e[1], e[2]) for e in ev]))
    flops = 2 * rows * wl.hid * wl.vocab
    nbytes = 2 * wl.vocab * wl.hid + rows * (2 * wl.hid + 8)
    ach = flops / (lm_ms / 1e3) / 1e12
    ridge = MFMA_BF16_PEAK_TFS * 1e12 / (HBM_PEAK_GBS * 1e9)
    assert flops / nbytes >= ridge
    roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": MFMA_BF16_PEAK_TFS,
            "unit": "TFLOP/s", "frac": round(ach / MFMA_BF16_PEAK_TFS, 4), "traffic": None,
            "kernel": "lm_head_confidence", "algorithmic_flops": flops,
            "algorithmic_bytes": nbytes, "avg_launch_us": round(lm_ms * 1e3, 2)}
    log(f"lm_head_confidence {lm_ms * 1e3:.1f} us ({ach:.0f} TFLOP/s), verify_accept "
        f"{ver_ms * 1e3:.1f} us; accept {acc.cpu().numpy().tolist()}")
    cpu = None
    if args.cpu_budget > 0:
        import oracle as O
        w_h = w.view(torch.int16).cpu().numpy().view(np.uint16)
        h_h = h_all.view(torch.int16).cpu().numpy().view(np.uint16)
        n = 16
        t0 = time.perf_counter()
        O.lm_head_confidence(h_h[:n], w_h)
        el = time.perf_counter() - t0
        cpu = {"value": n / el, "unit": "rows/s", "cores": int(_threads()), "kind": "oracle",
               "sample": f"{n} of the {rows} rows through the whole head (fp64 numpy, {el:.1f} s)"}
        log(f"cpu oracle {cpu['value']:.2f} rows/s")
    ms_per_step = total_ms / steps_k
    line = {
        "metric": LM_METRIC, "value": round(rows / (ms_per_step / 1e3), 1), "unit": "rows/s",
        "n_gpus": 1, "steps": steps_k, "warmup": warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": LM_WORKLOAD, "rows": rows, "vocab": wl.vocab, "hidden": wl.hid},
        "roofline": roof, "cpu_baseline": cpu,
        "step_breakdown_us": {"lm_head_confidence": round(lm_ms * 1e3, 2),
                              "verify_accept": round(ver_ms * 1e3, 2)},
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 200; 5 for the 32-layer stack)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps (default 20; 1 for the 32-layer stack)")
    ap.add_argument("--workload", default="llada8b_stack32_b16_l4096", choices=sorted(WORKLOADS))
    ap.add_argument("--copies", type=int, default=0,
                    help="resident copies rotated per step (0: enough to exceed ~560 MB)")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle timing for the cpu_baseline (0 disables it)")
    ap.add_argument("--unfused", action="store_true",
                    help="time the three-launch ablation (flash_cache_step_unfused) instead of the "
                         "fused projection step")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one 100 MiB device-to-device copy before timing (a dispatch of "
                         "known size that scales rocprofv3 FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--fused", action="store_true",
                    help="time flash_cache_attention_step (projection, attention and mass in one "
                         "call) in place of the two calls")
    ap.add_argument("--single-launch", action="store_true",
                    help="time flash_cache_attention_step_single_launch (projection, attention "
                         "and mass in one persistent launch) in place of the two calls")
    ap.add_argument("--loop", action="store_true",
                    help="time the multi-step decode loop (batch 32, planned on the device) and "
                         "report steps/s instead of the single-step metric")
    ap.add_argument("--lm-head", action="store_true",
                    help="time the mask-view confidence producer (LM head over 512 window rows) "
                         "and the accept scan, instead of the single-step metric")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for {args.gpus}). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.loop:
        run_loop(args)
        return
    if args.lm_head:
        run_lm_head(args)
        return
    stack = args.workload == "llada8b_stack32_b16_l4096"
    steps_k = args.steps if args.steps is not None else (5 if stack else 200)
    warmup = args.warmup if args.warmup is not None else (1 if stack else 20)

    import numpy as np
    import torch

    import kv_cache_attention_flash_amd as fd
    import synth

    fd.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if stack:
        wl = synth.llada8b_stack32_layout()
    else:
        wl = {"llada8b_b1_l768": synth.llada8b_b1, "llada8b_ragged_b32": synth.llada8b_ragged_b32,
              "llada8b_verify_b8": synth.llada8b_verify_b8}[args.workload]()
    log(f"workload {wl.name}: rows={wl.rows} hidden={wl.hid} heads={wl.num_heads}x{wl.head_dim} "
        f"batch={wl.batch} max_kv_len={wl.max_kv_len} topb={wl.topb} layers={wl.layers}")

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    def i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)

    cu, pos, slots, kv = i32(wl.cu_rows), i32(wl.positions), i32(wl.slots), i32(wl.kv_len)
    bt = i32(wl.block_table)
    views = i32(wl.views) if wl.views is not None else None
    verify = None
    if wl.verify is not None:
        v = wl.verify
        nb = wl.batch  # the scan runs on the step's sequences (the crafted rows are test cases)
        verify = (i32(v["draft"][:nb]), i32(v["mask"][:nb]),
                  torch.from_numpy(np.ascontiguousarray(v["conf"][:nb])).to(dev),
                  float(v["threshold"]))
    max_rows = int(np.diff(wl.cu_rows).max())

    def make_step(cache, x, w):
        return fd.DecodeStep(cache, x, w, cu, pos, slots, kv, wl.rope_base, wl.max_kv_len,
                             max_rows, views=views, topb=wl.topb, verify=verify,
                             unfused=args.unfused, fused=args.fused,
                             single_launch=args.single_launch)

    # units[i % len(units)] = the per-layer steps that make up logical step i
    units = []
    if stack:
        layer_steps = []
        for layer in range(wl.layers):
            x, w, k, v = synth.stack_layer_tensors(wl, layer, dev)
            layer_steps.append(make_step(fd.PagedKVCache(k, v, bt), x, w))
        units.append(layer_steps)
        layers_per_step = wl.layers
        log(f"stack resident: {torch.cuda.memory_allocated(dev) / 1e9:.1f} GB")
    else:
        per_copy = 2 * (wl.x.size + wl.w.size + wl.k_cache.size + wl.v_cache.size)
        copies = args.copies or max(1, math.ceil(ROTATION_BYTES / per_copy))
        for _ in range(copies):
            cache = fd.PagedKVCache(bf(wl.k_cache), bf(wl.v_cache), bt)
            units.append([make_step(cache, bf(wl.x), bf(wl.w))])
        layers_per_step = 1
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream

    if args.calibrate_copy:
        src = torch.ones(100 * 1024 * 1024, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for i in range(warmup):
        for st in units[i % len(units)]:
            st.run(sh)
    torch.cuda.synchronize()
    log(f"warm-up done ({warmup} steps, {len(units)} resident unit(s))")

    K = steps_k
    ht = HipTimer()
    # Pass 1: K steps exactly as they run (nothing recorded between the calls):
    # the step time and `value`.  Each event record between kernels costs
    # about a microsecond of GPU time, so the per-call brackets come from
    # pass 2, K more steps with an event around every call.
    start, end = ht.event(), ht.event()
    torch.cuda.synchronize()
    ht.record(start, sh)
    for i in range(K):
        for st in units[i % len(units)]:
            st.run(sh)
    ht.record(end, sh)
    torch.cuda.synchronize()
    total_ms = ht.ms(start, end)
    ms_per_step = total_ms / K

    ev = [[[ht.event() for _ in range(3)] for _ in units[i % len(units)]] for i in range(K)]
    start2, end2 = ht.event(), ht.event()
    torch.cuda.synchronize()
    ht.record(start2, sh)
    for i in range(K):
        for st, e in zip(units[i % len(units)], ev[i]):
            ht.record(e[0], sh)
            if args.fused or args.single_launch:
                st.run_fused(sh)  # one call: its time is booked to the first bracket
            else:
                st.run_flash_cache(sh)
            ht.record(e[1], sh)
            if not (args.fused or args.single_launch):
                st.run_attention(sh)
            ht.record(e[2], sh)
            st.run_topb(sh)
            st.run_verify(sh)
    ht.record(end2, sh)
    torch.cuda.synchronize()
    ms_per_step_instr = ht.ms(start2, end2) / K
    fcs_ms = float(np.mean([ht.ms(e[0], e[1]) for evs in ev for e in evs]))
    att_ms = float(np.mean([ht.ms(e[1], e[2]) for evs in ev for e in evs]))
    value = wl.rows * layers_per_step / (ms_per_step / 1e3)

    fc_call = "flash_cache_step_unfused" if args.unfused else "flash_cache_step"
    rf_fc = roofline_entry(fc_call, wl, fcs_ms, args.workload)
    rf_att = roofline_entry("scheduled_attention", wl, att_ms, args.workload)
    dominant, other = (rf_fc, rf_att) if fcs_ms >= att_ms else (rf_att, rf_fc)
    if args.fused or args.single_launch:
        # one call: its algorithmic bytes are both calls' (HBM-bound at this AI)
        nb_f = step_bytes(wl)
        ach = nb_f / (fcs_ms / 1e3) / 1e9
        dominant = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None,
                    "kernel": ("flash_cache_attention_step_single_launch" if args.single_launch
                               else "flash_cache_attention_step"), "algorithmic_bytes": nb_f,
                    "algorithmic_flops": flash_cache_flops(wl) + attention_flops(wl),
                    "avg_launch_us": round(fcs_ms * 1e3, 2)}
        other = None
    log(f"step {ms_per_step * 1e3:.1f} us ({layers_per_step} layer(s)); flash_cache_step "
        f"{fcs_ms * 1e3:.1f} us ({rf_fc['achieved']} {rf_fc['unit']}); scheduled_attention "
        f"{att_ms * 1e3:.1f} us ({rf_att['achieved']} {rf_att['unit']})")

    cpu, parity = None, None
    if args.cpu_budget > 0:
        st = units[0][0]
        if stack:
            # Layer 0 as it is on the device now: the timed steps rewrote the
            # active slots with the same values, so the pools are valid inputs.
            def host(t):
                return t.view(torch.int16).cpu().numpy().view(np.uint16)
            x_h, w_h = host(st.x), host(st.w)
            k_h, v_h = host(st.cache.k_cache), host(st.cache.v_cache)
            seqs, desc = [0], "layer 0, sequence 0 of 16"
        else:
            x_h, w_h, k_h, v_h = wl.x, wl.w, wl.k_cache, wl.v_cache
            seqs = list(range(wl.batch)) if wl.batch <= 8 else [0, 1]
            desc = ("the whole workload" if len(seqs) == wl.batch
                    else f"sequences {seqs} of {wl.batch}")
        sub = sequence_subset(wl, seqs, x_h, k_h, v_h)
        cpu, ref = cpu_baseline(wl, sub, w_h, args.cpu_budget, desc)
        parity = parity_against(ref, sub, st, wl)
        log(f"cpu oracle {cpu['value']:.1f} tokens/s/layer on {cpu['cores']} threads; parity {parity}")

    hd = wl.num_heads * wl.head_dim
    sb = step_bytes(wl)
    layer_s = ms_per_step / layers_per_step / 1e3
    step_ach = sb / layer_s / 1e9
    step_roof = {"bound": "hbm", "achieved": round(step_ach, 1), "peak": HBM_PEAK_GBS,
                 "unit": "GB/s", "frac": round(step_ach / HBM_PEAK_GBS, 4),
                 "algorithmic_bytes": sb, "layer_us": round(layer_s * 1e6, 2),
                 "what": "one layer's whole step (every call of it) against its algorithmic "
                         "bytes: W + R(2 hid + 4 HD + 4 HD) + 4 HD sum(L) + 4 sum(L)"}
    tail = (" + scheduled_attention(+mass) + track_topb" if wl.topb else " + scheduled_attention")
    if args.unfused:
        tail += " [ablation: flash_cache_step_unfused, three launches with HBM intermediates]"
    if args.single_launch:
        tail += (" [flash_cache_attention_step_single_launch: projection, attention and mass in "
                 "one persistent launch; its whole time is in the flash_cache_step bracket]")
    elif args.fused:
        tail += (" [flash_cache_attention_step: projection, attention and mass in one call; "
                 "its whole time is in the flash_cache_step bracket]")
    tail += " + verify_accept" if verify is not None else ""
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s/layer", "n_gpus": 1,
        "steps": K, "warmup": warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: {WORKLOADS[args.workload]}; "
                               f"step = flash_cache_step{tail}",
                   "batch": wl.batch, "active_rows": wl.rows, "max_kv_len": wl.max_kv_len,
                   "hidden": wl.hid, "heads": wl.num_heads, "head_dim": wl.head_dim,
                   "layers_per_step": layers_per_step, "resident_units": len(units)},
        "roofline": dominant,
        "roofline_other": other,
        "cpu_baseline": cpu,
        "step_breakdown_us": {"flash_cache_step": round(fcs_ms * 1e3, 2),
                              "scheduled_attention": round(att_ms * 1e3, 2),
                              "layer_total": round(ms_per_step * 1e3 / layers_per_step, 2),
                              "layer_total_with_call_events": round(
                                  ms_per_step_instr * 1e3 / layers_per_step, 2)},
        "step_roofline": step_roof,
        "step_hbm_fraction": step_roof["frac"],
        "step_algorithmic_bytes": sb,
        "non_algorithmic_bytes": {"q_round_trip": q_round_trip_bytes(wl)},
        "qkv_dims": [wl.rows, wl.hid, 3 * hd],
        "parity": parity,
    }
    print(json.dumps(line), flush=True)
    # Release the resident tensors while the runtime is whole, in a fixed order.
    torch.cuda.synchronize()
    units = st = None
    torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
