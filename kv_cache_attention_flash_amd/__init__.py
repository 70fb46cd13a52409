"""MI355X (gfx950) implementation of the per-layer hot path of one Flash-dLLM
decoding step, behind a small C ABI (include/fdllm.h, libfdllm.so).

This package is argument marshalling only: every step of the path runs in the
HIP kernels of libfdllm.so.  torch provides device memory and streams.  If the
library is missing every call raises; nothing falls back to the CPU.

Calls (same names as the C ABI):
  flash_cache_step     QKV projection + rotary embedding + paged cache write
  scheduled_attention  block-table attention (two-view mask; optional mass)
  track_topb           next tracking set from the attention mass
  verify_accept        Flash-Verify accepted-prefix lengths
  decode_plan          next loop step's rows, planned on the device
  gather_hidden        hidden-state rows of the planned rows
  lm_head_confidence   argmax token and softmax confidence of each row (LM head)
  flash_cache_attention_step  flash_cache_step + scheduled_attention (+ mass) in one call
  flash_cache_attention_step_single_launch  the same as one persistent launch (slower here)

DecodeStep binds one step to fixed buffers; DecodeLoop chains steps with the
planning on the device (no host round trip between steps).

Page key: [P4] "Flash-dLLM: I/O-Aware KV Caching and Parallel Decoding for Fast,
Memory-Efficient Diffusion LLMs" (ai4snews.wisdomeyes.cn summary), paras 1-3.
"""

from __future__ import annotations

import atexit
import contextlib
import ctypes
import dataclasses
from typing import Optional

import torch

from . import _lib
from ._lib import FdlError, KVCacheStruct  # noqa: F401

__all__ = ["PagedKVCache", "flash_cache_step", "flash_cache_step_unfused", "scheduled_attention",
           "track_topb", "verify_accept", "attention_workspace_bytes",
           "flash_cache_workspace_bytes", "flash_cache_unfused_workspace_bytes", "DecodeStep",
           "decode_plan", "gather_hidden", "DecodeLoop", "lm_head_confidence",
           "lm_head_workspace_bytes", "flash_cache_attention_step",
           "flash_cache_attention_step_single_launch", "fused_step_workspace_bytes",
           "fused_step_error", "attention_error", "attention_path", "scheduled_attention_static",
           "static_scratch_bytes", "FdlError", "load"]


def load():
    return _lib.load()


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, ndim: Optional[int] = None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device, got {t.device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")


def _on_stream(stream_handle: int, device):
    """Context in which torch allocates (and fills) in the order of the launch
    stream: memory handed to a call on that stream is then free with respect to
    it, and a fill (zeros) is complete before the call's kernels start.  A
    no-op when the launch stream is torch's current stream."""
    if torch.cuda.current_stream(device).cuda_stream == stream_handle:
        return contextlib.nullcontext()
    return torch.cuda.stream(torch.cuda.ExternalStream(stream_handle, device=device))


_FC_WS = {}


def _flash_cache_workspace(device, stream_handle: int, nbytes: int):
    """Split-reduction scratch, one per (device, stream), allocated in the
    stream's order."""
    key = (device.index if device.index is not None else torch.cuda.current_device(), stream_handle)
    ws = _FC_WS.get(key)
    if ws is None or ws.numel() < nbytes:
        with _on_stream(stream_handle, device):
            ws = torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=device)
        _FC_WS[key] = ws
    return ws


def _release_cached_workspaces():
    """At interpreter exit: wait for the device, then drop the cached
    workspaces while the HIP runtime is still whole, so that their memory is
    returned in a fixed order rather than during interpreter teardown."""
    if not (_FC_WS or _FUSED_WS):
        return
    try:
        torch.cuda.synchronize()
    except Exception:  # pragma: no cover - nothing more to do at exit
        pass
    _FC_WS.clear()
    _FUSED_WS.clear()


atexit.register(_release_cached_workspaces)


def flash_cache_workspace_bytes(num_rows, hidden, num_heads, head_dim) -> int:
    return int(_lib.load().fdl_flash_cache_workspace_bytes(num_rows, hidden, num_heads, head_dim))


def _stream(stream, device) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


@dataclasses.dataclass
class PagedKVCache:
    """One layer's paged cache: bf16 pools [num_blocks, H, block_size, D] and an
    int32 block table [batch, max_blocks_per_seq] (logical -> physical block)."""
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    block_table: torch.Tensor

    def __post_init__(self):
        _need(self.k_cache, "k_cache", torch.bfloat16, 4)
        _need(self.v_cache, "v_cache", torch.bfloat16, 4)
        _need(self.block_table, "block_table", torch.int32, 2)
        if self.k_cache.shape != self.v_cache.shape:
            raise ValueError("k_cache and v_cache shapes differ")

    @property
    def num_blocks(self):
        return self.k_cache.shape[0]

    @property
    def num_heads(self):
        return self.k_cache.shape[1]

    @property
    def block_size(self):
        return self.k_cache.shape[2]

    @property
    def head_dim(self):
        return self.k_cache.shape[3]

    def struct(self) -> KVCacheStruct:
        return KVCacheStruct(self.num_heads, self.head_dim, self.block_size, self.num_blocks,
                             self.block_table.shape[1], self.k_cache.data_ptr(),
                             self.v_cache.data_ptr(), self.block_table.data_ptr())


def _flash_cache_call(unfused, cache, x, w_qkv, cu_rows, positions, slots, rope_base, q_out,
                      slot_mapping_out, stream):
    lib = _lib.load()
    _need(x, "x", torch.bfloat16, 2)
    _need(w_qkv, "w_qkv", torch.bfloat16, 2)
    for t, n in ((cu_rows, "cu_rows"), (positions, "positions"), (slots, "slots")):
        _need(t, n, torch.int32, 1)
    r, hid = x.shape
    h, d = cache.num_heads, cache.head_dim
    if tuple(w_qkv.shape) != (3 * h * d, hid):
        raise ValueError(f"w_qkv must be [{3 * h * d}, {hid}], got {tuple(w_qkv.shape)}")
    if positions.numel() != r or slots.numel() != r:
        raise ValueError("positions/slots must have one entry per row")
    batch = cu_rows.numel() - 1
    sh = _stream(stream, x.device)
    with _on_stream(sh, x.device):
        if q_out is None:
            q_out = torch.empty((r, h, d), dtype=torch.bfloat16, device=x.device)
        if slot_mapping_out is None:
            slot_mapping_out = torch.empty((r,), dtype=torch.int64, device=x.device)
    _need(q_out, "q_out", torch.bfloat16, 3)
    _need(slot_mapping_out, "slot_mapping_out", torch.int64, 1)
    cs = cache.struct()
    if unfused:
        need = flash_cache_unfused_workspace_bytes(r, hid, h, d)
        fn, name = lib.flash_cache_step_unfused, "flash_cache_step_unfused"
    else:
        need = flash_cache_workspace_bytes(r, hid, h, d)
        fn, name = lib.flash_cache_step, "flash_cache_step"
    ws = _flash_cache_workspace(x.device, sh, need) if need else None
    st = fn(ctypes.byref(cs), x.data_ptr(), hid, w_qkv.data_ptr(), batch, r, cu_rows.data_ptr(),
            positions.data_ptr(), slots.data_ptr(), float(rope_base), q_out.data_ptr(),
            slot_mapping_out.data_ptr(), _ptr(ws), need, sh)
    _lib.check(name, st)
    return q_out, slot_mapping_out


def flash_cache_step(cache: PagedKVCache, x, w_qkv, cu_rows, positions, slots, rope_base,
                     q_out=None, slot_mapping_out=None, stream=None):
    """Fused QKV projection + RoPE + K/V cache write for the active rows.
    Returns (q_out bf16 [R, H, D], slot_mapping int64 [R])."""
    return _flash_cache_call(False, cache, x, w_qkv, cu_rows, positions, slots, rope_base, q_out,
                             slot_mapping_out, stream)


def flash_cache_step_unfused(cache: PagedKVCache, x, w_qkv, cu_rows, positions, slots,
                             rope_base, q_out=None, slot_mapping_out=None, stream=None):
    """The same step as three launches with the intermediates in HBM (the
    unfused ablation); bitwise the same results as flash_cache_step."""
    return _flash_cache_call(True, cache, x, w_qkv, cu_rows, positions, slots, rope_base, q_out,
                             slot_mapping_out, stream)


def flash_cache_unfused_workspace_bytes(num_rows, hidden, num_heads, head_dim) -> int:
    return int(_lib.load().fdl_flash_cache_unfused_workspace_bytes(num_rows, hidden, num_heads,
                                                                  head_dim))

def attention_workspace_bytes(batch, num_rows, num_heads, head_dim, max_kv_len,
                              max_rows_per_seq, mass_stride=0) -> int:
    return int(_lib.load().fdl_attention_workspace_bytes(batch, num_rows, num_heads, head_dim,
                                                         max_kv_len, max_rows_per_seq,
                                                         mass_stride))


ATTENTION_PATHS = {1: "row_groups", 2: "split", 3: "split_mass_exchange", 4: "split_mass_reread"}


def attention_path(batch, num_rows, num_heads, head_dim, max_kv_len, max_rows_per_seq,
                   mass_stride=0) -> str:
    """Which kernels scheduled_attention runs for these sizes (see include/fdllm.h)."""
    k = int(_lib.load().fdl_attention_path(batch, num_rows, num_heads, head_dim, max_kv_len,
                                           max_rows_per_seq, mass_stride))
    if k not in ATTENTION_PATHS:
        raise ValueError("invalid sizes")
    return ATTENTION_PATHS[k]


def scheduled_attention(cache: PagedKVCache, q, cu_rows, kv_len, max_kv_len, max_rows_per_seq,
                        views=None, softmax_scale=0.0, out=None, want_mass=False, mass=None,
                        mass_stride=None, workspace=None, stream=None):
    """Block-table attention of the active rows (two-view mask when ``views`` is
    given, int32 [batch, 3]).  Returns (out fp32 [R, H, D], mass fp32
    [batch, mass_stride] or None)."""
    lib = _lib.load()
    _need(q, "q", torch.bfloat16, 3)
    _need(cu_rows, "cu_rows", torch.int32, 1)
    _need(kv_len, "kv_len", torch.int32, 1)
    batch = kv_len.numel()
    if cu_rows.numel() != batch + 1:
        raise ValueError("cu_rows must have batch + 1 entries")
    if views is not None:
        _need(views, "views", torch.int32, 2)
        if tuple(views.shape) != (batch, 3):
            raise ValueError("views must be int32 [batch, 3]")
    r = q.shape[0]
    sh = _stream(stream, q.device)
    with _on_stream(sh, q.device):
        if out is None:
            out = torch.empty((r, cache.num_heads, cache.head_dim), dtype=torch.float32,
                              device=q.device)
        if (want_mass or mass is not None) and mass is None:
            if mass_stride is None:
                mass_stride = int(max_kv_len)
            mass = torch.empty((batch, mass_stride), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, 3)
    if mass is not None:
        if mass_stride is None:
            mass_stride = mass.shape[1]
        _need(mass, "mass", torch.float32, 2)
    ms = int(mass_stride) if mass is not None else 0
    need = attention_workspace_bytes(batch, r, cache.num_heads, cache.head_dim, int(max_kv_len),
                                     int(max_rows_per_seq), ms)
    if workspace is None or workspace.numel() < need:
        with _on_stream(sh, q.device):
            workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=q.device)
    cs = cache.struct()
    st = lib.scheduled_attention(ctypes.byref(cs), q.data_ptr(), batch, r, cu_rows.data_ptr(),
                                 kv_len.data_ptr(), int(max_kv_len), int(max_rows_per_seq),
                                 _ptr(views), float(softmax_scale), out.data_ptr(),
                                 _ptr(mass), ms, workspace.data_ptr(), workspace.numel(), sh)
    _lib.check("scheduled_attention", st)
    return out, mass


ATTENTION_ERROR_OFFSET = 4  # byte offset of scheduled_attention's error word in its workspace


def attention_error(workspace: torch.Tensor, stream=None) -> int:
    """scheduled_attention's error word, for calls whose cache needs more than
    one 1024-key split with the mass asked for (the splits wait for each
    other): 1 if such a wait ever timed out on this workspace (those results
    are invalid; the word stays set until cleared), else 0.  Synchronises the
    stream."""
    sh = _stream(stream, workspace.device)
    with _on_stream(sh, workspace.device):
        word = workspace[ATTENTION_ERROR_OFFSET:ATTENTION_ERROR_OFFSET + 4].view(torch.int32).item()
    return int(word)


def static_scratch_bytes() -> int:
    return int(_lib.load().fdl_static_scratch_bytes())


def scheduled_attention_static(cache: PagedKVCache, q, cu_rows, kv_len, max_kv_len,
                               max_rows_per_seq, out, mass=None, views=None, softmax_scale=0.0,
                               stream=None):
    """scheduled_attention without a workspace, for callers that cannot
    allocate: the library's static per-GPU scratch buffer stands in for it
    (include/fdllm.h).  Nothing is allocated here either: ``out`` (and
    ``mass`` when the mass is wanted) must be given.  Returns (out, mass)."""
    lib = _lib.load()
    _need(q, "q", torch.bfloat16, 3)
    _need(cu_rows, "cu_rows", torch.int32, 1)
    _need(kv_len, "kv_len", torch.int32, 1)
    _need(out, "out", torch.float32, 3)
    batch = kv_len.numel()
    if cu_rows.numel() != batch + 1:
        raise ValueError("cu_rows must have batch + 1 entries")
    if views is not None:
        _need(views, "views", torch.int32, 2)
    ms = 0
    if mass is not None:
        _need(mass, "mass", torch.float32, 2)
        ms = mass.shape[1]
    cs = cache.struct()
    st = lib.scheduled_attention_static(ctypes.byref(cs), q.data_ptr(), batch, q.shape[0],
                                        cu_rows.data_ptr(), kv_len.data_ptr(), int(max_kv_len),
                                        int(max_rows_per_seq), _ptr(views), float(softmax_scale),
                                        out.data_ptr(), _ptr(mass), ms, _stream(stream, q.device))
    _lib.check("scheduled_attention_static", st)
    return out, mass


def track_topb(mass, kv_len, topb, out=None, stream=None):
    """Top-``topb`` most-attended keys per sequence, ascending indices, -1 padded."""
    lib = _lib.load()
    _need(mass, "mass", torch.float32, 2)
    _need(kv_len, "kv_len", torch.int32, 1)
    batch = mass.shape[0]
    if kv_len.numel() != batch:
        raise ValueError("kv_len must have one entry per sequence")
    sh = _stream(stream, mass.device)
    if out is None:
        with _on_stream(sh, mass.device):
            out = torch.empty((batch, int(topb)), dtype=torch.int32, device=mass.device)
    _need(out, "out", torch.int32, 2)
    st = lib.track_topb(mass.data_ptr(), mass.shape[1], kv_len.data_ptr(), batch, int(topb),
                        out.data_ptr(), sh)
    _lib.check("track_topb", st)
    return out


def verify_accept(draft_tok, mask_tok, conf, threshold, out=None, stream=None):
    """Accepted-prefix length per sequence (int32 [batch])."""
    lib = _lib.load()
    _need(draft_tok, "draft_tok", torch.int32, 2)
    _need(mask_tok, "mask_tok", torch.int32, 2)
    _need(conf, "conf", torch.float32, 2)
    if draft_tok.shape != mask_tok.shape or draft_tok.shape != conf.shape:
        raise ValueError("draft_tok, mask_tok and conf must have the same shape")
    batch, window = draft_tok.shape
    sh = _stream(stream, draft_tok.device)
    if out is None:
        with _on_stream(sh, draft_tok.device):
            out = torch.empty((batch,), dtype=torch.int32, device=draft_tok.device)
    _need(out, "out", torch.int32, 1)
    st = lib.verify_accept(draft_tok.data_ptr(), mask_tok.data_ptr(), conf.data_ptr(), batch,
                           window, ctypes.c_float(float(threshold)), out.data_ptr(), sh)
    _lib.check("verify_accept", st)
    return out


class DecodeStep:
    """One per-layer decode step bound to fixed device buffers:
    flash_cache_step -> scheduled_attention (+ mass) -> track_topb, and the
    accept scan when ``verify`` inputs are given.

    The ctypes argument lists are built once, so ``run()`` only issues the three
    asynchronous library calls on the given stream (suitable for timing loops
    and HIP-graph capture).  The buffers are allocated on torch's current
    stream at construction; a caller that runs the step on another stream
    keeps the object alive until that stream is done with it."""

    def __init__(self, cache: PagedKVCache, x, w_qkv, cu_rows, positions, slots, kv_len,
                 rope_base, max_kv_len, max_rows_per_seq, views=None, topb=0,
                 softmax_scale=0.0, verify=None, unfused=False, fused=False,
                 single_launch=False):
        self.lib = _lib.load()
        dev = x.device
        r = x.shape[0]
        h, d = cache.num_heads, cache.head_dim
        self.cache, self.x, self.w = cache, x, w_qkv
        self.cu_rows, self.positions, self.slots, self.kv_len, self.views = (
            cu_rows, positions, slots, kv_len, views)
        self.batch = kv_len.numel()
        self.rows = r
        self.topb = int(topb)
        self.q = torch.empty((r, h, d), dtype=torch.bfloat16, device=dev)
        self.slot_mapping = torch.empty((r,), dtype=torch.int64, device=dev)
        self.out = torch.empty((r, h, d), dtype=torch.float32, device=dev)
        self.mass_stride = int(max_kv_len)
        self.mass = (torch.empty((self.batch, self.mass_stride), dtype=torch.float32, device=dev)
                     if self.topb else None)
        self.idx = (torch.empty((self.batch, self.topb), dtype=torch.int32, device=dev)
                    if self.topb else None)
        ms = self.mass_stride if self.topb else 0
        need = attention_workspace_bytes(self.batch, r, h, d, int(max_kv_len),
                                         int(max_rows_per_seq), ms)
        self.workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
        # unfused: the three-launch ablation of the projection step
        self._fc_fn = self.lib.flash_cache_step_unfused if unfused else self.lib.flash_cache_step
        self._fc_name = "flash_cache_step_unfused" if unfused else "flash_cache_step"
        fneed = (flash_cache_unfused_workspace_bytes if unfused else flash_cache_workspace_bytes)(
            r, x.shape[1], h, d)
        self.fc_workspace = torch.empty((max(fneed, 1),), dtype=torch.uint8, device=dev)
        self.cs = cache.struct()
        self._fcs = (ctypes.byref(self.cs), x.data_ptr(), x.shape[1], w_qkv.data_ptr(),
                     self.batch, r, cu_rows.data_ptr(), positions.data_ptr(), slots.data_ptr(),
                     float(rope_base), self.q.data_ptr(), self.slot_mapping.data_ptr(),
                     self.fc_workspace.data_ptr(), fneed)
        self._att = (ctypes.byref(self.cs), self.q.data_ptr(), self.batch, r, cu_rows.data_ptr(),
                     kv_len.data_ptr(), int(max_kv_len), int(max_rows_per_seq), _ptr(views),
                     float(softmax_scale), self.out.data_ptr(), _ptr(self.mass), ms,
                     self.workspace.data_ptr(), self.workspace.numel())
        self._top = ((self.mass.data_ptr(), self.mass_stride, kv_len.data_ptr(), self.batch,
                      self.topb, self.idx.data_ptr()) if self.topb else None)
        # fused: flash_cache_attention_step in place of the two calls (needs the
        # mass); single_launch: its one-kernel form.
        self._fus = None
        self._fus_fn = (self.lib.flash_cache_attention_step_single_launch if single_launch
                        else self.lib.flash_cache_attention_step)
        self._fus_name = ("flash_cache_attention_step_single_launch" if single_launch
                          else "flash_cache_attention_step")
        if fused or single_launch:
            if not self.topb:
                raise ValueError("the one-call step forms the mass: topb must be > 0")
            fus_need = fused_step_workspace_bytes(self.batch, r, h, d, int(max_kv_len),
                                                  int(max_rows_per_seq), self.mass_stride)
            self.fused_workspace = torch.zeros((max(fus_need, 256),), dtype=torch.uint8,
                                               device=dev)
            # run() may use another stream: the fill must be complete first
            torch.cuda.current_stream(dev).synchronize()
            self._fus = (ctypes.byref(self.cs), x.data_ptr(), x.shape[1], w_qkv.data_ptr(),
                         self.batch, r, cu_rows.data_ptr(), positions.data_ptr(),
                         slots.data_ptr(), float(rope_base), self.q.data_ptr(),
                         self.slot_mapping.data_ptr(), kv_len.data_ptr(), int(max_kv_len),
                         int(max_rows_per_seq), _ptr(views), float(softmax_scale),
                         self.out.data_ptr(), self.mass.data_ptr(), self.mass_stride,
                         self.fused_workspace.data_ptr(), self.fused_workspace.numel())
        # Optional accept scan after the step: (draft, mask, conf, threshold).
        self._ver = None
        if verify is not None:
            d, m, c, thr = verify
            _need(d, "draft_tok", torch.int32, 2)
            _need(m, "mask_tok", torch.int32, 2)
            _need(c, "conf", torch.float32, 2)
            self.verify_inputs = (d, m, c)
            self.accept_len = torch.empty((d.shape[0],), dtype=torch.int32, device=dev)
            self._ver = (d.data_ptr(), m.data_ptr(), c.data_ptr(), d.shape[0], d.shape[1],
                         ctypes.c_float(float(thr)), self.accept_len.data_ptr())

    def run_flash_cache(self, stream: int):
        _lib.check(self._fc_name, self._fc_fn(*self._fcs, stream))

    def run_fused(self, stream: int):
        _lib.check(self._fus_name, self._fus_fn(*self._fus, stream))

    def fused_error(self) -> int:
        """The single-launch step's error word after the runs so far (waits
        for the device); 0 when every wait completed."""
        torch.cuda.synchronize(self.x.device)
        return int(self.fused_workspace[FUSED_ERROR_OFFSET:FUSED_ERROR_OFFSET + 4]
                   .view(torch.int32).item())

    def run_attention(self, stream: int):
        _lib.check("scheduled_attention", self.lib.scheduled_attention(*self._att, stream))

    def run_topb(self, stream: int):
        if self._top is not None:
            _lib.check("track_topb", self.lib.track_topb(*self._top, stream))

    def run_verify(self, stream: int):
        if self._ver is not None:
            _lib.check("verify_accept", self.lib.verify_accept(*self._ver, stream))

    def run(self, stream: Optional[int] = None):
        s = _stream(stream, self.x.device) if not isinstance(stream, int) else stream
        if self._fus is not None:
            self.run_fused(s)
        else:
            self.run_flash_cache(s)
            self.run_attention(s)
        self.run_topb(s)
        self.run_verify(s)


def decode_plan(kv_len, frontier, tracked, accept_len, step, window_len, block_size,
                refresh_period, cu_rows_out=None, positions_out=None, slots_out=None,
                stage_out=None, stream=None):
    """Plan loop step ``step`` on the device (rules in include/fdllm.h):
    commits the previous accept lengths into ``frontier`` (in place) and writes
    the rows.  Returns (cu_rows int32 [batch+1], positions, slots int32
    [capacity], stage int32 [batch]) with capacity = batch * (W + topb)."""
    lib = _lib.load()
    _need(kv_len, "kv_len", torch.int32, 1)
    _need(frontier, "frontier", torch.int32, 1)
    batch = kv_len.numel()
    if frontier.numel() != batch:
        raise ValueError("frontier must have one entry per sequence")
    topb = 0
    if tracked is not None:
        _need(tracked, "tracked", torch.int32, 2)
        if tracked.shape[0] != batch:
            raise ValueError("tracked must be int32 [batch, topb]")
        topb = tracked.shape[1]
    if accept_len is not None:
        _need(accept_len, "accept_len", torch.int32, 1)
        if accept_len.numel() != batch:
            raise ValueError("accept_len must have one entry per sequence")
    dev = kv_len.device
    cap = batch * (int(window_len) + topb)
    sh = _stream(stream, dev)
    with _on_stream(sh, dev):
        if cu_rows_out is None:
            cu_rows_out = torch.empty((batch + 1,), dtype=torch.int32, device=dev)
        if positions_out is None:
            positions_out = torch.empty((max(cap, 1),), dtype=torch.int32, device=dev)
        if slots_out is None:
            slots_out = torch.empty((max(cap, 1),), dtype=torch.int32, device=dev)
        if stage_out is None:
            stage_out = torch.empty((max(batch, 1),), dtype=torch.int32, device=dev)
    for t, n in ((cu_rows_out, "cu_rows_out"), (positions_out, "positions_out"),
                 (slots_out, "slots_out"), (stage_out, "stage_out")):
        _need(t, n, torch.int32, 1)
    if positions_out.numel() < cap or slots_out.numel() < cap:
        raise ValueError(f"positions_out/slots_out need {cap} entries")
    st = lib.decode_plan(batch, kv_len.data_ptr(), int(window_len), int(block_size),
                         int(refresh_period), int(step), _ptr(tracked), topb, _ptr(accept_len),
                         frontier.data_ptr(), cu_rows_out.data_ptr(), positions_out.data_ptr(),
                         slots_out.data_ptr(), stage_out.data_ptr(), positions_out.numel(), sh)
    _lib.check("decode_plan", st)
    return cu_rows_out, positions_out, slots_out, stage_out


def gather_hidden(cu_rows, positions, frontier, hidden_committed, hidden_masked, x_out=None,
                  stream=None):
    """Hidden-state rows of the planned rows: the committed-token table's row
    for positions below the frontier, the masked-token table's otherwise
    (tables bf16 [batch, max_len, hidden]).  Returns x_out bf16 [capacity, hidden]."""
    lib = _lib.load()
    _need(cu_rows, "cu_rows", torch.int32, 1)
    _need(positions, "positions", torch.int32, 1)
    _need(frontier, "frontier", torch.int32, 1)
    _need(hidden_committed, "hidden_committed", torch.bfloat16, 3)
    _need(hidden_masked, "hidden_masked", torch.bfloat16, 3)
    if hidden_committed.shape != hidden_masked.shape:
        raise ValueError("the two hidden-state tables must have the same shape")
    batch, max_len, hid = hidden_committed.shape
    if cu_rows.numel() != batch + 1 or frontier.numel() != batch:
        raise ValueError("cu_rows/frontier do not match the tables' batch")
    cap = positions.numel()
    sh = _stream(stream, positions.device)
    if x_out is None:
        with _on_stream(sh, positions.device):
            x_out = torch.empty((cap, hid), dtype=torch.bfloat16, device=positions.device)
    _need(x_out, "x_out", torch.bfloat16, 2)
    if x_out.shape[1] != hid or x_out.shape[0] < cap:
        raise ValueError(f"x_out must be [>= {cap}, {hid}]")
    st = lib.gather_hidden(batch, cap, cu_rows.data_ptr(), positions.data_ptr(),
                           frontier.data_ptr(), hidden_committed.data_ptr(),
                           hidden_masked.data_ptr(), max_len, hid, x_out.data_ptr(), sh)
    _lib.check("gather_hidden", st)
    return x_out


class DecodeLoop:
    """A multi-step decoding loop of one layer whose every step runs on the
    device: decode_plan -> gather_hidden -> flash_cache_step ->
    scheduled_attention (+ mass) -> track_topb -> verify_accept.

    Step t plans from step t-1's top-B set (``tracked``) and accept lengths;
    the rows' count is chosen on the device, so the projection and attention
    launch over the row capacity batch * (W + topb) and skip the inactive tail.
    ``scan`` = (draft, mask, conf, threshold) with [steps, batch, W'] tensors
    gives each step's accept-scan inputs; without it every step commits one
    token.  Nothing synchronises the host inside ``step``."""

    def __init__(self, cache: PagedKVCache, w_qkv, hidden_committed, hidden_masked, kv_len,
                 frontier0, tracked0, window_len, rope_base, refresh_period, max_kv_len,
                 scan=None, softmax_scale=0.0):
        self.lib = _lib.load()
        dev = w_qkv.device
        _need(tracked0, "tracked0", torch.int32, 2)
        self.cache, self.w = cache, w_qkv
        self.hc, self.hm = hidden_committed, hidden_masked
        self.kv_len = kv_len
        self.batch = kv_len.numel()
        self.window = int(window_len)
        self.topb = tracked0.shape[1]
        self.refresh_period = int(refresh_period)
        self.cap = self.batch * (self.window + self.topb)
        h, d = cache.num_heads, cache.head_dim
        hid = hidden_committed.shape[2]
        self.frontier = frontier0.clone()
        self.tracked = tracked0.clone()
        self.accept = torch.zeros((self.batch,), dtype=torch.int32, device=dev)
        self.cu_rows = torch.empty((self.batch + 1,), dtype=torch.int32, device=dev)
        self.positions = torch.empty((self.cap,), dtype=torch.int32, device=dev)
        self.slots = torch.empty((self.cap,), dtype=torch.int32, device=dev)
        self.stage = torch.empty((self.batch,), dtype=torch.int32, device=dev)
        self.x = torch.empty((self.cap, hid), dtype=torch.bfloat16, device=dev)
        self.q = torch.empty((self.cap, h, d), dtype=torch.bfloat16, device=dev)
        self.slot_mapping = torch.empty((self.cap,), dtype=torch.int64, device=dev)
        self.out = torch.empty((self.cap, h, d), dtype=torch.float32, device=dev)
        self.max_kv_len = int(max_kv_len)
        self.mass = torch.empty((self.batch, self.max_kv_len), dtype=torch.float32, device=dev)
        need = attention_workspace_bytes(self.batch, self.cap, h, d, self.max_kv_len,
                                         self.window + self.topb, self.max_kv_len)
        self.workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
        fneed = flash_cache_workspace_bytes(self.cap, hid, h, d)
        self.fc_workspace = torch.empty((max(fneed, 1),), dtype=torch.uint8, device=dev)
        self.cs = cache.struct()
        self._plan = (self.batch, kv_len.data_ptr(), self.window, cache.block_size,
                      self.refresh_period)
        self._plan_tail = (self.tracked.data_ptr(), self.topb, self.accept.data_ptr(),
                           self.frontier.data_ptr(), self.cu_rows.data_ptr(),
                           self.positions.data_ptr(), self.slots.data_ptr(),
                           self.stage.data_ptr(), self.cap)
        self._gather = (self.batch, self.cap, self.cu_rows.data_ptr(), self.positions.data_ptr(),
                        self.frontier.data_ptr(), hidden_committed.data_ptr(),
                        hidden_masked.data_ptr(), hidden_committed.shape[1], hid,
                        self.x.data_ptr())
        self._fcs = (ctypes.byref(self.cs), self.x.data_ptr(), hid, w_qkv.data_ptr(), self.batch,
                     self.cap, self.cu_rows.data_ptr(), self.positions.data_ptr(),
                     self.slots.data_ptr(), float(rope_base), self.q.data_ptr(),
                     self.slot_mapping.data_ptr(), self.fc_workspace.data_ptr(), fneed)
        self._att = (ctypes.byref(self.cs), self.q.data_ptr(), self.batch, self.cap,
                     self.cu_rows.data_ptr(), kv_len.data_ptr(), self.max_kv_len,
                     self.window + self.topb, None, float(softmax_scale), self.out.data_ptr(),
                     self.mass.data_ptr(), self.max_kv_len, self.workspace.data_ptr(),
                     self.workspace.numel())
        self._top = (self.mass.data_ptr(), self.max_kv_len, kv_len.data_ptr(), self.batch,
                     self.topb, self.tracked.data_ptr())
        self.scan = None
        if scan is not None:
            dr, mk, cf, thr = scan
            _need(dr, "draft", torch.int32, 3)
            _need(mk, "mask", torch.int32, 3)
            _need(cf, "conf", torch.float32, 3)
            if dr.shape != mk.shape or dr.shape != cf.shape or dr.shape[1] != self.batch:
                raise ValueError("scan tensors must be [steps, batch, W] alike")
            self.scan = (dr, mk, cf, float(thr))

    def run_plan(self, t: int, stream: int):
        _lib.check("decode_plan", self.lib.decode_plan(*self._plan, int(t), *self._plan_tail,
                                                       stream))

    def run_gather(self, stream: int):
        _lib.check("gather_hidden", self.lib.gather_hidden(*self._gather, stream))

    def run_flash_cache(self, stream: int):
        _lib.check("flash_cache_step", self.lib.flash_cache_step(*self._fcs, stream))

    def run_attention(self, stream: int):
        _lib.check("scheduled_attention", self.lib.scheduled_attention(*self._att, stream))

    def run_topb(self, stream: int):
        if self.topb:
            _lib.check("track_topb", self.lib.track_topb(*self._top, stream))

    def run_verify(self, t: int, stream: int):
        if self.scan is None:
            return
        dr, mk, cf, thr = self.scan
        if t >= dr.shape[0]:
            raise ValueError(f"no scan inputs for step {t}")
        _lib.check("verify_accept", self.lib.verify_accept(
            dr[t].data_ptr(), mk[t].data_ptr(), cf[t].data_ptr(), self.batch, dr.shape[2],
            ctypes.c_float(thr), self.accept.data_ptr(), stream))

    def step(self, t: int, stream=None):
        s = _stream(stream, self.w.device) if not isinstance(stream, int) else stream
        self.run_plan(t, s)
        self.run_gather(s)
        self.run_flash_cache(s)
        self.run_attention(s)
        self.run_topb(s)
        self.run_verify(t, s)


def lm_head_workspace_bytes(rows, vocab) -> int:
    return int(_lib.load().fdl_lm_head_workspace_bytes(int(rows), int(vocab)))


def lm_head_confidence(hidden_states, w_lm, token_out=None, conf_out=None, workspace=None,
                       stream=None):
    """Per row of ``hidden_states`` (bf16 [rows, hidden]) the argmax token of
    the logits h . w_lm^T (w_lm bf16 [vocab, hidden]; equal logits go to the
    lower id) and its softmax probability.  Returns (token int32 [rows],
    conf fp32 [rows])."""
    lib = _lib.load()
    _need(hidden_states, "hidden_states", torch.bfloat16, 2)
    _need(w_lm, "w_lm", torch.bfloat16, 2)
    rows, hid = hidden_states.shape
    vocab = w_lm.shape[0]
    if w_lm.shape[1] != hid:
        raise ValueError(f"w_lm must be [vocab, {hid}], got {tuple(w_lm.shape)}")
    dev = hidden_states.device
    sh = _stream(stream, dev)
    with _on_stream(sh, dev):
        if token_out is None:
            token_out = torch.empty((rows,), dtype=torch.int32, device=dev)
        if conf_out is None:
            conf_out = torch.empty((rows,), dtype=torch.float32, device=dev)
    _need(token_out, "token_out", torch.int32, 1)
    _need(conf_out, "conf_out", torch.float32, 1)
    if token_out.numel() < rows or conf_out.numel() < rows:
        raise ValueError("token_out/conf_out need one entry per row")
    need = lm_head_workspace_bytes(rows, vocab)
    if workspace is None or workspace.numel() < need:
        with _on_stream(sh, dev):
            workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    st = lib.lm_head_confidence(hidden_states.data_ptr(), w_lm.data_ptr(), rows, vocab, hid,
                                token_out.data_ptr(), conf_out.data_ptr(),
                                workspace.data_ptr(), workspace.numel(), sh)
    _lib.check("lm_head_confidence", st)
    return token_out, conf_out


def fused_step_workspace_bytes(batch, num_rows, num_heads, head_dim, max_kv_len, max_rows_per_seq,
                               mass_stride) -> int:
    return int(_lib.load().fdl_fused_step_workspace_bytes(batch, num_rows, num_heads, head_dim,
                                                          max_kv_len, max_rows_per_seq,
                                                          mass_stride))


_FUSED_WS = {}


def _fused_workspace(device, stream_handle: int, nbytes: int):
    """Zero-filled workspace per (device, stream), allocated and filled in the
    stream's order (so the fill is done before the call's kernel starts): its
    first FUSED_SYNC_BYTES bytes are the single-launch step's counters, which
    every call leaves at zero."""
    key = (device.index if device.index is not None else torch.cuda.current_device(), stream_handle)
    ws = _FUSED_WS.get(key)
    if ws is None or ws.numel() < nbytes:
        with _on_stream(stream_handle, device):
            ws = torch.zeros((max(nbytes, 256),), dtype=torch.uint8, device=device)
        _FUSED_WS[key] = ws
    return ws


FUSED_ERROR_OFFSET = 12  # byte offset of the single-launch step's error word
FUSED_SYNC_BYTES = 4096  # the one-call steps' leading counter bytes (attention workspace after)


def fused_step_error(workspace: torch.Tensor, stream=None) -> int:
    """The single-launch step's error word (1 if a phase wait timed out; the
    results of that call are then invalid).  Synchronises the stream."""
    sh = _stream(stream, workspace.device)
    with _on_stream(sh, workspace.device):
        word = workspace[FUSED_ERROR_OFFSET:FUSED_ERROR_OFFSET + 4].view(torch.int32).item()
    return int(word)


def _one_call_step(single_launch, cache, x, w_qkv, cu_rows, positions, slots, rope_base, kv_len,
                   max_kv_len, max_rows_per_seq, views, softmax_scale, mass_stride, q_out,
                   slot_mapping_out, out, mass, workspace, stream, check):
    lib = _lib.load()
    _need(x, "x", torch.bfloat16, 2)
    _need(w_qkv, "w_qkv", torch.bfloat16, 2)
    for t, n in ((cu_rows, "cu_rows"), (positions, "positions"), (slots, "slots"),
                 (kv_len, "kv_len")):
        _need(t, n, torch.int32, 1)
    r, hid = x.shape
    h, d = cache.num_heads, cache.head_dim
    batch = kv_len.numel()
    if cu_rows.numel() != batch + 1:
        raise ValueError("cu_rows must have batch + 1 entries")
    if tuple(w_qkv.shape) != (3 * h * d, hid):
        raise ValueError(f"w_qkv must be [{3 * h * d}, {hid}], got {tuple(w_qkv.shape)}")
    if positions.numel() != r or slots.numel() != r:
        raise ValueError("positions/slots must have one entry per row")
    if views is not None:
        _need(views, "views", torch.int32, 2)
    dev = x.device
    sh = _stream(stream, dev)
    if mass_stride is None:
        mass_stride = mass.shape[1] if mass is not None else int(max_kv_len)
    with _on_stream(sh, dev):
        if q_out is None:
            q_out = torch.empty((r, h, d), dtype=torch.bfloat16, device=dev)
        if slot_mapping_out is None:
            slot_mapping_out = torch.empty((r,), dtype=torch.int64, device=dev)
        if out is None:
            out = torch.empty((r, h, d), dtype=torch.float32, device=dev)
        if mass is None:
            mass = torch.empty((batch, int(mass_stride)), dtype=torch.float32, device=dev)
    _need(q_out, "q_out", torch.bfloat16, 3)
    _need(slot_mapping_out, "slot_mapping_out", torch.int64, 1)
    _need(out, "out", torch.float32, 3)
    _need(mass, "mass", torch.float32, 2)
    need = fused_step_workspace_bytes(batch, r, h, d, int(max_kv_len), int(max_rows_per_seq),
                                      int(mass_stride))
    if workspace is None:
        workspace = _fused_workspace(dev, sh, need)
    cs = cache.struct()
    fn = lib.flash_cache_attention_step_single_launch if single_launch else \
        lib.flash_cache_attention_step
    name = "flash_cache_attention_step_single_launch" if single_launch else \
        "flash_cache_attention_step"
    st = fn(ctypes.byref(cs), x.data_ptr(), hid, w_qkv.data_ptr(), batch, r, cu_rows.data_ptr(),
            positions.data_ptr(), slots.data_ptr(), float(rope_base), q_out.data_ptr(),
            slot_mapping_out.data_ptr(), kv_len.data_ptr(), int(max_kv_len),
            int(max_rows_per_seq), _ptr(views), float(softmax_scale), out.data_ptr(),
            mass.data_ptr(), int(mass_stride), workspace.data_ptr(), workspace.numel(), sh)
    _lib.check(name, st)
    if single_launch and check and fused_step_error(workspace, sh):
        raise RuntimeError(f"{name}: a phase wait timed out (results invalid)")
    return q_out, slot_mapping_out, out, mass


def flash_cache_attention_step(cache: PagedKVCache, x, w_qkv, cu_rows, positions, slots,
                               rope_base, kv_len, max_kv_len, max_rows_per_seq, views=None,
                               softmax_scale=0.0, mass_stride=None, q_out=None,
                               slot_mapping_out=None, out=None, mass=None, workspace=None,
                               stream=None):
    """flash_cache_step then scheduled_attention with the mass, in one call
    (their kernels back to back; bitwise the same results).  Returns (q_out,
    slot_mapping, out, mass)."""
    return _one_call_step(False, cache, x, w_qkv, cu_rows, positions, slots, rope_base, kv_len,
                          max_kv_len, max_rows_per_seq, views, softmax_scale, mass_stride, q_out,
                          slot_mapping_out, out, mass, workspace, stream, False)


def flash_cache_attention_step_single_launch(cache: PagedKVCache, x, w_qkv, cu_rows, positions,
                                             slots, rope_base, kv_len, max_kv_len,
                                             max_rows_per_seq, views=None, softmax_scale=0.0,
                                             mass_stride=None, q_out=None, slot_mapping_out=None,
                                             out=None, mass=None, workspace=None, stream=None,
                                             check=True):
    """The same step as one persistent launch, items dealt to the XCDs by
    head (row-group shapes only; the results agree with the two calls', up to
    the order of the split-K projection's fp32 sums, and every call repeats
    the last bitwise).  ``workspace``, if given, must be zero-filled
    before its first use, in the launch stream's order.  With ``check`` the
    call waits for its stream and raises if the kernel reported a timed-out
    wait.  Returns (q_out, slot_mapping, out, mass)."""
    return _one_call_step(True, cache, x, w_qkv, cu_rows, positions, slots, rope_base, kv_len,
                          max_kv_len, max_rows_per_seq, views, softmax_scale, mass_stride, q_out,
                          slot_mapping_out, out, mass, workspace, stream, check)
