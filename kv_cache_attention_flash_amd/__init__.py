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

Page key: [P4] "Flash-dLLM: I/O-Aware KV Caching and Parallel Decoding for Fast,
Memory-Efficient Diffusion LLMs" (ai4snews.wisdomeyes.cn summary), paras 1-3.
"""

from __future__ import annotations

import ctypes
import dataclasses
from typing import Optional

import torch

from . import _lib
from ._lib import FdlError, KVCacheStruct  # noqa: F401

__all__ = ["PagedKVCache", "flash_cache_step", "flash_cache_step_unfused", "scheduled_attention",
           "track_topb", "verify_accept", "attention_workspace_bytes",
           "flash_cache_workspace_bytes", "flash_cache_unfused_workspace_bytes", "DecodeStep",
           "FdlError", "load"]


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


_FC_WS = {}


def _flash_cache_workspace(device, stream_handle: int, nbytes: int):
    """Split-reduction scratch, one per (device, stream)."""
    key = (device.index if device.index is not None else torch.cuda.current_device(), stream_handle)
    ws = _FC_WS.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=device)
        _FC_WS[key] = ws
    return ws


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
    if q_out is None:
        q_out = torch.empty((r, h, d), dtype=torch.bfloat16, device=x.device)
    _need(q_out, "q_out", torch.bfloat16, 3)
    if slot_mapping_out is None:
        slot_mapping_out = torch.empty((r,), dtype=torch.int64, device=x.device)
    _need(slot_mapping_out, "slot_mapping_out", torch.int64, 1)
    cs = cache.struct()
    sh = _stream(stream, x.device)
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
    if out is None:
        out = torch.empty((r, cache.num_heads, cache.head_dim), dtype=torch.float32,
                          device=q.device)
    _need(out, "out", torch.float32, 3)
    if want_mass or mass is not None:
        if mass_stride is None:
            mass_stride = mass.shape[1] if mass is not None else int(max_kv_len)
        if mass is None:
            mass = torch.empty((batch, mass_stride), dtype=torch.float32, device=q.device)
        _need(mass, "mass", torch.float32, 2)
    ms = int(mass_stride) if mass is not None else 0
    need = attention_workspace_bytes(batch, r, cache.num_heads, cache.head_dim, int(max_kv_len),
                                     int(max_rows_per_seq), ms)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=q.device)
    cs = cache.struct()
    st = lib.scheduled_attention(ctypes.byref(cs), q.data_ptr(), batch, r, cu_rows.data_ptr(),
                                 kv_len.data_ptr(), int(max_kv_len), int(max_rows_per_seq),
                                 _ptr(views), float(softmax_scale), out.data_ptr(),
                                 _ptr(mass), ms, workspace.data_ptr(), workspace.numel(),
                                 _stream(stream, q.device))
    _lib.check("scheduled_attention", st)
    return out, mass


def track_topb(mass, kv_len, topb, out=None, stream=None):
    """Top-``topb`` most-attended keys per sequence, ascending indices, -1 padded."""
    lib = _lib.load()
    _need(mass, "mass", torch.float32, 2)
    _need(kv_len, "kv_len", torch.int32, 1)
    batch = mass.shape[0]
    if kv_len.numel() != batch:
        raise ValueError("kv_len must have one entry per sequence")
    if out is None:
        out = torch.empty((batch, int(topb)), dtype=torch.int32, device=mass.device)
    _need(out, "out", torch.int32, 2)
    st = lib.track_topb(mass.data_ptr(), mass.shape[1], kv_len.data_ptr(), batch, int(topb),
                        out.data_ptr(), _stream(stream, mass.device))
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
    if out is None:
        out = torch.empty((batch,), dtype=torch.int32, device=draft_tok.device)
    _need(out, "out", torch.int32, 1)
    st = lib.verify_accept(draft_tok.data_ptr(), mask_tok.data_ptr(), conf.data_ptr(), batch,
                           window, ctypes.c_float(float(threshold)), out.data_ptr(),
                           _stream(stream, draft_tok.device))
    _lib.check("verify_accept", st)
    return out


class DecodeStep:
    """One per-layer decode step bound to fixed device buffers:
    flash_cache_step -> scheduled_attention (+ mass) -> track_topb, and the
    accept scan when ``verify`` inputs are given.

    The ctypes argument lists are built once, so ``run()`` only issues the three
    asynchronous library calls on the given stream (suitable for timing loops
    and HIP-graph capture)."""

    def __init__(self, cache: PagedKVCache, x, w_qkv, cu_rows, positions, slots, kv_len,
                 rope_base, max_kv_len, max_rows_per_seq, views=None, topb=0,
                 softmax_scale=0.0, verify=None, unfused=False):
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
        self.run_flash_cache(s)
        self.run_attention(s)
        self.run_topb(s)
        self.run_verify(s)
