"""kvq: rotated low-bit KV-cache quantize-append and split-K decode attention on MI355X.

A thin ctypes binding over ``libkvq.so`` (hand-written HIP kernels for gfx950 behind
the C ABI declared in ``include/kvq.h``). These functions only marshal torch tensors
into the C calls; every step of the computation runs in the library's kernels. If
the library is not built, importing works but every call raises ``KVQError``: there
is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# KVQ_LIBRARY may point at another build of the same library (e.g. for A/B timing)
LIB_PATH = os.environ.get("KVQ_LIBRARY") or os.path.join(_PKG, "libkvq.so")

OK, ERR_INVALID, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, 1, 2, 3, 4


class KVQError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status) if _lib_or_none() else status}")


class _Desc(ctypes.Structure):
    _fields_ = [
        ("head_dim", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("bits", ctypes.c_int32),
        ("group_size", ctypes.c_int32),
        ("hadamard_block", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int64),
        ("k_codes", ctypes.c_void_p),
        ("k_meta", ctypes.c_void_p),
        ("v_codes", ctypes.c_void_p),
        ("v_meta", ctypes.c_void_p),
        ("quant_mode", ctypes.c_int32),
        ("v_grouping", ctypes.c_int32),
    ]


class _Window(ctypes.Structure):
    _fields_ = [
        ("sink", ctypes.c_int32),
        ("recent", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("residual", ctypes.c_int32),
    ]


_lib = None

# name -> (restype, argtypes); every symbol include/kvq.h declares
_vp, _i32, _i64, _f32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
_DP = ctypes.POINTER(_Desc)
_WP = ctypes.POINTER(_Window)
SIGNATURES = {
    "kvq_cache_plane_bytes": (_i64, [_DP, _i32]),
    "kvq_quantize_append": (ctypes.c_int, [_DP, _vp, _vp, _vp, _i64, _vp]),
    "kvq_decode_workspace_bytes": (_sz, [_DP, _i32, _i32, _i32, _i32]),
    "kvq_decode_num_splits": (_i32, [_DP, _i32, _i32, _i32, _i32]),
    "kvq_decode_attention": (ctypes.c_int, [_DP, _vp, _i32, _i32, _vp, _i32, _vp, _i32, _f32, _i32, _vp, _sz,
                                            _vp, _vp]),
    "kvq_decode_attention_timed": (ctypes.c_int, [_DP, _vp, _i32, _i32, _vp, _i32, _vp, _i32, _f32, _i32, _vp,
                                                  _sz, _vp, _vp, _vp, _vp]),
    "kvq_decode_attention_reference": (ctypes.c_int, [_DP, _vp, _i32, _i32, _vp, _i32, _vp, _i32, _f32, _i32,
                                                      _vp, _sz, _vp, _vp]),
    "kvq_decode_step": (ctypes.c_int, [_DP, _vp, _vp, _vp, _i32, _i32, _vp, _i32, _vp, _i32, _f32, _i32, _vp, _sz,
                                       _vp, _vp]),
    "kvq_decode_step_timed": (ctypes.c_int, [_DP, _vp, _vp, _vp, _i32, _i32, _vp, _i32, _vp, _i32, _f32, _i32, _vp,
                                             _sz, _vp, _vp, _vp, _vp]),
    "kvq_window_plane_bytes": (_i64, [_DP, _WP]),
    "kvq_window_append": (ctypes.c_int, [_DP, _WP, _vp, _vp, _vp, _vp, _vp, _i64, _vp]),
    "kvq_decode_window_workspace_bytes": (_sz, [_DP, _WP, _i32, _i32, _i32, _i32]),
    "kvq_decode_attention_window": (ctypes.c_int, [_DP, _WP, _vp, _i32, _i32, _vp, _i32, _vp, _i32, _f32, _i32,
                                                   _vp, _sz, _vp, _vp]),
    "kvq_decode_attention_window_timed": (ctypes.c_int, [_DP, _WP, _vp, _i32, _i32, _vp, _i32, _vp, _i32, _f32,
                                                         _i32, _vp, _sz, _vp, _vp, _vp, _vp]),
    "kvq_decode_attention_noalloc": (ctypes.c_int, [_DP, _vp, _i32, _i32, _vp, _i32, _vp, _i32, _f32, _i32, _vp,
                                                    _vp]),
    "kvq_decode_attention_pruned": (ctypes.c_int, [_DP, _vp, _i32, _i32, _vp, _i32, _vp, _i32, _f32, _i32, _i32,
                                                   _vp, _vp, _sz, _vp, _vp, _vp, _vp]),
    "kvq_dequantize": (ctypes.c_int, [_DP, _i32, _vp, _i64, _vp, _vp]),
    "kvq_stream_read": (ctypes.c_int, [_vp, _sz, _vp, _i32, _i32, _vp, _vp, _vp]),
    "kvq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "kvq_version": (ctypes.c_char_p, []),
}


def _lib_or_none():
    return _lib


def lib() -> ctypes.CDLL:
    """The loaded libkvq.so; raises KVQError if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise KVQError(ERR_HIP, f"{LIB_PATH} is not built (run __graft_entry__.build())")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


def status_string(status: int) -> str:
    return lib().kvq_status_string(status).decode()


def version() -> str:
    return lib().kvq_version().decode()


def _check(status: int, what: str) -> None:
    if status != OK:
        raise KVQError(status, what)


def _ptr(t: torch.Tensor | None) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr() if t is not None else None)


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t: torch.Tensor, dtype: torch.dtype, name: str) -> None:
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


@dataclass
class KVCache:
    """A quantized KV cache: four caller-owned device planes plus the description.

    Layout (see include/kvq.h): 16-token tiles; K codes chunk-major per tile, K meta
    token-major, V codes word-major per tile with token pairs byte-interleaved, V meta
    in two 4-token parts per group and half-tile; fp16 {scale, zero} pairs.
    """

    head_dim: int
    num_kv_heads: int
    bits: int
    group_size: int
    hadamard_block: int
    page_size: int
    num_pages: int
    k_codes: torch.Tensor
    k_meta: torch.Tensor
    v_codes: torch.Tensor
    v_meta: torch.Tensor
    quant_mode: int = 0  # 0 = asymmetric min/max groups, 1 = hybrid symmetric/asymmetric
    v_grouping: int = 0  # 0 = value groups of G channels per token, 1 = of G tokens per channel

    @staticmethod
    def plane_bytes(head_dim, num_kv_heads, bits, group_size, hadamard_block, page_size, num_pages) -> list[int]:
        d = _Desc(head_dim, num_kv_heads, bits, group_size, hadamard_block, page_size, num_pages)
        sizes = [lib().kvq_cache_plane_bytes(ctypes.byref(d), i) for i in range(4)]
        if min(sizes) < 0:
            raise KVQError(ERR_INVALID, "cache description")
        return sizes

    @classmethod
    def allocate(cls, head_dim: int, num_kv_heads: int, bits: int, group_size: int, hadamard_block: int,
                 page_size: int, num_pages: int, device="cuda", quant_mode: int = 0,
                 v_grouping: int = 0) -> "KVCache":
        sizes = cls.plane_bytes(head_dim, num_kv_heads, bits, group_size, hadamard_block, page_size, num_pages)
        planes = [torch.zeros(n, dtype=torch.uint8, device=device) for n in sizes]
        return cls(head_dim, num_kv_heads, bits, group_size, hadamard_block, page_size, num_pages, *planes,
                   quant_mode=quant_mode, v_grouping=v_grouping)

    def clone(self) -> "KVCache":
        return KVCache(self.head_dim, self.num_kv_heads, self.bits, self.group_size, self.hadamard_block,
                       self.page_size, self.num_pages, *[p.clone() for p in self.planes()],
                       quant_mode=self.quant_mode, v_grouping=self.v_grouping)

    @property
    def desc(self) -> _Desc:
        return _Desc(self.head_dim, self.num_kv_heads, self.bits, self.group_size, self.hadamard_block,
                     self.page_size, self.num_pages, self.k_codes.data_ptr(), self.k_meta.data_ptr(),
                     self.v_codes.data_ptr(), self.v_meta.data_ptr(), self.quant_mode, self.v_grouping)

    def planes(self):
        return self.k_codes, self.k_meta, self.v_codes, self.v_meta

    @property
    def nbytes(self) -> int:
        return sum(p.numel() for p in self.planes())


def quantize_append(cache: KVCache, k_new: torch.Tensor, v_new: torch.Tensor, slots: torch.Tensor,
                    stream=None) -> None:
    """Rotate (K) and quantize K and V rows [n][Hkv][d] (bf16) into the cache at `slots` (int64)."""
    _need(k_new, torch.bfloat16, "k_new")
    _need(v_new, torch.bfloat16, "v_new")
    _need(slots, torch.int64, "slots")
    n = slots.numel()
    if k_new.shape != (n, cache.num_kv_heads, cache.head_dim) or v_new.shape != k_new.shape:
        raise ValueError(f"k_new/v_new must be [{n}][{cache.num_kv_heads}][{cache.head_dim}]")
    st = lib().kvq_quantize_append(ctypes.byref(cache.desc), _ptr(k_new), _ptr(v_new), _ptr(slots), n,
                                   _stream(stream))
    _check(st, "kvq_quantize_append")


def decode_workspace_bytes(cache: KVCache, batch: int, num_q_heads: int, max_seq_len: int,
                           num_splits: int = 0) -> int:
    return lib().kvq_decode_workspace_bytes(ctypes.byref(cache.desc), batch, num_q_heads, max_seq_len, num_splits)


def decode_num_splits(cache: KVCache, batch: int, num_q_heads: int, max_seq_len: int, num_splits: int = 0) -> int:
    return lib().kvq_decode_num_splits(ctypes.byref(cache.desc), batch, num_q_heads, max_seq_len, num_splits)


def decode_attention(cache: KVCache, q: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor,
                     max_seq_len: int, softmax_scale: float = 0.0, num_splits: int = 0,
                     workspace: torch.Tensor | None = None, out: torch.Tensor | None = None, stream=None,
                     events=None, reference: bool = False) -> torch.Tensor:
    """Split-K GQA decode attention; q bf16 [B][Hq][d] (original basis) -> fp32 [B][Hq][d].

    `num_splits` 0 lets the library choose: for 2..256 sequences one partition length
    for the whole batch, planned on the device from `seq_lens` (see include/kvq.h);
    otherwise a fixed number of partitions per max_seq_len sequence.
    `events` = (begin, end) raw hipEvent_t handles (ints) recorded around the split-K kernel.
    `reference` routes to the plain-VALU kernel (for cross-checks).
    """
    _need(q, torch.bfloat16, "q")
    _need(block_table, torch.int32, "block_table")
    _need(seq_lens, torch.int32, "seq_lens")
    B, Hq, d = q.shape
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    _need(out, torch.float32, "out")
    need = decode_workspace_bytes(cache, B, Hq, max_seq_len, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _need(workspace, torch.uint8, "workspace")
    args = [ctypes.byref(cache.desc), _ptr(q), B, Hq, _ptr(block_table), block_table.shape[1], _ptr(seq_lens),
            max_seq_len, softmax_scale, num_splits, _ptr(workspace), workspace.numel(), _ptr(out), _stream(stream)]
    if reference:
        st = lib().kvq_decode_attention_reference(*args)
    elif events is not None:
        st = lib().kvq_decode_attention_timed(*args, ctypes.c_void_p(events[0]), ctypes.c_void_p(events[1]))
    else:
        st = lib().kvq_decode_attention(*args)
    _check(st, "kvq_decode_attention")
    return out


def decode_step(cache: KVCache, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor,
                block_table: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int, softmax_scale: float = 0.0,
                num_splits: int = 0, workspace: torch.Tensor | None = None, out: torch.Tensor | None = None,
                stream=None, events=None) -> torch.Tensor:
    """One decode step with the append fused into the split-K kernel (kvq_decode_step):
    k_new/v_new bf16 [B][Hkv][d] are each sequence's new token, written at position
    seq_lens[b] - 1, then the decode of q over seq_lens[b] tokens. The same cache bytes and
    output as quantize_append at those slots followed by decode_attention."""
    _need(k_new, torch.bfloat16, "k_new")
    _need(v_new, torch.bfloat16, "v_new")
    _need(q, torch.bfloat16, "q")
    _need(block_table, torch.int32, "block_table")
    _need(seq_lens, torch.int32, "seq_lens")
    B, Hq, d = q.shape
    if k_new.shape != (B, cache.num_kv_heads, cache.head_dim) or v_new.shape != k_new.shape:
        raise ValueError(f"k_new/v_new must be [{B}][{cache.num_kv_heads}][{cache.head_dim}]")
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    _need(out, torch.float32, "out")
    need = decode_workspace_bytes(cache, B, Hq, max_seq_len, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _need(workspace, torch.uint8, "workspace")
    args = [ctypes.byref(cache.desc), _ptr(k_new), _ptr(v_new), _ptr(q), B, Hq, _ptr(block_table),
            block_table.shape[1], _ptr(seq_lens), max_seq_len, softmax_scale, num_splits, _ptr(workspace),
            workspace.numel(), _ptr(out), _stream(stream)]
    if events is not None:
        st = lib().kvq_decode_step_timed(*args, ctypes.c_void_p(events[0]), ctypes.c_void_p(events[1]))
    else:
        st = lib().kvq_decode_step(*args)
    _check(st, "kvq_decode_step")
    return out


NOALLOC_WORKSPACE_BYTES = 32 << 20  # KVQ_NOALLOC_WORKSPACE_BYTES


def decode_attention_noalloc(cache: KVCache, q: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor,
                             max_seq_len: int, out: torch.Tensor, softmax_scale: float = 0.0, num_splits: int = 0,
                             stream=None) -> torch.Tensor:
    """decode_attention with the library's own device workspace (kvq_decode_attention_noalloc):
    the C call allocates nothing, so `out` (fp32 [B][Hq][d]) is the caller's. Calls that
    overlap on one GPU share that workspace and race."""
    _need(q, torch.bfloat16, "q")
    _need(block_table, torch.int32, "block_table")
    _need(seq_lens, torch.int32, "seq_lens")
    _need(out, torch.float32, "out")
    B, Hq, d = q.shape
    st = lib().kvq_decode_attention_noalloc(ctypes.byref(cache.desc), _ptr(q), B, Hq, _ptr(block_table),
                                            block_table.shape[1], _ptr(seq_lens), max_seq_len, softmax_scale,
                                            num_splits, _ptr(out), _stream(stream))
    _check(st, "kvq_decode_attention_noalloc")
    return out


def decode_attention_pruned(cache: KVCache, q: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor,
                            max_seq_len: int, keep_chunks: int, softmax_scale: float = 0.0, num_splits: int = 0,
                            chunk_mask: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                            out: torch.Tensor | None = None, stream=None, events=None) -> torch.Tensor:
    """Decode with query-channel pruning: per (sequence, kv head) only the keep_chunks
    16-byte key chunks (128/bits channels each) with the largest rotated-query energy are
    read and scored. chunk_mask (int32 [B][Hkv], optional) receives the kept chunks."""
    _need(q, torch.bfloat16, "q")
    _need(block_table, torch.int32, "block_table")
    _need(seq_lens, torch.int32, "seq_lens")
    B, Hq, d = q.shape
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    _need(out, torch.float32, "out")
    if chunk_mask is not None:
        _need(chunk_mask, torch.int32, "chunk_mask")
        if chunk_mask.shape != (B, cache.num_kv_heads):
            raise ValueError(f"chunk_mask must be [{B}][{cache.num_kv_heads}]")
    need = decode_workspace_bytes(cache, B, Hq, max_seq_len, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _need(workspace, torch.uint8, "workspace")
    ev = events if events is not None else (None, None)
    st = lib().kvq_decode_attention_pruned(ctypes.byref(cache.desc), _ptr(q), B, Hq, _ptr(block_table),
                                           block_table.shape[1], _ptr(seq_lens), max_seq_len, softmax_scale,
                                           num_splits, keep_chunks, _ptr(chunk_mask), _ptr(workspace),
                                           workspace.numel(), _ptr(out), _stream(stream), ctypes.c_void_p(ev[0]),
                                           ctypes.c_void_p(ev[1]))
    _check(st, "kvq_decode_attention_pruned")
    return out


def dequantize(cache: KVCache, which: int, slots: torch.Tensor, out: torch.Tensor | None = None,
               stream=None) -> torch.Tensor:
    """fp32 [n][Hkv][d] = fma(code, scale, zero) of the K (which=0, rotated basis) or V rows at `slots`."""
    _need(slots, torch.int64, "slots")
    n = slots.numel()
    if out is None:
        out = torch.empty((n, cache.num_kv_heads, cache.head_dim), dtype=torch.float32, device=slots.device)
    _need(out, torch.float32, "out")
    st = lib().kvq_dequantize(ctypes.byref(cache.desc), which, _ptr(slots), n, _ptr(out), _stream(stream))
    _check(st, "kvq_dequantize")
    return out


@dataclass
class KVWindow:
    """High-precision windows: the first `sink` and last `recent` tokens of every sequence
    in bf16 [batch][sink + recent][Hkv][d] (keys unrotated); token t in row t (t < sink) or
    sink + (t - sink) % recent. Caller-owned device planes (see include/kvq.h)."""

    sink: int
    recent: int
    batch: int
    k: torch.Tensor
    v: torch.Tensor
    residual: int = 0  # 1: sink 0, the ring holds the incomplete last group of `recent` tokens

    @classmethod
    def allocate(cls, cache: KVCache, sink: int, recent: int, batch: int, device="cuda",
                 residual: int = 0) -> "KVWindow":
        w = _Window(sink, recent, batch, None, None, residual)
        n = lib().kvq_window_plane_bytes(ctypes.byref(cache.desc), ctypes.byref(w))
        if n < 0:
            raise KVQError(ERR_INVALID, "window description")
        shape = (batch, sink + recent, cache.num_kv_heads, cache.head_dim)
        k = torch.zeros(shape, dtype=torch.bfloat16, device=device)
        v = torch.zeros(shape, dtype=torch.bfloat16, device=device)
        assert k.numel() * 2 == n
        return cls(sink, recent, batch, k, v, residual)

    @property
    def desc(self) -> _Window:
        return _Window(self.sink, self.recent, self.batch, self.k.data_ptr(), self.v.data_ptr(), self.residual)

    def row(self, t: int) -> int:
        return t if t < self.sink else self.sink + (t - self.sink) % self.recent


def window_append(cache: KVCache, window: KVWindow, k_new: torch.Tensor, v_new: torch.Tensor, seqs: torch.Tensor,
                  positions: torch.Tensor, evict_slots: torch.Tensor, stream=None) -> None:
    """One new token per listed sequence through the windows; a token leaving the recent
    window is rotated and quantized into the cache at its evict slot (int64)."""
    _need(k_new, torch.bfloat16, "k_new")
    _need(v_new, torch.bfloat16, "v_new")
    _need(seqs, torch.int32, "seqs")
    _need(positions, torch.int32, "positions")
    _need(evict_slots, torch.int64, "evict_slots")
    n = seqs.numel()
    if positions.numel() != n or evict_slots.numel() != n:
        raise ValueError("seqs, positions and evict_slots must have one entry per new token")
    if k_new.shape != (n, cache.num_kv_heads, cache.head_dim) or v_new.shape != k_new.shape:
        raise ValueError(f"k_new/v_new must be [{n}][{cache.num_kv_heads}][{cache.head_dim}]")
    st = lib().kvq_window_append(ctypes.byref(cache.desc), ctypes.byref(window.desc), _ptr(k_new), _ptr(v_new),
                                 _ptr(seqs), _ptr(positions), _ptr(evict_slots), n, _stream(stream))
    _check(st, "kvq_window_append")


def decode_window_workspace_bytes(cache: KVCache, window: KVWindow, batch: int, num_q_heads: int,
                                  max_seq_len: int, num_splits: int = 0) -> int:
    return lib().kvq_decode_window_workspace_bytes(ctypes.byref(cache.desc), ctypes.byref(window.desc), batch,
                                                   num_q_heads, max_seq_len, num_splits)


def decode_attention_window(cache: KVCache, window: KVWindow, q: torch.Tensor, block_table: torch.Tensor,
                            seq_lens: torch.Tensor, max_seq_len: int, softmax_scale: float = 0.0,
                            num_splits: int = 0, workspace: torch.Tensor | None = None,
                            out: torch.Tensor | None = None, stream=None, events=None) -> torch.Tensor:
    """Decode attention over windows (bf16, original query) and cache (rotated query) in one
    softmax; q bf16 [B][Hq][d] -> fp32 [B][Hq][d]; seq_lens count all tokens. events: an
    optional (begin, end) pair of hipEvent_t handles recorded around the split-K kernel."""
    _need(q, torch.bfloat16, "q")
    _need(block_table, torch.int32, "block_table")
    _need(seq_lens, torch.int32, "seq_lens")
    B, Hq, d = q.shape
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    _need(out, torch.float32, "out")
    need = decode_window_workspace_bytes(cache, window, B, Hq, max_seq_len, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _need(workspace, torch.uint8, "workspace")
    args = (ctypes.byref(cache.desc), ctypes.byref(window.desc), _ptr(q), B, Hq, _ptr(block_table),
            block_table.shape[1], _ptr(seq_lens), max_seq_len, softmax_scale, num_splits, _ptr(workspace),
            workspace.numel(), _ptr(out), _stream(stream))
    if events is None:
        st = lib().kvq_decode_attention_window(*args)
    else:
        st = lib().kvq_decode_attention_window_timed(*args, ctypes.c_void_p(events[0]), ctypes.c_void_p(events[1]))
    _check(st, "kvq_decode_attention_window")
    return out


def stream_read(buf: torch.Tensor, nontemporal: bool = True, workgroups_per_cu: int = 8,
                sink: torch.Tensor | None = None, stream=None, events=None) -> None:
    """Read-bandwidth probe: read every byte of `buf` (a contiguous device tensor whose
    size is a multiple of 16 bytes) once with the decode kernel's 16-byte load shape.
    `events` = (begin, end) raw hipEvent_t handles recorded around the launch."""
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=buf.device)
    ev = events if events is not None else (None, None)
    st = lib().kvq_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), int(nontemporal),
                               workgroups_per_cu, _stream(stream), ctypes.c_void_p(ev[0]), ctypes.c_void_p(ev[1]))
    _check(st, "kvq_stream_read")
