"""kvq oracle: plain, slow CPU reference (C, fp64 attention) behind ctypes.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers. The product library never imports this
package, and this package never imports the product.

The arithmetic, the readings of the pages and the cache layout are documented in
``oracle/kvq_oracle.h``; each C function cites the passage it follows.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvq_oracle.cpp")
_LIB = os.path.join(_HERE, "libkvq_oracle.so")

# -ffp-contract=off: every fp32 operation of the contract is its own IEEE rounding.
CFLAGS = ["-std=c++17", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]


def build(src: str = _SRC, out: str = _LIB, extra: list[str] | None = None) -> str:
    """Compile the oracle with g++. Returns the path of the shared library."""
    cmd = ["g++", *CFLAGS, *(extra or []), src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


_lib = None


class _Cache(ctypes.Structure):
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


def _p(a: np.ndarray) -> ctypes.c_void_p:
    assert a.flags["C_CONTIGUOUS"]
    return ctypes.c_void_p(a.ctypes.data)


def load(path: str | None = None) -> ctypes.CDLL:
    """Load (building first if missing) the oracle library; cached per process."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


@contextlib.contextmanager
def using(path: str):
    """Temporarily route every wrapper in this module to another build of the oracle
    (the mutation tests build deliberately broken copies and check the pins fail)."""
    global _lib
    saved = _lib
    _lib = _bind(ctypes.CDLL(path))
    try:
        yield _lib
    finally:
        _lib = saved


def _bind(lib: ctypes.CDLL) -> ctypes.CDLL:
    vp, i32, i64, f32, f64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_double
    sig = {
        "orc_bf16_to_f32": (f32, [ctypes.c_uint16]),
        "orc_f32_to_f16": (ctypes.c_uint16, [f32]),
        "orc_f16_to_f32": (f32, [ctypes.c_uint16]),
        "orc_f32_to_f16_array": (None, [vp, vp, i64]),
        "orc_f16_to_f32_array": (None, [vp, vp, i64]),
        "orc_fmaf": (f32, [f32, f32, f32]),
        "orc_hadamard_sylvester": (None, [ctypes.c_int, vp]),
        "orc_fwht_unnormalized": (None, [vp, ctypes.c_int]),
        "orc_rotation_constant": (f32, [ctypes.c_int]),
        "orc_rotate": (None, [vp, ctypes.c_int, ctypes.c_int]),
        "orc_rotate_dense_f64": (None, [vp, vp, ctypes.c_int, ctypes.c_int]),
        "orc_quantize_row": (None, [vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp, vp]),
        "orc_quantize_row_hybrid": (None, [vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp, vp]),
        "orc_pack_row": (None, [vp, ctypes.c_int, ctypes.c_int, vp]),
        "orc_unpack_row": (None, [vp, ctypes.c_int, ctypes.c_int, vp]),
        "orc_plane_bytes": (i64, [ctypes.POINTER(_Cache), ctypes.c_int]),
        "orc_check_cache": (ctypes.c_int, [ctypes.POINTER(_Cache)]),
        "orc_quantize_append": (None, [ctypes.POINTER(_Cache), vp, vp, vp, i64]),
        "orc_dequantize": (None, [ctypes.POINTER(_Cache), ctypes.c_int, vp, i64, vp]),
        "orc_decode_attention": (None, [ctypes.POINTER(_Cache), vp, i32, i32, vp, i32, vp, f64, vp]),
        "orc_decode_attention_pruned": (None, [ctypes.POINTER(_Cache), vp, i32, i32, vp, i32, vp, f64, vp, vp]),
        "orc_prune_energy": (None, [ctypes.POINTER(_Cache), vp, i32, i32, vp]),
        "orc_attention_bf16": (None, [vp, vp, vp, i32, i32, i32, i32, i32, f64, vp]),
        "orc_window_slot": (ctypes.c_int, [ctypes.POINTER(_Window), ctypes.c_int]),
        "orc_window_append": (None, [ctypes.POINTER(_Cache), ctypes.POINTER(_Window), vp, vp, vp, vp, vp, i64]),
        "orc_decode_attention_window": (None, [ctypes.POINTER(_Cache), ctypes.POINTER(_Window), vp, i32, i32, vp,
                                               i32, vp, f64, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


# ----------------------------------------------------------------------------- formats

def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    load().orc_f32_to_f16_array(_p(x), _p(out), x.size)
    return out


def f16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, np.float32)
    load().orc_f16_to_f32_array(_p(h), _p(out), h.size)
    return out


def fmaf(a: float, b: float, c: float) -> float:
    return load().orc_fmaf(a, b, c)


# ----------------------------------------------------------------------------- rotation

def hadamard(n: int) -> np.ndarray:
    H = np.empty((n, n), np.int32)
    load().orc_hadamard_sylvester(n, _p(H))
    return H


def fwht_unnormalized(x: np.ndarray) -> np.ndarray:
    y = np.array(x, dtype=np.float32, copy=True, order="C")
    load().orc_fwht_unnormalized(_p(y), y.size)
    return y


def rotation_constant(n: int) -> float:
    return load().orc_rotation_constant(n)


def rotate(x: np.ndarray, block: int) -> np.ndarray:
    y = np.array(x, dtype=np.float32, copy=True, order="C")
    load().orc_rotate(_p(y), y.size, block)
    return y


def rotate_dense_f64(x: np.ndarray, block: int) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty_like(x)
    load().orc_rotate_dense_f64(_p(x), _p(y), x.size, block)
    return y


# ----------------------------------------------------------------------------- quantizer

def quantize_row(x: np.ndarray, bits: int, group: int, hybrid: bool = False):
    """One token row (already rotated if needed) -> (codes u8[d], scale f16 bits, zero f16 bits).
    hybrid: per group the symmetric or asymmetric pair with the smaller largest error."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    d = x.size
    codes = np.empty(d, np.uint8)
    sc = np.empty(d // group, np.uint16)
    ze = np.empty(d // group, np.uint16)
    fn = load().orc_quantize_row_hybrid if hybrid else load().orc_quantize_row
    fn(_p(x), d, bits, group, _p(codes), _p(sc), _p(ze))
    return codes, sc, ze


def pack_row(codes: np.ndarray, bits: int) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(codes.size * bits // 8, np.uint8)
    load().orc_pack_row(_p(codes), codes.size, bits, _p(out))
    return out


def unpack_row(packed: np.ndarray, d: int, bits: int) -> np.ndarray:
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    out = np.empty(d, np.uint8)
    load().orc_unpack_row(_p(packed), d, bits, _p(out))
    return out


# ----------------------------------------------------------------------------- cache

@dataclass
class Cache:
    """Host-memory KV cache in the layout described in kvq_oracle.h."""

    head_dim: int
    num_kv_heads: int
    bits: int
    group_size: int
    hadamard_block: int
    page_size: int
    num_pages: int
    quant_mode: int = 0  # 0 = asymmetric min/max, 1 = hybrid symmetric/asymmetric
    v_grouping: int = 0  # 0 = V groups of G channels per token, 1 = of G tokens per channel

    def __post_init__(self):
        desc = self._desc(None)
        rc = load().orc_check_cache(ctypes.byref(desc))
        if rc != 0:
            raise ValueError(f"cache description outside the oracle's domain (code {rc})")
        n = [load().orc_plane_bytes(ctypes.byref(desc), i) for i in range(4)]
        # zero-filled, like fresh device memory cleared by its owner
        self.k_codes = np.zeros(n[0], np.uint8)
        self.k_meta = np.zeros(n[1], np.uint8)
        self.v_codes = np.zeros(n[2], np.uint8)
        self.v_meta = np.zeros(n[3], np.uint8)

    def _desc(self, planes) -> _Cache:
        d = _Cache(self.head_dim, self.num_kv_heads, self.bits, self.group_size, self.hadamard_block,
                   self.page_size, self.num_pages)
        d.quant_mode = self.quant_mode
        d.v_grouping = self.v_grouping
        if planes is not None:
            d.k_codes, d.k_meta, d.v_codes, d.v_meta = [p.ctypes.data for p in planes]
        return d

    @property
    def desc(self) -> _Cache:
        return self._desc((self.k_codes, self.k_meta, self.v_codes, self.v_meta))

    def planes(self):
        return self.k_codes, self.k_meta, self.v_codes, self.v_meta

    def append(self, k_bf16: np.ndarray, v_bf16: np.ndarray, slots: np.ndarray) -> None:
        """k_bf16, v_bf16: uint16 bf16 bit patterns [n][Hkv][d]; slots int64 [n]."""
        k = np.ascontiguousarray(k_bf16, dtype=np.uint16)
        v = np.ascontiguousarray(v_bf16, dtype=np.uint16)
        s = np.ascontiguousarray(slots, dtype=np.int64)
        assert k.shape == v.shape == (s.size, self.num_kv_heads, self.head_dim)
        load().orc_quantize_append(ctypes.byref(self.desc), _p(k), _p(v), _p(s), s.size)

    def dequantize(self, which: int, slots: np.ndarray) -> np.ndarray:
        s = np.ascontiguousarray(slots, dtype=np.int64)
        out = np.empty((s.size, self.num_kv_heads, self.head_dim), np.float32)
        load().orc_dequantize(ctypes.byref(self.desc), which, _p(s), s.size, _p(out))
        return out

    def decode(self, q_bf16: np.ndarray, block_table: np.ndarray, seq_lens: np.ndarray,
               softmax_scale: float = 0.0) -> np.ndarray:
        q = np.ascontiguousarray(q_bf16, dtype=np.uint16)
        bt = np.ascontiguousarray(block_table, dtype=np.int32)
        sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
        B, Hq, d = q.shape
        assert d == self.head_dim and Hq % self.num_kv_heads == 0 and bt.shape[0] == B and sl.size == B
        out = np.empty((B, Hq, d), np.float64)
        load().orc_decode_attention(ctypes.byref(self.desc), _p(q), B, Hq, _p(bt), bt.shape[1], _p(sl),
                                    float(softmax_scale), _p(out))
        return out

    def decode_pruned(self, q_bf16: np.ndarray, block_table: np.ndarray, seq_lens: np.ndarray,
                      keep_mask: np.ndarray, softmax_scale: float = 0.0) -> np.ndarray:
        """Decode with the rotated query restricted to the kept key chunks: keep_mask int32
        [B][Hkv], bit j = channels j*W..j*W+W-1, W = 128 / bits."""
        q = np.ascontiguousarray(q_bf16, dtype=np.uint16)
        bt = np.ascontiguousarray(block_table, dtype=np.int32)
        sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
        km = np.ascontiguousarray(keep_mask, dtype=np.int32)
        B, Hq, d = q.shape
        assert km.shape == (B, self.num_kv_heads)
        out = np.empty((B, Hq, d), np.float64)
        load().orc_decode_attention_pruned(ctypes.byref(self.desc), _p(q), B, Hq, _p(bt), bt.shape[1], _p(sl),
                                           float(softmax_scale), _p(km), _p(out))
        return out

    def prune_energy(self, q_bf16: np.ndarray) -> np.ndarray:
        """fp64 [B][Hkv][n_chunks]: per key chunk, the kv head's summed squared rotated query."""
        q = np.ascontiguousarray(q_bf16, dtype=np.uint16)
        B, Hq, d = q.shape
        out = np.empty((B, self.num_kv_heads, d * self.bits // 128), np.float64)
        load().orc_prune_energy(ctypes.byref(self.desc), _p(q), B, Hq, _p(out))
        return out


# ----------------------------------------------------------------------------- windows

class _Window(ctypes.Structure):
    _fields_ = [
        ("head_dim", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("sink", ctypes.c_int32),
        ("recent", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("residual", ctypes.c_int32),
    ]


@dataclass
class Window:
    """bf16 high-precision windows (first `sink`, last `recent` tokens per sequence), or
    with residual=1 the bf16 residual of the incomplete last group of `recent` tokens."""

    head_dim: int
    num_kv_heads: int
    sink: int
    recent: int
    batch: int
    residual: int = 0

    def __post_init__(self):
        shape = (self.batch, self.sink + self.recent, self.num_kv_heads, self.head_dim)
        self.k = np.zeros(shape, np.uint16)
        self.v = np.zeros(shape, np.uint16)

    @property
    def desc(self) -> _Window:
        return _Window(self.head_dim, self.num_kv_heads, self.sink, self.recent, self.batch, self.k.ctypes.data,
                       self.v.ctypes.data, self.residual)

    def slot(self, t: int) -> int:
        return load().orc_window_slot(ctypes.byref(self.desc), t)

    def append(self, cache: Cache, k_bf16, v_bf16, seqs, positions, evict_slots) -> None:
        """One token per row: bf16 bits [n][Hkv][d]; int32 seqs, positions; int64 evict_slots."""
        k = np.ascontiguousarray(k_bf16, dtype=np.uint16)
        v = np.ascontiguousarray(v_bf16, dtype=np.uint16)
        sq = np.ascontiguousarray(seqs, dtype=np.int32)
        pos = np.ascontiguousarray(positions, dtype=np.int32)
        ev = np.ascontiguousarray(evict_slots, dtype=np.int64)
        n = sq.size
        assert k.shape == v.shape == (n, self.num_kv_heads, self.head_dim) and pos.size == n and ev.size == n
        load().orc_window_append(ctypes.byref(cache.desc), ctypes.byref(self.desc), _p(k), _p(v), _p(sq), _p(pos),
                                 _p(ev), n)

    def decode(self, cache: Cache, q_bf16, block_table, seq_lens, softmax_scale: float = 0.0) -> np.ndarray:
        q = np.ascontiguousarray(q_bf16, dtype=np.uint16)
        bt = np.ascontiguousarray(block_table, dtype=np.int32)
        sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
        B, Hq, d = q.shape
        out = np.empty((B, Hq, d), np.float64)
        load().orc_decode_attention_window(ctypes.byref(cache.desc), ctypes.byref(self.desc), _p(q), B, Hq, _p(bt),
                                           bt.shape[1], _p(sl), float(softmax_scale), _p(out))
        return out


def attention_bf16(q, k, v, num_kv_heads: int, softmax_scale: float = 0.0) -> np.ndarray:
    """fp64 attention on unquantized bf16 K/V [B][T][Hkv][d] (information only)."""
    q = np.ascontiguousarray(q, dtype=np.uint16)
    k = np.ascontiguousarray(k, dtype=np.uint16)
    v = np.ascontiguousarray(v, dtype=np.uint16)
    B, Hq, d = q.shape
    T = k.shape[1]
    out = np.empty((B, Hq, d), np.float64)
    load().orc_attention_bf16(_p(q), _p(k), _p(v), B, Hq, num_kv_heads, d, T, float(softmax_scale), _p(out))
    return out


def bits_per_element(head_dim: int, bits: int, group_size: int) -> float:
    """Stored bits per cached element, codes plus fp16 scale and zero, from the plane sizes."""
    c = Cache(head_dim, 1, bits, group_size, 0, 16, 1)
    total = sum(p.size for p in c.planes()) * 8
    return total / (2 * 16 * head_dim)
