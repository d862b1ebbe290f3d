"""Pins of the oracle: checks against facts fixed outside the oracle itself.

Each ``check_*`` function raises AssertionError on failure. They run against the real
oracle (tests/test_oracle_pins.py) and against deliberately broken copies of it
(tests/test_oracle_mutants.py), which must each fail at least one check.

What pins what (the pages print no worked example, so the pins are mathematics,
IEEE definitions, library routines and hand derivations):
  Hadamard           scipy.linalg.hadamard (Sylvester construction); H H^T = n I;
                     butterfly == dense product exactly on small integers; involution.
  rotation constant  nearest-float property of 1/sqrt(n), checked with exact rationals.
  one-hot key        a single outlier channel spreads to +-A/sqrt(n) in every channel.
  q.k invariance     (Rq).(Rk) == q.k (Dual-QK, Abstract: paired transform preserves q.k).
  fp16 conversion    x86 F16C instruction (exhaustive over the finite range) and numpy.
  fmaf               exact rational arithmetic rounded to nearest-even binary32.
  quantizer          hand-derived worked examples (tests/golden); code range; round-trip
                     bound |x - xhat| <= scale/2 (+ zero rounding + ulps).
  hybrid quantizer   hand-derived worked examples (tests/golden/hybrid_worked_examples.json);
                     per group the asymmetric pair or an independently computed symmetric
                     candidate, never a larger largest error; a hybrid cache stores them.
  packing            documented nibble/crumb order; the documented cache byte layout.
  storage            bits per element = b + 32/G (2.25 at INT2 g128, as the QuaRot page's
                     "BPE ~2.25" for INT2 group 128).
  attention          torch scaled_dot_product_attention in fp64 on the oracle's own
                     dequantized K/V with a scipy-rotated query; T=1 gives v0; q=0 or
                     identical keys give the mean of V; page-permutation invariance.
"""
from __future__ import annotations

import ctypes
import json
import os
import subprocess
from fractions import Fraction

import numpy as np
import scipy.linalg
import torch

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden", "quantizer_worked_examples.json")


# ----------------------------------------------------------------------------- helpers

def nearest_f32(fr: Fraction) -> np.float32:
    """Round an exact rational to the nearest binary32, ties to even (normal range)."""
    f = np.float32(float(fr))  # candidate; may be off by one ulp through double rounding
    best = None
    for cand in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        err = abs(Fraction(float(cand)) - fr)
        key = (err, int(np.array(cand, np.float32).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, cand)
    return best[1]


def _f16c_lib():
    src = os.path.join(HERE, "native", "f16_check.c")
    out = os.path.join(HERE, "native", "libf16_check.so")
    if not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src):
        subprocess.run(["gcc", "-O2", "-mf16c", "-fPIC", "-shared", src, "-o", out], check=True)
    lib = ctypes.CDLL(out)
    lib.f16_check_range.restype = ctypes.c_int64
    lib.f16_check_range.argtypes = [ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint32,
                                    ctypes.POINTER(ctypes.c_uint32)]
    return lib


# ----------------------------------------------------------------------------- Hadamard

def check_hadamard_is_sylvester():
    for n in (2, 4, 8, 16, 32, 64, 128, 256):
        H = oracle.hadamard(n)
        assert np.array_equal(H, scipy.linalg.hadamard(n)), n


def check_hadamard_orthogonal():
    for n in (2, 4, 8, 16, 32, 64, 128, 256):
        H = oracle.hadamard(n).astype(np.int64)
        assert np.array_equal(H @ H.T, n * np.eye(n, dtype=np.int64)), n


def check_fwht_equals_dense_on_integers():
    rng = np.random.default_rng(1)
    for n in (2, 8, 32, 128):
        Hs = scipy.linalg.hadamard(n).astype(np.int64)
        for _ in range(20):
            x = rng.integers(-(1 << 16), (1 << 16) + 1, n)
            got = oracle.fwht_unnormalized(x.astype(np.float32)).astype(np.float64)
            assert np.array_equal(got, (Hs @ x).astype(np.float64)), n


def check_fwht_involution():
    rng = np.random.default_rng(2)
    for n in (4, 64, 128):
        x = rng.integers(-1000, 1001, n).astype(np.float32)
        y = oracle.fwht_unnormalized(oracle.fwht_unnormalized(x))
        assert np.array_equal(y, n * x)


def check_rotation_constant():
    for k in range(1, 9):
        n = 1 << k
        c = np.float32(oracle.rotation_constant(n))
        # c is the float nearest 1/sqrt(n): |c^2 n - 1| is minimal among c and its neighbours
        def err(v):
            return abs(Fraction(float(v)) ** 2 * n - 1)
        for nb in (np.nextafter(c, np.float32(0)), np.nextafter(c, np.float32(1))):
            assert err(c) < err(nb), (n, c)
    assert np.array(np.float32(oracle.rotation_constant(128))).view(np.uint32) == 0x3DB504F3


def check_rotate_one_hot():
    n = 128
    H = scipy.linalg.hadamard(n)
    for c in (0, 5, 77, 127):
        for A in (10.0, -3.5):
            x = np.zeros(n, np.float32)
            x[c] = A
            y = oracle.rotate(x, n)
            mag = np.float32(A) * np.float32(oracle.rotation_constant(n))
            assert np.array_equal(y, (H[:, c] * mag).astype(np.float32)), (c, A)


def check_rotate_matches_dense():
    rng = np.random.default_rng(3)
    n = 128
    R = scipy.linalg.hadamard(n) / np.sqrt(n)
    for block in (32, 64, 128):
        Rb = np.kron(np.eye(n // block), scipy.linalg.hadamard(block) / np.sqrt(block))
        for _ in range(10):
            x = rng.standard_normal(n).astype(np.float32)
            y32 = oracle.rotate(x, block).astype(np.float64)
            y64 = oracle.rotate_dense_f64(x.astype(np.float64), block)
            ref = Rb @ x.astype(np.float64)
            assert np.max(np.abs(y64 - ref)) < 1e-13
            assert np.max(np.abs(y32 - ref)) < 1e-5 * np.max(np.abs(ref)) + 1e-6
    assert R.shape == (n, n)


def check_qk_invariance():
    rng = np.random.default_rng(4)
    for _ in range(20):
        q = rng.standard_normal(128)
        k = rng.standard_normal(128) * np.where(rng.random(128) < 0.03, 10.0, 1.0)
        rq = oracle.rotate_dense_f64(q, 128)
        rk = oracle.rotate_dense_f64(k, 128)
        assert abs(rq @ rk - q @ k) <= 1e-12 * np.linalg.norm(q) * np.linalg.norm(k)
        rq32 = oracle.rotate(q.astype(np.float32), 128).astype(np.float64)
        rk32 = oracle.rotate(k.astype(np.float32), 128).astype(np.float64)
        q32, k32 = q.astype(np.float32).astype(np.float64), k.astype(np.float32).astype(np.float64)
        assert abs(rq32 @ rk32 - q32 @ k32) <= 1e-5 * np.linalg.norm(q) * np.linalg.norm(k)


# ----------------------------------------------------------------------------- formats

def check_f16_conversion_f16c(full: bool = True):
    """Every binary32 whose binary16 rounding is not trivially 0 or inf, against F16C."""
    lib = _f16c_lib()
    fn = ctypes.cast(oracle.load().orc_f32_to_f16, ctypes.c_void_p)
    first = ctypes.c_uint32(0)
    if full:
        ranges = [(0x33000000, 0x47800000)]   # [2^-25, 2^16]: every rounding case
    else:
        ranges = [(0x33000000 + i * 0x100000, 0x33000000 + i * 0x100000 + 0x3FFF) for i in range(0x148)]
    # below 2^-25 everything rounds to zero, above 2^16 to infinity: check the edges
    ranges += [(0x0, 0x2000), (0x32FF0000, 0x33000000), (0x47800000, 0x47810000),
               (0x7F7FF000, 0x7F800010), (0x7FC00000, 0x7FC00010)]
    for lo, hi in ranges:
        bad = lib.f16_check_range(fn, lo, hi, ctypes.byref(first))
        assert bad == 0, f"{bad} mismatches, first 0x{first.value:08x}"


def check_f16_conversion_numpy():
    rng = np.random.default_rng(5)
    u = rng.integers(0, 1 << 32, 1 << 22, dtype=np.uint64).astype(np.uint32)
    x = u.view(np.float32)
    finite = np.isfinite(x)
    got = oracle.f32_to_f16_bits(x[finite])
    with np.errstate(over="ignore"):
        ref = x[finite].astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    back = oracle.f16_bits_to_f32(h)
    ref32 = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref32)
    assert np.array_equal(np.isnan(back), nan)
    assert np.array_equal(back[~nan].view(np.uint32), ref32[~nan].view(np.uint32))


def check_fmaf_exact():
    rng = np.random.default_rng(6)
    for _ in range(3000):
        c = float(rng.integers(0, 16))
        s = float(np.float16(abs(rng.standard_normal()) * 0.3))
        z = float(np.float16(rng.standard_normal() * 2))
        got = np.float32(oracle.fmaf(c, s, z))
        ref = nearest_f32(Fraction(c) * Fraction(s) + Fraction(z))
        assert got == ref or (got == 0 and ref == 0), (c, s, z, got, ref)
    # a case where fma and multiply-then-add differ
    a, b, cc = np.float32(1 + 2 ** -12), np.float32(1 + 2 ** -12), np.float32(-1)
    exact = Fraction(float(a)) * Fraction(float(b)) + Fraction(float(cc))
    assert np.float32(oracle.fmaf(float(a), float(b), float(cc))) == nearest_f32(exact)


# ----------------------------------------------------------------------------- quantizer

def _golden_cases():
    with open(GOLDEN) as f:
        data = json.load(f)
    for c in data["cases"]:
        if "x_rule" in c:
            pat_x = [0, 3, 1, 2, 0.5, 1.5, 2.5, 2.4]
            pat_c = [0, 3, 1, 2, 0, 2, 2, 2]
            x = [pat_x[i % 8] for i in range(c["group"])]
            codes = [pat_c[i % 8] for i in range(c["group"])]
        else:
            x, codes = c["x"], c["codes"]
        yield c["name"], c["bits"], c["group"], np.array(x, np.float32), np.array(codes, np.uint8), \
            int(c["scale_bits"], 16), int(c["zero_bits"], 16)


def check_quantizer_worked_examples():
    for name, bits, group, x, codes, sb, zb in _golden_cases():
        got_c, got_s, got_z = oracle.quantize_row(x, bits, group)
        assert got_s[0] == sb, (name, hex(got_s[0]), hex(sb))
        assert got_z[0] == zb, (name, hex(got_z[0]), hex(zb))
        assert np.array_equal(got_c, codes), (name, got_c, codes)


def check_codes_in_range_and_extremes():
    rng = np.random.default_rng(7)
    for bits in (2, 4):
        for group in (32, 64, 128):
            for _ in range(50):
                x = (rng.standard_normal(128) * np.exp(rng.standard_normal())).astype(np.float32)
                codes, sc, ze = oracle.quantize_row(x, bits, group)
                assert codes.max() <= (1 << bits) - 1
                for g in range(128 // group):
                    cg = codes[g * group:(g + 1) * group]
                    xg = x[g * group:(g + 1) * group]
                    # the group minimum maps to code 0 and the maximum to the top code
                    # unless fp16 rounding of scale/zero moves them by one level
                    assert cg[np.argmin(xg)] <= 1 and cg[np.argmax(xg)] >= (1 << bits) - 2


def check_codes_in_range_offset_groups():
    """Large mean, small range: the fp16 zero can land above the minimum, so the
    unclamped code would be negative; codes must still lie in [0, 2^bits-1] and the
    round trip obey the bound with the zero's rounding included."""
    rng = np.random.default_rng(17)
    for bits in (2, 4):
        for base in (1000.1, -777.7, 3.3e4):
            x = (base + rng.random(128) * 0.9).astype(np.float32)
            codes, sc, ze = oracle.quantize_row(x, bits, 32)
            assert codes.max() <= (1 << bits) - 1
            s = sc.view(np.float16).astype(np.float64)
            z = ze.view(np.float16).astype(np.float64)
            for g in range(4):
                xg = x[g * 32:(g + 1) * 32].astype(np.float64)
                xh = np.array([oracle.fmaf(float(c), float(s[g]), float(z[g])) for c in codes[g * 32:(g + 1) * 32]])
                ulp = float(np.spacing(np.float32(np.max(np.abs(xg)))))
                assert np.all(np.abs(xg - xh) <= s[g] / 2 + abs(xg.min() - z[g]) + 4 * ulp)


def check_round_trip_bound():
    """|x - xhat| <= scale/2 + |min - zero| + 4 ulp(max|x|), per element."""
    rng = np.random.default_rng(8)
    for bits in (2, 4):
        for group in (32, 64, 128):
            for trial in range(100):
                x = rng.standard_normal(128).astype(np.float32)
                if trial % 3 == 0:
                    x[rng.integers(0, 128, 3)] *= 10
                codes, sc, ze = oracle.quantize_row(x, bits, group)
                s = sc.view(np.float16).astype(np.float64)
                z = ze.view(np.float16).astype(np.float64)
                for g in range(128 // group):
                    xg = x[g * group:(g + 1) * group].astype(np.float64)
                    xh = np.array([oracle.fmaf(float(c), float(s[g]), float(z[g]))
                                   for c in codes[g * group:(g + 1) * group]])
                    ulp = np.spacing(np.float32(np.max(np.abs(xg)))).astype(np.float64)
                    bound = s[g] / 2 + abs(xg.min() - z[g]) + 4 * ulp
                    assert np.all(np.abs(xg - xh) <= bound), (bits, group, trial)


def check_packing_order():
    codes4 = np.arange(16, dtype=np.uint8)
    assert list(oracle.pack_row(codes4, 4)) == [0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE]
    codes2 = np.array([0, 1, 2, 3, 3, 2, 1, 0], np.uint8)
    assert list(oracle.pack_row(codes2, 2)) == [0b11100100, 0b00011011]
    rng = np.random.default_rng(9)
    for bits in (2, 4):
        c = rng.integers(0, 1 << bits, 128).astype(np.uint8)
        assert np.array_equal(oracle.unpack_row(oracle.pack_row(c, bits), 128, bits), c)


def check_storage_bits_per_element():
    assert oracle.bits_per_element(128, 2, 128) == 2.25
    assert oracle.bits_per_element(128, 4, 32) == 5.0
    assert oracle.bits_per_element(128, 4, 64) == 4.5


def _bf16(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def check_cache_layout_bytes():
    """One token with known codes lands at the documented byte offsets."""
    d, Hkv, P = 128, 2, 32
    c = oracle.Cache(d, Hkv, 4, 32, 0, P, 3)
    # K row for kv head 1: group g holds values 0..15,15..0 -> scale 1, zero 0
    ramp = np.concatenate([np.arange(16), np.arange(15, -1, -1)]).astype(np.float32)
    x = np.tile(ramp, 4)
    k = np.zeros((1, Hkv, d), np.float32)
    v = np.zeros((1, Hkv, d), np.float32)
    k[0, 1] = x
    v[0, 1] = x
    page, off = 2, 21
    c.append(_bf16(k), _bf16(v), np.array([page * P + off]))
    packed = oracle.pack_row(x.astype(np.uint8), 4)
    rb = d * 4 // 8
    o = off % 16
    # K codes: 16-token tiles, rows cut into 16-byte chunks stored chunk-major
    ktile = ((page * Hkv + 1) * P + (off // 16) * 16) * rb
    for k in range(rb):
        assert c.k_codes[ktile + ((k // 16) * 16 + o) * 16 + k % 16] == packed[k], k
    kmeta = ((page * Hkv + 1) * P + off) * 4 * 4
    assert list(c.k_meta[kmeta:kmeta + 4]) == [0x00, 0x3C, 0x00, 0x00]  # scale 1.0, zero 0.0
    vbase = (page * Hkv + 1) * P * rb + (off // 16) * 16 * rb
    for k in range(rb):
        w, b = divmod(k, 2)
        assert c.v_codes[vbase + w * 32 + (o // 2) * 4 + b * 2 + o % 2] == packed[k], k
    # V meta: per tile NG*16 entries; token o = 8*half + 4*part + i of group g at
    # entry ((part*NG + g)*2 + half)*4 + i
    half, part, i = o // 8, (o % 8) // 4, o % 4
    vtile = ((page * Hkv + 1) * (P // 16) + off // 16) * 4 * 16
    for g in range(4):
        e = vtile + ((part * 4 + g) * 2 + half) * 4 + i
        assert list(c.v_meta[e * 4:e * 4 + 4]) == [0x00, 0x3C, 0x00, 0x00], g
    # nothing else was written
    assert np.count_nonzero(c.k_codes) == np.count_nonzero(packed)
    assert np.count_nonzero(c.v_codes) == np.count_nonzero(packed)
    assert np.count_nonzero(c.k_meta) == 4 and np.count_nonzero(c.v_meta) == 4


def check_v_not_rotated_and_k_rotated():
    """Dequantized V is within the round-trip bound of raw V; dequantized K of R k."""
    rng = np.random.default_rng(10)
    d, Hkv, n = 128, 2, 8
    c = oracle.Cache(d, Hkv, 4, 32, 128, 16, 1)
    k = _bf16(rng.standard_normal((n, Hkv, d)))
    v = _bf16(rng.standard_normal((n, Hkv, d)))
    slots = np.arange(n)
    c.append(k, v, slots)
    R = scipy.linalg.hadamard(d) / np.sqrt(d)
    kh, vh = c.dequantize(0, slots), c.dequantize(1, slots)
    kf, vf = oracle.bf16_to_f32(k).astype(np.float64), oracle.bf16_to_f32(v).astype(np.float64)
    krot = kf @ R.T
    for ref, got in ((krot, kh), (vf, vh)):
        for g in range(4):
            sl = slice(32 * g, 32 * (g + 1))
            rng_g = ref[..., sl].max(-1) - ref[..., sl].min(-1)
            assert np.all(np.abs(ref[..., sl] - got[..., sl]).max(-1) <= rng_g / 15 * 0.5 * 1.01 + 1e-3)


# ----------------------------------------------------------------------------- attention

def _rand_cache(rng, d=128, Hkv=2, T=40, bits=4, G=32, hb=128, P=16, paged_perm=None, B=2, mode=0):
    pages_per = (T + P - 1) // P
    num_pages = B * pages_per
    c = oracle.Cache(d, Hkv, bits, G, hb, P, num_pages, quant_mode=mode)
    perm = np.arange(num_pages) if paged_perm is None else paged_perm
    bt = perm.reshape(B, pages_per).astype(np.int32)
    k = _bf16(rng.standard_normal((B, T, Hkv, d)))
    v = _bf16(rng.standard_normal((B, T, Hkv, d)))
    for b in range(B):
        t = np.arange(T)
        slots = bt[b][t // P].astype(np.int64) * P + t % P
        c.append(k[b], v[b], slots)
    return c, bt, k, v


def check_attention_matches_sdpa():
    rng = np.random.default_rng(11)
    for hb, bits, G, mode in ((128, 4, 32, 0), (0, 4, 64, 0), (128, 2, 128, 0), (64, 4, 32, 0), (128, 2, 32, 1)):
        B, Hq, Hkv, d, T, P = 2, 8, 2, 128, 45, 16
        c, bt, k, v = _rand_cache(rng, d, Hkv, T, bits, G, hb, P, B=B, mode=mode)
        q = _bf16(rng.standard_normal((B, Hq, d)))
        lens = np.array([T, 17], np.int32)
        out = c.decode(q, bt, lens, 0.0)
        # independent: scipy Hadamard, oracle-free dequant via page table, torch SDPA in fp64
        blk = hb if hb else d
        R = np.kron(np.eye(d // blk), scipy.linalg.hadamard(blk) / np.sqrt(blk)) if hb else np.eye(d)
        for b in range(B):
            t = np.arange(lens[b])
            slots = bt[b][t // P].astype(np.int64) * P + t % P
            kh = torch.from_numpy(c.dequantize(0, slots).astype(np.float64))  # [T][Hkv][d]
            vh = torch.from_numpy(c.dequantize(1, slots).astype(np.float64))
            qf = oracle.bf16_to_f32(q[b]).astype(np.float64) @ R.T            # [Hq][d]
            qt = torch.from_numpy(qf).reshape(Hkv, Hq // Hkv, 1, d)
            kt = kh.permute(1, 0, 2).reshape(Hkv, 1, -1, d).contiguous()
            vt = vh.permute(1, 0, 2).reshape(Hkv, 1, -1, d).contiguous()
            ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)  # scale 1/sqrt(d)
            ref = ref.reshape(Hq, d).numpy()
            assert np.max(np.abs(out[b] - ref)) < 1e-12, (hb, bits, G, b)


def check_attention_special_cases():
    rng = np.random.default_rng(12)
    B, Hq, Hkv, d, P = 1, 4, 1, 128, 16
    c, bt, k, v = _rand_cache(rng, d, Hkv, 32, 4, 32, 128, P, B=B)
    q = _bf16(rng.standard_normal((B, Hq, d)))
    # T = 1: output is the first dequantized value row exactly
    out = c.decode(q, bt, np.array([1], np.int32))
    v0 = c.dequantize(1, np.array([bt[0][0] * P]))[0, 0].astype(np.float64)
    assert np.all(out[0] == v0)
    # q = 0: uniform weights -> mean of dequantized V
    out = c.decode(np.zeros_like(q), bt, np.array([32], np.int32))
    slots = bt[0][np.arange(32) // P].astype(np.int64) * P + np.arange(32) % P
    vm = c.dequantize(1, slots)[:, 0].astype(np.float64).mean(0)
    assert np.max(np.abs(out[0] - vm)) < 1e-12
    # seq_len 0: zeros
    out = c.decode(q, bt, np.array([0], np.int32))
    assert np.all(out == 0)
    # identical keys: uniform weights again
    c2 = oracle.Cache(d, 1, 4, 32, 128, P, 2)
    kk = np.repeat(_bf16(rng.standard_normal((1, 1, d))), 32, axis=0)
    vv = _bf16(rng.standard_normal((32, 1, d)))
    c2.append(kk, vv, np.arange(32))
    out = c2.decode(q, np.array([[0, 1]], np.int32), np.array([32], np.int32))
    vm = c2.dequantize(1, np.arange(32))[:, 0].astype(np.float64).mean(0)
    assert np.max(np.abs(out[0] - vm)) < 1e-12


def check_attention_page_permutation():
    B, T, P = 2, 64, 16
    pages = B * T // P
    outs = []
    for perm in (np.arange(pages), np.random.default_rng(13).permutation(pages)):
        rng = np.random.default_rng(14)
        c, bt, k, v = _rand_cache(rng, 128, 2, T, 4, 32, 128, P, paged_perm=perm, B=B)
        q = _bf16(np.random.default_rng(15).standard_normal((B, 8, 128)))
        outs.append(c.decode(q, bt, np.array([T, T - 5], np.int32)))
    assert np.array_equal(outs[0], outs[1])


# ----------------------------------------------------------------------------- windows

def _window_stream(rng, T, S, R, B=2, Hkv=2, d=128, P=16, bits=4, G=32, hb=128):
    """Append T tokens one at a time through the windows; returns the oracle objects and
    the raw bf16 tokens [B][T][Hkv][d]. Contiguous pages: slot of position t = b*cap + t."""
    cap = (T + P - 1) // P * P
    c = oracle.Cache(d, Hkv, bits, G, hb, cap, B)
    w = oracle.Window(d, Hkv, S, R, B)
    k = _bf16(rng.standard_normal((B, T, Hkv, d)) * np.exp(rng.standard_normal((1, 1, Hkv, d))))
    v = _bf16(rng.standard_normal((B, T, Hkv, d)))
    for t in range(T):
        ev = np.array([b * cap + (t - R) for b in range(B)], np.int64)
        w.append(c, k[:, t], v[:, t], np.arange(B), np.full(B, t), ev)
    bt = np.arange(B, dtype=np.int32).reshape(B, 1)
    return c, w, bt, k, v, cap


def check_window_all_tokens_in_windows():
    """Every token still in a window: plain fp64 attention over the raw bf16 rows."""
    rng = np.random.default_rng(31)
    for T, S, R in ((40, 32, 16), (20, 32, 4), (33, 32, 1)):
        c, w, bt, k, v, cap = _window_stream(rng, T, S, R)
        q = _bf16(rng.standard_normal((2, 8, 128)))
        out = w.decode(c, q, bt, np.array([T, T], np.int32))
        ref = oracle.attention_bf16(q, k, v, 2)
        assert np.max(np.abs(out - ref)) < 1e-12, (T, S, R)
        assert not c.k_codes.any() and not c.v_codes.any()  # nothing was quantized


def check_window_evictions_match_direct_quantization():
    """Tokens that left the recent window are in the cache exactly as a direct append of
    them would put them; the windows hold the sink tokens and the last R tokens."""
    rng = np.random.default_rng(32)
    T, S, R = 100, 32, 8
    c, w, bt, k, v, cap = _window_stream(rng, T, S, R)
    ref = oracle.Cache(128, 2, 4, 32, 128, cap, 2)
    for b in range(2):
        t = np.arange(S, T - R)
        ref.append(k[b, S:T - R], v[b, S:T - R], b * cap + t)
    for g, r in zip(c.planes(), ref.planes()):
        assert np.array_equal(g, r)
    for b in range(2):
        for t in list(range(S)) + list(range(T - R, T)):
            slot = S + (t - S) % R if t >= S else t
            assert np.array_equal(w.k[b, slot], k[b, t]) and np.array_equal(w.v[b, slot], v[b, t]), (b, t)


def check_window_decode_mixed():
    """Window tokens with the original query and raw rows, cache tokens with the rotated
    query (scipy Hadamard) and the oracle's dequantized rows, one softmax: against a
    direct fp64 softmax written out in numpy over the assembled rows."""
    rng = np.random.default_rng(33)
    T, S, R, P = 100, 32, 8, 16
    c, w, bt, k, v, cap = _window_stream(rng, T, S, R)
    q = _bf16(rng.standard_normal((2, 8, 128)))
    lens = np.array([T, T], np.int32)  # the windows hold the state after T appends
    out = w.decode(c, q, bt, lens)
    Rm = scipy.linalg.hadamard(128) / np.sqrt(128)
    for b in range(2):
        qf = oracle.bf16_to_f32(q[b]).astype(np.float64)  # [Hq][d]
        logits = np.empty((8, T))
        vals = np.empty((T, 2, 128))
        for t in range(T):
            if t < S or t >= T - R:  # window token: raw rows, original query
                kt = oracle.bf16_to_f32(k[b, t]).astype(np.float64)
                vals[t] = oracle.bf16_to_f32(v[b, t]).astype(np.float64)
                logits[:, t] = np.einsum("jd,jd->j", qf, np.repeat(kt, 4, axis=0))
            else:  # cache token: dequantized rows, rotated query
                kt = c.dequantize(0, np.array([b * cap + t]))[0].astype(np.float64)
                vals[t] = c.dequantize(1, np.array([b * cap + t]))[0].astype(np.float64)
                logits[:, t] = np.einsum("jd,jd->j", qf @ Rm.T, np.repeat(kt, 4, axis=0))
        logits /= np.sqrt(128)
        p = np.exp(logits - logits.max(1, keepdims=True))
        ref = np.einsum("jt,jtd->jd", p, np.repeat(vals, 4, axis=1).transpose(1, 0, 2)) / p.sum(1, keepdims=True)
        assert np.max(np.abs(out[b] - ref)) < 1e-12, b


# ----------------------------------------------------------------------------- hybrid quantizer

HYBRID_GOLDEN = os.path.join(HERE, "golden", "hybrid_worked_examples.json")


def check_hybrid_worked_examples():
    with open(HYBRID_GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        x = np.array(c["x"], np.float32)
        codes, sc, ze = oracle.quantize_row(x, c["bits"], c["group"], hybrid=True)
        assert sc[0] == int(c["scale_bits"], 16), (c["name"], hex(sc[0]))
        assert ze[0] == int(c["zero_bits"], 16), (c["name"], hex(ze[0]))
        assert np.array_equal(codes, np.array(c["codes"], np.uint8)), (c["name"], codes)


def _max_err(x, codes, sc, ze, group):
    """Largest |x - fma(code, s, z)| per group, fma evaluated exactly in fp64 then rounded."""
    s = np.repeat(sc.view(np.float16).astype(np.float64), group)
    z = np.repeat(ze.view(np.float16).astype(np.float64), group)
    xh = (codes.astype(np.float64) * s + z).astype(np.float32)  # one rounding: the product is exact
    return np.abs(x - xh).reshape(-1, group).max(axis=1)


def check_hybrid_never_worse_and_one_of_two():
    """Per group the hybrid pair is the asymmetric one or the symmetric candidate
    (computed here in numpy: scale = f16(max|x| / (2^(b-1)-1)), zero = -2^(b-1) scale,
    codes by the shared formula), and its largest error never exceeds the asymmetric one."""
    rng = np.random.default_rng(41)
    n_sym = 0
    for bits in (2, 4):
        mid = 1 << (bits - 1)
        for group in (32, 64, 128):
            for trial in range(60):
                kind = trial % 3
                x = rng.standard_normal(128) if kind == 0 else (
                    rng.uniform(-1, 1, 128) if kind == 1 else rng.laplace(size=128))
                x = (x * np.exp(rng.standard_normal())).astype(np.float32)
                ca, sa, za = oracle.quantize_row(x, bits, group)
                ch, sh, zh = oracle.quantize_row(x, bits, group, hybrid=True)
                ea, eh = _max_err(x, ca, sa, za, group), _max_err(x, ch, sh, zh, group)
                assert np.all(eh <= ea), (bits, group, trial)
                for g in range(128 // group):
                    sl = slice(g * group, (g + 1) * group)
                    if sh[g] == sa[g] and zh[g] == za[g]:
                        assert np.array_equal(ch[sl], ca[sl])
                        continue
                    n_sym += 1
                    xg = x[sl]
                    a = np.float32(np.max(np.abs(xg)))
                    s16 = np.float16(a / np.float32(mid - 1))
                    z16 = np.float16(-np.float32(mid) * np.float32(s16))
                    assert sh[g] == s16.view(np.uint16) and zh[g] == z16.view(np.uint16), (bits, group, trial, g)
                    s, z = np.float32(s16), np.float32(z16)
                    u = ((xg - z) * (np.float32(1.0) / s)).astype(np.float32)
                    want = np.clip(np.rint(u), 0, (1 << bits) - 1).astype(np.uint8)
                    assert np.array_equal(ch[sl], want)
                    assert eh[g] < ea[g]
    assert n_sym > 0  # the symmetric branch was exercised


def check_hybrid_cache_append_stores_the_hybrid_rows():
    """A hybrid cache dequantizes every appended row to the hybrid quantizer's values
    (keys after the rotation), and an asymmetric cache to the asymmetric ones."""
    rng = np.random.default_rng(42)
    for mode in (0, 1):
        c = oracle.Cache(128, 2, 2, 32, 128, 16, 2, quant_mode=mode)
        k = _bf16(rng.uniform(-1, 1, (20, 2, 128)))
        # ternary values (power-of-two scaled) make the symmetric INT2 pair exact
        v = _bf16(rng.integers(-1, 2, (20, 2, 128)) * 2.0 ** rng.integers(-3, 4, (20, 2, 1)))
        slots = np.arange(20, dtype=np.int64) + 5
        c.append(k, v, slots)
        if mode == 1:  # the mode matters: some stored V groups are symmetric (zero = -2 scale)
            ve = oracle.Cache(128, 2, 2, 32, 128, 16, 2)
            ve.append(k, v, slots)
            assert not np.array_equal(c.dequantize(1, slots), ve.dequantize(1, slots))
        for which, src in ((0, k), (1, v)):
            got = c.dequantize(which, slots)
            for r in range(20):
                for h in range(2):
                    x = oracle.bf16_to_f32(src[r, h])
                    if which == 0:
                        x = oracle.rotate(x, 128)
                    codes, sc, ze = oracle.quantize_row(x, 2, 32, hybrid=bool(mode))
                    s = np.repeat(sc.view(np.float16).astype(np.float64), 32)
                    z = np.repeat(ze.view(np.float16).astype(np.float64), 32)
                    want = (codes * s + z).astype(np.float32)
                    assert np.array_equal(got[r, h], want), (mode, which, r, h)


# ----------------------------------------------------------------------------- query-channel pruning

def check_pruned_all_kept_equals_plain():
    rng = np.random.default_rng(51)
    for bits, G in ((4, 32), (2, 128)):
        c, bt, k, v = _rand_cache(rng, 128, 2, 40, bits, G, 128, 16)
        q = _bf16(rng.standard_normal((2, 8, 128)))
        lens = np.array([40, 23], np.int32)
        full = np.full((2, 2), (1 << bits) - 1, np.int32)  # d * bits / 128 = bits chunks per key row
        assert np.array_equal(c.decode_pruned(q, bt, lens, full), c.decode(q, bt, lens))


def check_pruned_matches_restricted_sdpa():
    """Pruned decode = fp64 SDPA with the scipy-rotated query zeroed outside the kept
    chunks (W = 128 / bits channels each), on the oracle's dequantized K/V."""
    rng = np.random.default_rng(52)
    for bits, G, hb in ((4, 32, 128), (4, 64, 64), (2, 128, 128), (2, 32, 0)):
        B, Hq, Hkv, d, T, P = 2, 8, 2, 128, 45, 16
        W, nch = 128 // bits, bits
        c, bt, k, v = _rand_cache(rng, d, Hkv, T, bits, G, hb, P, B=B)
        q = _bf16(rng.standard_normal((B, Hq, d)))
        lens = np.array([T, 29], np.int32)
        mask = rng.integers(1, 1 << nch, (B, Hkv)).astype(np.int32)
        out = c.decode_pruned(q, bt, lens, mask)
        Rm = np.kron(np.eye(d // hb), scipy.linalg.hadamard(hb) / np.sqrt(hb)) if hb else np.eye(d)
        for b in range(B):
            t = np.arange(lens[b])
            slots = bt[b][t // P].astype(np.int64) * P + t % P
            kh = torch.from_numpy(c.dequantize(0, slots).astype(np.float64))
            vh = torch.from_numpy(c.dequantize(1, slots).astype(np.float64))
            qf = oracle.bf16_to_f32(q[b]).astype(np.float64) @ Rm.T
            for h in range(Hkv):
                keep = np.repeat([(mask[b, h] >> j) & 1 for j in range(nch)], W).astype(np.float64)
                qf[h * (Hq // Hkv):(h + 1) * (Hq // Hkv)] *= keep
            qt = torch.from_numpy(qf).reshape(Hkv, Hq // Hkv, 1, d)
            kt = kh.permute(1, 0, 2).reshape(Hkv, 1, -1, d).contiguous()
            vt = vh.permute(1, 0, 2).reshape(Hkv, 1, -1, d).contiguous()
            ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt).reshape(Hq, d).numpy()
            assert np.max(np.abs(out[b] - ref)) < 1e-12, (bits, G, hb, b)


def check_prune_energy():
    rng = np.random.default_rng(53)
    for bits, hb in ((4, 128), (2, 32)):
        c = oracle.Cache(128, 2, bits, 32, hb, 16, 1)
        q = _bf16(rng.standard_normal((3, 8, 128)))
        e = c.prune_energy(q)
        Rm = np.kron(np.eye(128 // hb), scipy.linalg.hadamard(hb) / np.sqrt(hb))
        qf = oracle.bf16_to_f32(q).astype(np.float64) @ Rm.T          # [B][Hq][d]
        want = (qf ** 2).reshape(3, 2, 4, bits, 128 // bits).sum(axis=(2, 4))
        assert np.allclose(e, want, rtol=1e-12, atol=0), bits


# ----------------------------------------------------------------------------- V token groups

def _vt_entry(bits, ch):
    """Entry of channel ch in a token group's {scale, zero} list: the documented formula
    c = 4(n + 16(t>>2)) + 2(t&1) + ((t>>1)&1) (INT4) / 8n + (t>>1) + 4(t&1) (INT2) at 8n + t,
    evaluated forward over all (n, t) and inverted here."""
    table = {}
    for n in range(16):
        for t in range(8):
            c = 4 * (n + 16 * (t >> 2)) + 2 * (t & 1) + ((t >> 1) & 1) if bits == 4 else 8 * n + (t >> 1) + 4 * (t & 1)
            table[c] = 8 * n + t
    return table[ch]


def check_vt_entry_is_a_permutation():
    for bits in (2, 4):
        assert sorted(_vt_entry(bits, c) for c in range(128)) == list(range(128))


def _vt_cache(P, pages, bits=4, G=32, hb=128, mode=0):
    return oracle.Cache(128, 2, bits, G, hb, P, pages, quant_mode=mode, v_grouping=1)


def check_vt_worked_example_and_layout():
    """V channel 37 of kv head 1 holds the ramp 0..31 across the 32 tokens of a group (the
    golden ramp: scale 0x4022, zero 0, codes 0,0,1,1,..,15,15), every other channel a
    constant; read back at the documented byte offsets (V codes: 16-token tiles of 16-bit
    words, token pairs interleaved; V meta: [u][P/G][128] entries)."""
    golden = {n: (x, c, sb, zb) for n, _, _, x, c, sb, zb in _golden_cases()}
    x, codes, sb, zb = golden["ramp_0_to_31_int4_g32"]
    P, pages, H, d = 64, 3, 2, 128
    c = _vt_cache(P, pages)
    v = np.full((32, H, d), 1.25, np.float32)
    v[:, 1, 37] = x
    k = np.zeros((32, H, d), np.float32)
    page, gi = 2, 1                              # token group 1 of page 2: slots 160..191
    slots = np.arange(32, dtype=np.int64) + page * P + gi * 32
    c.append(_bf16(k), _bf16(v), slots)
    u = page * H + 1
    meta = c.v_meta.view(np.uint16).reshape(-1, 2)
    e = (u * (P // 32) + gi) * 128 + _vt_entry(4, 37)
    assert meta[e, 0] == sb and meta[e, 1] == zb, (hex(meta[e, 0]), hex(meta[e, 1]))
    e1 = (u * (P // 32) + gi) * 128 + _vt_entry(4, 36)   # a constant channel: scale 0, zero 1.25
    assert meta[e1, 0] == 0 and meta[e1, 1] == np.float16(1.25).view(np.uint16)
    for i in range(32):
        off = gi * 32 + i
        tile = (u * P + off - off % 16) * 64
        o = off % 16
        byte = c.v_codes[tile + (37 // 2 // 2) * 32 + (o // 2) * 4 + ((37 // 2) % 2) * 2 + o % 2]
        assert (byte >> 4) & 15 == codes[i], (i, byte, codes[i])   # channel 37: high nibble of byte 18


def check_vt_groups_run_along_tokens():
    """A V that is constant along tokens but varies across channels is reproduced exactly
    (every token group of a channel is constant: scale 0, zero = the value), which
    channel groups would not do."""
    rng = np.random.default_rng(71)
    P = 32
    c = _vt_cache(P, 2, bits=2, G=32)
    ch_vals = _bf16(rng.standard_normal((2, 128)))
    v = np.broadcast_to(ch_vals, (64, 2, 128)).copy()
    k = _bf16(rng.standard_normal((64, 2, 128)))
    slots = np.arange(64, dtype=np.int64)
    c.append(k, v, slots)
    got = c.dequantize(1, slots)
    want = np.broadcast_to(oracle.bf16_to_f32(ch_vals), got.shape)
    assert np.array_equal(got, want)
    cc = oracle.Cache(128, 2, 2, 32, 128, P, 2)
    cc.append(k, v, slots)
    assert not np.array_equal(cc.dequantize(1, slots), want)


def check_vt_round_trip_per_channel():
    """Per token group and channel: the group's min maps within one level of code 0, and
    every element is within half a step (plus the zero's rounding and ulps) of its value."""
    rng = np.random.default_rng(72)
    for bits, G in ((4, 32), (2, 64), (4, 128)):
        P = 128
        c = _vt_cache(P, 2, bits=bits, G=G)
        v = _bf16(rng.standard_normal((128, 2, 128)) * np.exp(rng.standard_normal((1, 2, 128))))
        k = _bf16(rng.standard_normal((128, 2, 128)))
        slots = np.arange(128, dtype=np.int64) + P
        c.append(k, v, slots)
        got = c.dequantize(1, slots).astype(np.float64)
        x = oracle.bf16_to_f32(v).astype(np.float64)
        meta = c.v_meta.view(np.uint16).reshape(-1, 2)
        for h in range(2):
            for gi in range(128 // G):
                for ch in range(128):
                    e = ((1 * 2 + h) * (P // G) + gi) * 128 + _vt_entry(bits, ch)
                    sc = float(np.uint16(meta[e, 0]).view(np.float16))
                    ze = float(np.uint16(meta[e, 1]).view(np.float16))
                    xs = x[gi * G:(gi + 1) * G, h, ch]
                    err = np.abs(got[gi * G:(gi + 1) * G, h, ch] - xs)
                    assert err.max() <= sc / 2 + abs(xs.min() - ze) + 4 * np.spacing(np.abs(xs).max()), \
                        (bits, G, h, gi, ch)


def check_vt_attention_matches_sdpa():
    rng = np.random.default_rng(73)
    for bits, G, hb, mode in ((4, 32, 128, 0), (2, 64, 0, 1), (4, 128, 64, 0)):
        B, Hq, Hkv, d, P = 2, 8, 2, 128, 128
        T = 256
        pages_per = T // P
        perm = rng.permutation(B * pages_per)
        bt = perm.reshape(B, pages_per).astype(np.int32)
        c = oracle.Cache(d, Hkv, bits, G, hb, P, B * pages_per, quant_mode=mode, v_grouping=1)
        k = _bf16(rng.standard_normal((B, T, Hkv, d)))
        v = _bf16(rng.standard_normal((B, T, Hkv, d)))
        for b in range(B):
            t = np.arange(T)
            c.append(k[b], v[b], bt[b][t // P].astype(np.int64) * P + t % P)
        q = _bf16(rng.standard_normal((B, Hq, d)))
        lens = np.array([T, 3 * G if 3 * G <= T else G], np.int32)
        out = c.decode(q, bt, lens, 0.0)
        Rm = np.kron(np.eye(d // hb), scipy.linalg.hadamard(hb) / np.sqrt(hb)) if hb else np.eye(d)
        for b in range(B):
            t = np.arange(lens[b])
            slots = bt[b][t // P].astype(np.int64) * P + t % P
            kh = torch.from_numpy(c.dequantize(0, slots).astype(np.float64))
            vh = torch.from_numpy(c.dequantize(1, slots).astype(np.float64))
            qf = oracle.bf16_to_f32(q[b]).astype(np.float64) @ Rm.T
            qt = torch.from_numpy(qf).reshape(Hkv, Hq // Hkv, 1, d)
            kt = kh.permute(1, 0, 2).reshape(Hkv, 1, -1, d).contiguous()
            vt = vh.permute(1, 0, 2).reshape(Hkv, 1, -1, d).contiguous()
            ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt).reshape(Hq, d).numpy()
            assert np.max(np.abs(out[b] - ref)) < 1e-12, (bits, G, hb, b)


def check_residual_stream():
    """Tokens streamed through a residual of G rows: every completed group is in the cache
    exactly as a direct append of it writes it (token groups or channel groups), the
    residual holds the incomplete last group at rows t % G, and a decode equals a softmax
    written out over dequantized cache tokens (rotated query) and raw residual rows
    (original query)."""
    rng = np.random.default_rng(74)
    for vg, T in ((1, 100), (0, 77), (1, 64)):
        B, H, d, G, P = 2, 2, 128, 32, 64
        cap = (T + P - 1) // P * P
        c = oracle.Cache(d, H, 4, G, 128, cap, B, v_grouping=vg)
        w = oracle.Window(d, H, 0, G, B, residual=1)
        k = _bf16(rng.standard_normal((B, T, H, d)) * np.exp(rng.standard_normal((1, 1, H, d))))
        v = _bf16(rng.standard_normal((B, T, H, d)))
        for t in range(T):
            first = t - G + 1
            ev = np.array([b * cap + max(first, 0) for b in range(B)], np.int64)
            w.append(c, k[:, t], v[:, t], np.arange(B), np.full(B, t), ev)
        done = T - T % G
        ref = oracle.Cache(d, H, 4, G, 128, cap, B, v_grouping=vg)
        for b in range(B):
            if done:
                ref.append(k[b, :done], v[b, :done], b * cap + np.arange(done, dtype=np.int64))
        for g_, r_ in zip(c.planes(), ref.planes()):
            assert np.array_equal(g_, r_), (vg, T)
        for b in range(B):
            for t in range(done, T):
                assert np.array_equal(w.k[b, t % G], k[b, t]) and np.array_equal(w.v[b, t % G], v[b, t])
        q = _bf16(rng.standard_normal((B, 8, d)))
        bt = np.arange(B, dtype=np.int32).reshape(B, 1)
        out = w.decode(c, q, bt, np.array([T, T], np.int32))
        Rm = scipy.linalg.hadamard(d) / np.sqrt(d)
        for b in range(B):
            qf = oracle.bf16_to_f32(q[b]).astype(np.float64)
            logits = np.empty((8, T))
            vals = np.empty((T, H, d))
            for t in range(T):
                if t >= done:
                    kt = oracle.bf16_to_f32(k[b, t]).astype(np.float64)
                    vals[t] = oracle.bf16_to_f32(v[b, t]).astype(np.float64)
                    logits[:, t] = np.einsum("jd,jd->j", qf, np.repeat(kt, 4, axis=0))
                else:
                    kt = c.dequantize(0, np.array([b * cap + t]))[0].astype(np.float64)
                    vals[t] = c.dequantize(1, np.array([b * cap + t]))[0].astype(np.float64)
                    logits[:, t] = np.einsum("jd,jd->j", qf @ Rm.T, np.repeat(kt, 4, axis=0))
            logits /= np.sqrt(d)
            p = np.exp(logits - logits.max(1, keepdims=True))
            want = np.einsum("jt,jtd->jd", p, np.repeat(vals, 4, axis=1).transpose(1, 0, 2)) / p.sum(1, keepdims=True)
            assert np.max(np.abs(out[b] - want)) < 1e-12, (vg, T, b)


ALL_CHECKS = [
    check_hadamard_is_sylvester,
    check_hadamard_orthogonal,
    check_fwht_equals_dense_on_integers,
    check_fwht_involution,
    check_rotation_constant,
    check_rotate_one_hot,
    check_rotate_matches_dense,
    check_qk_invariance,
    check_f16_conversion_numpy,
    check_fmaf_exact,
    check_quantizer_worked_examples,
    check_codes_in_range_and_extremes,
    check_codes_in_range_offset_groups,
    check_round_trip_bound,
    check_packing_order,
    check_storage_bits_per_element,
    check_cache_layout_bytes,
    check_v_not_rotated_and_k_rotated,
    check_attention_matches_sdpa,
    check_attention_special_cases,
    check_attention_page_permutation,
    check_window_all_tokens_in_windows,
    check_window_evictions_match_direct_quantization,
    check_window_decode_mixed,
    check_hybrid_worked_examples,
    check_hybrid_never_worse_and_one_of_two,
    check_hybrid_cache_append_stores_the_hybrid_rows,
    check_pruned_all_kept_equals_plain,
    check_pruned_matches_restricted_sdpa,
    check_prune_energy,
    check_vt_entry_is_a_permutation,
    check_vt_worked_example_and_layout,
    check_vt_groups_run_along_tokens,
    check_vt_round_trip_per_channel,
    check_vt_attention_matches_sdpa,
    check_residual_stream,
]
