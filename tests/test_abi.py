"""The C ABI on the CPU: the library loads, exports what include/kvq.h declares, and
rejects every malformed argument with its documented status before launching
anything. Every call here returns before any kernel launch (invalid arguments, or
empty work), so these tests are safe on machines with or without a GPU; the fake
device pointers below are never dereferenced."""
import ctypes
import os
import re

import pytest

import bit_kv_cache_quantize_amd as kvq
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")

FAKE = 0x10000  # 16-byte aligned, never dereferenced


def _desc(**kw):
    base = dict(head_dim=128, num_kv_heads=8, bits=4, group_size=32, hadamard_block=128, page_size=16,
                num_pages=64)
    base.update(kw)
    d = kvq._Desc(base["head_dim"], base["num_kv_heads"], base["bits"], base["group_size"],
                  base["hadamard_block"], base["page_size"], base["num_pages"])
    for f in ("k_codes", "k_meta", "v_codes", "v_meta"):
        setattr(d, f, kw.get(f, FAKE))
    d.quant_mode = kw.get("quant_mode", 0)
    d.v_grouping = kw.get("v_grouping", 0)
    return d


def test_library_exports_every_declared_symbol():
    names = set(re.findall(r"\b(kvq_[a-z0-9_]+)\s*\(", open(HEADER).read()))
    assert len(names) >= 9
    lib = kvq.lib()
    for n in sorted(names):
        assert hasattr(lib, n), n
    assert set(kvq.SIGNATURES) == names


def test_status_strings():
    for s, text in ((0, "ok"), (1, "invalid argument"), (2, "unsupported configuration"),
                    (3, "workspace too small"), (4, "HIP runtime error")):
        assert kvq.status_string(s) == text
    assert "gfx950" in kvq.version()


def test_plane_bytes_match_oracle_layout():
    for bits, G, P, pages in ((4, 32, 16, 10), (2, 128, 32, 3), (4, 64, 1024, 2)):
        d = _desc(bits=bits, group_size=G, page_size=P, num_pages=pages)
        got = [kvq.lib().kvq_cache_plane_bytes(ctypes.byref(d), i) for i in range(4)]
        ref = oracle.Cache(128, 8, bits, G, 128, P, pages)
        assert got == [p.size for p in ref.planes()]
    assert kvq.lib().kvq_cache_plane_bytes(ctypes.byref(_desc()), 4) == -1
    assert kvq.lib().kvq_cache_plane_bytes(ctypes.byref(_desc(page_size=24)), 0) == -1


INVALID_CACHES = [
    (dict(head_dim=0), kvq.ERR_INVALID),
    (dict(num_kv_heads=0), kvq.ERR_INVALID),
    (dict(num_pages=0), kvq.ERR_INVALID),
    (dict(bits=3), kvq.ERR_UNSUPPORTED),
    (dict(bits=0), kvq.ERR_INVALID),
    (dict(group_size=48), kvq.ERR_INVALID),          # does not divide head_dim
    (dict(group_size=16), kvq.ERR_UNSUPPORTED),      # divides, but no kernel for it
    (dict(hadamard_block=96), kvq.ERR_INVALID),      # not a power of two
    (dict(hadamard_block=-1), kvq.ERR_INVALID),
    (dict(hadamard_block=256), kvq.ERR_INVALID),     # does not divide head_dim
    (dict(page_size=0), kvq.ERR_INVALID),
    (dict(page_size=24), kvq.ERR_INVALID),           # not a multiple of 16
    (dict(head_dim=64, group_size=32, hadamard_block=64), kvq.ERR_UNSUPPORTED),
    (dict(k_codes=0), kvq.ERR_INVALID),
    (dict(v_meta=FAKE + 4), kvq.ERR_INVALID),        # misaligned plane
    (dict(quant_mode=2), kvq.ERR_INVALID),            # neither asymmetric nor hybrid
    (dict(v_grouping=2), kvq.ERR_INVALID),
    (dict(v_grouping=1, page_size=16), kvq.ERR_INVALID),   # token groups of 32 do not fit a page
    (dict(quant_mode=-1), kvq.ERR_INVALID),
]


@pytest.mark.parametrize("kw,status", INVALID_CACHES)
def test_append_rejects_bad_cache(kw, status):
    d = _desc(**kw)
    st = kvq.lib().kvq_quantize_append(ctypes.byref(d), ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE),
                                       ctypes.c_void_p(FAKE), 4, None)
    assert st == status


def test_append_argument_checks():
    d = _desc()
    L = kvq.lib()
    v = ctypes.c_void_p
    assert L.kvq_quantize_append(None, v(FAKE), v(FAKE), v(FAKE), 1, None) == kvq.ERR_INVALID
    assert L.kvq_quantize_append(ctypes.byref(d), v(FAKE), v(FAKE), v(FAKE), -1, None) == kvq.ERR_INVALID
    assert L.kvq_quantize_append(ctypes.byref(d), None, v(FAKE), v(FAKE), 1, None) == kvq.ERR_INVALID
    assert L.kvq_quantize_append(ctypes.byref(d), v(FAKE + 2), v(FAKE), v(FAKE), 1, None) == kvq.ERR_INVALID
    assert L.kvq_quantize_append(ctypes.byref(d), v(FAKE), v(FAKE), v(FAKE + 4), 1, None) == kvq.ERR_INVALID
    assert L.kvq_quantize_append(ctypes.byref(d), None, None, None, 0, None) == kvq.OK  # empty: no launch


def _decode(d, **kw):
    a = dict(q=FAKE, batch=2, hq=32, bt=FAKE, maxp=64, lens=FAKE, maxlen=1000, scale=0.0, splits=0, ws=FAKE,
             wsb=1 << 40, out=FAKE)
    a.update(kw)
    v = ctypes.c_void_p
    return kvq.lib().kvq_decode_attention(ctypes.byref(d) if d is not None else None, v(a["q"]), a["batch"],
                                          a["hq"], v(a["bt"]), a["maxp"], v(a["lens"]), a["maxlen"], a["scale"],
                                          a["splits"], v(a["ws"]), a["wsb"], v(a["out"]), None)


@pytest.mark.parametrize("kw,status", [
    (dict(hq=12), kvq.ERR_INVALID),          # not a multiple of Hkv
    (dict(hq=64), kvq.ERR_UNSUPPORTED),      # GQA ratio 8
    (dict(batch=-1), kvq.ERR_INVALID),
    (dict(maxlen=-5), kvq.ERR_INVALID),
    (dict(splits=-1), kvq.ERR_INVALID),
    (dict(maxp=0), kvq.ERR_INVALID),
    (dict(maxp=10), kvq.ERR_INVALID),        # 10 pages * 16 < 1000 tokens
    (dict(q=0), kvq.ERR_INVALID),
    (dict(q=FAKE + 8), kvq.ERR_INVALID),
    (dict(bt=0), kvq.ERR_INVALID),
    (dict(lens=FAKE + 2), kvq.ERR_INVALID),
    (dict(out=FAKE + 4), kvq.ERR_INVALID),
    (dict(ws=0), kvq.ERR_INVALID),
    (dict(wsb=100), kvq.ERR_WORKSPACE),      # too small: rejected before launch
])
def test_decode_argument_checks(kw, status):
    assert _decode(_desc(), **kw) == status


def test_decode_bad_cache_and_empty_batch():
    assert _decode(None) == kvq.ERR_INVALID
    assert _decode(_desc(bits=3)) == kvq.ERR_UNSUPPORTED
    assert _decode(_desc(), batch=0) == kvq.OK  # empty: no launch


def _step(d, **kw):
    a = dict(k=FAKE, v=FAKE, q=FAKE, batch=2, hq=32, bt=FAKE, maxp=64, lens=FAKE, maxlen=1000, scale=0.0,
             splits=0, ws=FAKE, wsb=1 << 40, out=FAKE)
    a.update(kw)
    v = ctypes.c_void_p
    return kvq.lib().kvq_decode_step(ctypes.byref(d) if d is not None else None, v(a["k"]), v(a["v"]), v(a["q"]),
                                     a["batch"], a["hq"], v(a["bt"]), a["maxp"], v(a["lens"]), a["maxlen"],
                                     a["scale"], a["splits"], v(a["ws"]), a["wsb"], v(a["out"]), None)


@pytest.mark.parametrize("kw,status", [
    (dict(k=0), kvq.ERR_INVALID),
    (dict(v=0), kvq.ERR_INVALID),
    (dict(k=FAKE + 2), kvq.ERR_INVALID),     # rows are read 16 bytes at a time
    (dict(v=FAKE + 8), kvq.ERR_INVALID),
    (dict(hq=12), kvq.ERR_INVALID),          # the decode checks apply as they are
    (dict(hq=64), kvq.ERR_UNSUPPORTED),
    (dict(q=FAKE + 8), kvq.ERR_INVALID),
    (dict(wsb=100), kvq.ERR_WORKSPACE),
])
def test_decode_step_argument_checks(kw, status):
    assert _step(_desc(), **kw) == status


def test_decode_step_cache_kinds():
    assert _step(None) == kvq.ERR_INVALID
    # value token groups append a whole group at a time: no fused single-token step
    assert _step(_desc(v_grouping=1, page_size=32)) == kvq.ERR_UNSUPPORTED
    assert _step(_desc(), batch=0) == kvq.OK  # empty: no launch
    assert _step(_desc(quant_mode=1), batch=0) == kvq.OK


def test_dequantize_argument_checks():
    d = _desc()
    L = kvq.lib()
    v = ctypes.c_void_p
    assert L.kvq_dequantize(ctypes.byref(d), 2, v(FAKE), 4, v(FAKE), None) == kvq.ERR_INVALID
    assert L.kvq_dequantize(ctypes.byref(d), 0, v(FAKE), -1, v(FAKE), None) == kvq.ERR_INVALID
    assert L.kvq_dequantize(ctypes.byref(d), 0, v(FAKE + 4), 4, v(FAKE), None) == kvq.ERR_INVALID
    assert L.kvq_dequantize(ctypes.byref(d), 1, v(FAKE), 4, v(FAKE + 8), None) == kvq.ERR_INVALID
    assert L.kvq_dequantize(ctypes.byref(d), 1, None, 0, None, None) == kvq.OK


def _balanced_table(B):
    """Bytes of the balanced layout's per-sequence table (two int32 per sequence, in
    whole 256-byte blocks) after its partials."""
    return -(-8 * B // 256) * 256


def _balanced_slots(B, T, cus=256, hkv=8):
    """Units per kv head the balanced plan's grid holds, in 256-token units C = B *
    ceil(T / 256): at most C / k + B partitions, C / k <= 8 * CUs / Hkv (one round of
    waves) unless k is held at 64; at most C."""
    uph = -(-8 * cus // hkv)
    C = B * -(-max(T, 1) // 256)
    return min(C, max(uph, -(-C // 64)) + B)


def test_split_sizing_and_workspace():
    """Automatic split-K sizing. The matrix kernel's partitions are balanced: one length
    for the batch in whole 256-token units, as long as it takes for the partitions to fit
    one round of waves (8 per CU over the kv heads; reported for a batch of max_seq_len
    sequences); its workspace is [Hq][units per kv head][d+2] fp32. The reference kernel
    keeps fixed partitions of at most 2048 tokens, workspace [B][Hq][S][d+2]; the automatic
    size covers both. (Off a GPU the library assumes 256 compute units, the MI355X count.)"""
    L = kvq.lib()
    d = _desc(page_size=32768, num_pages=64)
    cases = {  # (B, T) -> (matrix splits, reference splits)
        (64, 32768): (4, 16),   # 8192-token partitions: 2048 units, one round (reference: 2048 tokens)
        (16, 8192): (16, 32),   # 512-token partitions (reference: 256)
        (1, 1024): (4, 4),      # one sequence: fixed partitions, at least 256 tokens
        (3, 5000): (20, 18),    # 256-token partitions (9 blocks for the reference)
        (48, 32768): (5, 16),   # k = 24 gives 48 * 6 partitions > 256: k = 26, 6656 tokens
    }
    for (B, T), (want, want_ref) in cases.items():
        assert L.kvq_decode_num_splits(ctypes.byref(d), B, 32, T, 0) == want
        # a batch of one takes fixed partitions (nothing to balance)
        mine = 32 * _balanced_slots(B, T) * 130 * 4 + _balanced_table(B) if B > 1 else B * 32 * want * 130 * 4
        assert L.kvq_decode_workspace_bytes(ctypes.byref(d), B, 32, T, 0) == max(mine, B * 32 * want_ref * 130 * 4)
    # an explicit count: fixed partitions for both kernels
    assert L.kvq_decode_workspace_bytes(ctypes.byref(d), 4, 32, 8192, 6) == 4 * 32 * 6 * 130 * 4
    # past 256 sequences the plan would cost every workgroup too much: fixed partitions
    # (matrix kernel: one 2048-token partition per sequence, 2400 units already fill a
    # round; reference kernel: two of 1024; the workspace covers the larger)
    assert L.kvq_decode_num_splits(ctypes.byref(d), 300, 32, 2048, 0) == 1
    assert L.kvq_decode_workspace_bytes(ctypes.byref(d), 300, 32, 2048, 0) == 300 * 32 * 2 * 130 * 4
    d3 = _desc(group_size=64, page_size=131072, num_pages=1)
    assert L.kvq_decode_num_splits(ctypes.byref(d3), 1, 32, 131072, 0) >= 256
    # explicit requests are honoured up to one partition per 32-token block
    assert L.kvq_decode_num_splits(ctypes.byref(d), 1, 32, 1000, 7) == 7
    assert L.kvq_decode_num_splits(ctypes.byref(d), 1, 32, 100, 50) == 4
    assert L.kvq_decode_workspace_bytes(ctypes.byref(_desc(bits=3)), 1, 32, 100, 0) == 0


def _plan_partitions(lens, cus=256, hkv=8):
    """The balanced plan written out (decode over the whole span, no windows): spans in
    256-token units c_b, k from ceil(C / U) up until sum ceil(c_b / k) <= U (U = one round
    of waves per kv head, k at most 64); ceil(c_b / k) partitions per sequence."""
    uph = -(-8 * cus // hkv)
    c = [-(-max(int(t), 0) // 256) for t in lens]
    C = sum(c)
    count = lambda k: sum(-(-x // k) for x in c)
    k = 64 if C >= 64 * uph else (-(-C // uph) if C > uph else 1)
    while k < 64 and count(k) > uph:
        k += 1
    return k, count(k)


def test_balanced_plan_fits_the_grid():
    """Whatever the lengths (all <= max_seq_len), the plan's partitions per kv head never
    exceed the units the grid and the workspace provide (the workspace size is
    Hq * U * 130 * 4 bytes, U the bound), so no partition is dropped; for a uniform batch
    the reported split count is the plan's."""
    import random
    L = kvq.lib()
    d = _desc(page_size=65536, num_pages=4096)
    rnd = random.Random(7)
    for trial in range(400):
        B = rnd.choice([2, 3, 16, 63, 64, 65, 130, 256])
        maxlen = rnd.choice([1, 255, 256, 257, 4096, 8191, 32768, 65536, 200000])
        kind = trial % 4
        if kind == 0:
            lens = [maxlen] * B
        elif kind == 1:
            lens = [rnd.randint(0, maxlen) for _ in range(B)]
        elif kind == 2:  # one long, the rest tiny
            lens = [maxlen] + [rnd.randint(0, 3) for _ in range(B - 1)]
        else:  # most at the maximum, a few empty
            lens = [maxlen if rnd.random() < 0.8 else 0 for _ in range(B)]
        ws = L.kvq_decode_workspace_bytes(ctypes.byref(d), B, 32, maxlen, 0)
        ref = L.kvq_decode_num_splits(ctypes.byref(d), B, 32, maxlen, 0)
        U = _balanced_slots(B, maxlen)
        assert ws >= 32 * U * 130 * 4 + _balanced_table(B)
        k, n = _plan_partitions(lens)
        assert n <= U, (B, maxlen, kind, k, n, U)
        if kind == 0:
            assert ref == -(-(-(-maxlen // 256)) // k)


def test_page_index_limit():
    """The decode kernels index a page's rows of one kv head as page * Hkv + head in 32
    bits: a pool whose num_pages * Hkv passes 2^32 is reported unsupported before any
    launch (the device pointers here are never touched)."""
    L, v = kvq.lib(), ctypes.c_void_p
    big = _desc(num_pages=(1 << 29) + 1)  # x 8 kv heads > 2^32
    ok = _desc(num_pages=(1 << 29) - 1)
    args = [v(FAKE), 2, 32, v(FAKE), 4, v(FAKE), 64, 0.0, 0, v(FAKE), 1 << 40, v(FAKE), None]
    assert L.kvq_decode_attention(ctypes.byref(big), *args) == kvq.ERR_UNSUPPORTED
    assert L.kvq_decode_workspace_bytes(ctypes.byref(ok), 2, 32, 64, 0) > 0


def test_tile_index_limit():
    """The paged decode loads index a kv head's 16-token tiles as (page * Hkv + head) *
    page_size / 16 + offset / 16 in 32 bits: a pool of 2^32 tiles or more is reported
    unsupported before any launch, one tile fewer is accepted."""
    L, v = kvq.lib(), ctypes.c_void_p
    args = [v(FAKE), 2, 32, v(FAKE), 4, v(FAKE), 64, 0.0, 0, v(FAKE), 1 << 40, v(FAKE), None]
    for page in (64, 256):
        pages_at_limit = (1 << 32) // (8 * page // 16)  # x 8 kv heads x page / 16 tiles = 2^32
        big = _desc(page_size=page, num_pages=pages_at_limit)
        ok = _desc(page_size=page, num_pages=pages_at_limit - 1)
        assert L.kvq_decode_attention(ctypes.byref(big), *args) == kvq.ERR_UNSUPPORTED, page
        assert L.kvq_decode_workspace_bytes(ctypes.byref(big), 2, 32, 64, 0) == 0, page
        assert L.kvq_decode_workspace_bytes(ctypes.byref(ok), 2, 32, 64, 0) > 0, page


def _win(**kw):
    base = dict(sink=32, recent=128, batch=4, k=FAKE, v=FAKE, residual=0)
    base.update(kw)
    return kvq._Window(base["sink"], base["recent"], base["batch"], base["k"], base["v"], base.get("residual", 0))


@pytest.mark.parametrize("kw,status", [
    (dict(recent=0), kvq.ERR_INVALID),
    (dict(sink=-16), kvq.ERR_INVALID),
    (dict(batch=-1), kvq.ERR_INVALID),
    (dict(sink=8), kvq.ERR_UNSUPPORTED),          # not on a 16-token tile boundary
    (dict(sink=512, recent=513), kvq.ERR_UNSUPPORTED),  # more than 1024 window rows
    (dict(k=0), kvq.ERR_INVALID),
    (dict(v=FAKE + 2), kvq.ERR_INVALID),
])
def test_window_append_rejects_bad_window(kw, status):
    v = ctypes.c_void_p
    st = kvq.lib().kvq_window_append(ctypes.byref(_desc()), ctypes.byref(_win(**kw)), v(FAKE), v(FAKE), v(FAKE),
                                     v(FAKE), v(FAKE), 2, None)
    assert st == status


def test_window_append_argument_checks():
    L, v = kvq.lib(), ctypes.c_void_p
    d, w = ctypes.byref(_desc()), ctypes.byref(_win())
    args = [v(FAKE)] * 5
    assert L.kvq_window_append(None, w, *args, 1, None) == kvq.ERR_INVALID
    assert L.kvq_window_append(d, None, *args, 1, None) == kvq.ERR_INVALID
    assert L.kvq_window_append(d, w, *args, -1, None) == kvq.ERR_INVALID
    assert L.kvq_window_append(d, w, *args, 5, None) == kvq.ERR_INVALID   # more rows than sequences
    for i, bad in ((0, FAKE + 2), (2, FAKE + 2), (3, 0), (4, FAKE + 4)):
        a = list(args)
        a[i] = v(bad)
        assert L.kvq_window_append(d, w, *a, 1, None) == kvq.ERR_INVALID, i
    assert L.kvq_window_append(ctypes.byref(_desc(bits=3)), w, *args, 1, None) == kvq.ERR_UNSUPPORTED
    assert L.kvq_window_append(d, w, None, None, None, None, None, 0, None) == kvq.OK  # empty: no launch


def test_window_sizes():
    L = kvq.lib()
    d = _desc(page_size=32768, num_pages=64)
    w = _win(sink=64, recent=64, batch=3)
    assert L.kvq_window_plane_bytes(ctypes.byref(d), ctypes.byref(w)) == 3 * 128 * 8 * 128 * 2
    assert L.kvq_window_plane_bytes(ctypes.byref(d), ctypes.byref(_win(recent=0))) == -1
    # the split count follows the quantized span (max_seq_len - sink - recent), plus one
    # window partial per (sequence, query head)
    for B, T in ((64, 32768), (3, 5000), (2, 100)):
        span = max(T - 128, 0)
        slots = _balanced_slots(B, span)
        assert L.kvq_decode_window_workspace_bytes(ctypes.byref(d), ctypes.byref(w), B, 32, T, 0) == \
            (32 * slots + B * 32) * 130 * 4 + _balanced_table(B)
        s = L.kvq_decode_num_splits(ctypes.byref(d), B, 32, span, 5)
        assert L.kvq_decode_window_workspace_bytes(ctypes.byref(d), ctypes.byref(w), B, 32, T, 5) == \
            B * 32 * (s + 1) * 130 * 4
    # a batch of one: fixed partitions
    s = L.kvq_decode_num_splits(ctypes.byref(d), 1, 32, 5000 - 128, 0)
    assert L.kvq_decode_window_workspace_bytes(ctypes.byref(d), ctypes.byref(w), 1, 32, 5000, 0) == \
        32 * (s + 1) * 130 * 4
    assert L.kvq_decode_window_workspace_bytes(ctypes.byref(d), ctypes.byref(_win(sink=8)), 1, 32, 100, 0) == 0


def _decode_window(d, w, **kw):
    a = dict(q=FAKE, batch=2, hq=32, bt=FAKE, maxp=64, lens=FAKE, maxlen=1000, scale=0.0, splits=0, ws=FAKE,
             wsb=1 << 40, out=FAKE)
    a.update(kw)
    v = ctypes.c_void_p
    return kvq.lib().kvq_decode_attention_window(
        ctypes.byref(d) if d is not None else None, ctypes.byref(w) if w is not None else None, v(a["q"]),
        a["batch"], a["hq"], v(a["bt"]), a["maxp"], v(a["lens"]), a["maxlen"], a["scale"], a["splits"], v(a["ws"]),
        a["wsb"], v(a["out"]), None)


def test_decode_window_argument_checks():
    d, w = _desc(), _win()
    assert _decode_window(None, w) == kvq.ERR_INVALID
    assert _decode_window(d, None) == kvq.ERR_INVALID
    assert _decode_window(d, _win(recent=0)) == kvq.ERR_INVALID
    assert _decode_window(d, _win(sink=24)) == kvq.ERR_UNSUPPORTED
    assert _decode_window(d, w, batch=5) == kvq.ERR_INVALID      # more sequences than window rows
    assert _decode_window(d, w, hq=64) == kvq.ERR_UNSUPPORTED
    assert _decode_window(d, w, q=FAKE + 8) == kvq.ERR_INVALID
    assert _decode_window(d, w, wsb=100) == kvq.ERR_WORKSPACE
    assert _decode_window(d, w, batch=0) == kvq.OK  # empty: no launch


def _decode_pruned(d, **kw):
    a = dict(q=FAKE, batch=2, hq=32, bt=FAKE, maxp=64, lens=FAKE, maxlen=1000, scale=0.0, splits=0, keep=3,
             mask=FAKE, ws=FAKE, wsb=1 << 40, out=FAKE)
    a.update(kw)
    v = ctypes.c_void_p
    return kvq.lib().kvq_decode_attention_pruned(
        ctypes.byref(d), v(a["q"]), a["batch"], a["hq"], v(a["bt"]), a["maxp"], v(a["lens"]), a["maxlen"],
        a["scale"], a["splits"], a["keep"], v(a["mask"]), v(a["ws"]), a["wsb"], v(a["out"]), None, None, None)


def test_decode_pruned_argument_checks():
    d4, d2 = _desc(), _desc(bits=2, group_size=128)
    assert _decode_pruned(d4, keep=0) == kvq.ERR_INVALID
    assert _decode_pruned(d4, keep=5) == kvq.ERR_INVALID    # INT4 rows have 4 chunks
    assert _decode_pruned(d2, keep=3) == kvq.ERR_INVALID    # INT2 rows have 2 chunks
    assert _decode_pruned(d4, mask=FAKE + 2) == kvq.ERR_INVALID
    assert _decode_pruned(d4, q=FAKE + 8) == kvq.ERR_INVALID
    assert _decode_pruned(d4, wsb=100) == kvq.ERR_WORKSPACE
    assert _decode_pruned(d4, batch=0) == kvq.OK            # empty: no launch
    assert _decode_pruned(d2, keep=2, batch=0, mask=0) == kvq.OK


def test_vgroup_argument_checks():
    """Value token groups: appends of whole groups only; windows must be a residual of one
    group; the pruned kernel does not take them."""
    L, v = kvq.lib(), ctypes.c_void_p
    d = _desc(v_grouping=1, page_size=64)
    assert L.kvq_quantize_append(ctypes.byref(d), v(FAKE), v(FAKE), v(FAKE), 33, None) == kvq.ERR_INVALID
    assert L.kvq_quantize_append(ctypes.byref(d), v(FAKE), v(FAKE), v(FAKE), 0, None) == kvq.OK
    args = [v(FAKE)] * 5
    assert L.kvq_window_append(ctypes.byref(d), ctypes.byref(_win()), *args, 1, None) == kvq.ERR_UNSUPPORTED
    assert L.kvq_window_append(ctypes.byref(d), ctypes.byref(_win(sink=0, recent=64, residual=1)), *args, 1,
                               None) == kvq.ERR_UNSUPPORTED  # ring of 64 rows, groups of 32
    assert L.kvq_window_append(ctypes.byref(d), ctypes.byref(_win(sink=0, recent=32, residual=1)), *args, 0,
                               None) == kvq.OK
    assert L.kvq_window_append(ctypes.byref(_desc()), ctypes.byref(_win(sink=16, residual=1)), *args, 1,
                               None) == kvq.ERR_INVALID  # a residual has no sink
    assert L.kvq_window_append(ctypes.byref(_desc()), ctypes.byref(_win(residual=2)), *args, 1, None) == kvq.ERR_INVALID
    assert L.kvq_window_append(ctypes.byref(_desc(page_size=16)), ctypes.byref(_win(sink=0, recent=32, residual=1)),
                               *args, 1, None) == kvq.ERR_INVALID  # a group would cross pages
    assert _decode_pruned(d) == kvq.ERR_UNSUPPORTED


def test_stream_read_argument_checks():
    """The read probe rejects misaligned or odd-sized buffers and out-of-range settings
    before any launch; an empty read launches nothing."""
    L, v = kvq.lib(), ctypes.c_void_p

    def call(src=FAKE, nbytes=1 << 20, sink=FAKE, nt=1, wpc=8):
        return L.kvq_stream_read(v(src), nbytes, v(sink), nt, wpc, None, None, None)

    assert call(src=0) == kvq.ERR_INVALID
    assert call(src=FAKE + 4) == kvq.ERR_INVALID
    assert call(nbytes=(1 << 20) + 8) == kvq.ERR_INVALID
    assert call(sink=0) == kvq.ERR_INVALID
    assert call(sink=FAKE + 2) == kvq.ERR_INVALID
    assert call(nt=2) == kvq.ERR_INVALID
    assert call(wpc=0) == kvq.ERR_INVALID
    assert call(wpc=33) == kvq.ERR_INVALID
    assert call(nbytes=0) == kvq.OK


def test_size_limits():
    """Sizes past the documented limits are refused, never wrapped: a context beyond 2^30
    tokens is unsupported, and workspace sizes that do not fit in size_t are reported as 0
    (invalid) rather than as a small wrapped number."""
    L = kvq.lib()
    d = _desc(num_pages=1 << 20)
    assert L.kvq_decode_workspace_bytes(ctypes.byref(d), 4, 32, (1 << 30) + 1, 0) == 0
    assert L.kvq_decode_num_splits(ctypes.byref(d), 4, 32, (1 << 30) + 1, 0) == 0
    assert _decode(d, maxlen=(1 << 30) + 1, maxp=1 << 20) == kvq.ERR_UNSUPPORTED
    # batch * heads * splits * 520 B beyond 2^64
    big = L.kvq_decode_workspace_bytes(ctypes.byref(d), 2 ** 31 - 1, 32, 1 << 30, 2 ** 31 - 1)
    assert big == 0
    assert _decode(d, batch=2 ** 31 - 1, hq=32, maxlen=1 << 30, splits=2 ** 31 - 1, maxp=1 << 20,
                   wsb=2 ** 64 - 1) == kvq.ERR_INVALID
    # pools whose page count overflows int64 products
    huge = _desc(num_pages=2 ** 62)
    assert L.kvq_cache_plane_bytes(ctypes.byref(huge), 0) == -1
    w = kvq._Window(16, 128, 2 ** 31 - 1, FAKE, FAKE, 0)
    assert L.kvq_window_plane_bytes(ctypes.byref(_desc(num_kv_heads=2 ** 31 - 1, num_pages=1)), ctypes.byref(w)) == -1
