"""GPU path (through the C ABI) against the oracle on the same seeded inputs.

Bar: quantized codes and fp16 scale/zero bit-exact (every byte of all four cache
planes); dequantized rows bit-exact; attention output within 2e-3 max-abs of the
fp64 oracle. Shapes are scaled-down versions of the workloads (same head counts,
group sizes, outlier structure, paging) that span several 16/32-token tiles and end
on ragged tails; full-size shapes are sampled in test_gpu_fullsize.py.
"""
import numpy as np
import pytest
import torch

import bit_kv_cache_quantize_amd as kvq
import oracle
import workloads as wl
from kvq_harness import TOL, EventPair, append_step, decode_both, make_pair, max_err, planes_equal, record

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _small(name, **kw):
    return wl.get(name).with_(**kw)


APPEND_CASES = {
    "c1": _small("c1"),
    "c2_small": _small("c2", batch=3, context=700),
    "c3_g64_sink": _small("c3", context=1000),
    "c4_int2_g128": _small("c4", batch=2, context=333),
    "c5_paged": _small("c5", batch=5, ragged=(1, 300)),
    "int4_g128": _small("c2", batch=2, context=257, group_size=128),
    "int2_g32": _small("c2", batch=2, context=129, bits=2, group_size=32),
    "int2_g64_hb32": _small("c2", batch=2, context=95, bits=2, group_size=64, hadamard_block=32),
    "int4_g32_no_rotation": _small("c2", batch=2, context=200, hadamard_block=0),
    "int4_g32_hb64": _small("c2", batch=2, context=64, hadamard_block=64),
    "int4_g64_hb16": _small("c2", batch=1, context=48, group_size=64, hadamard_block=16),
    "int4_g32_hb2": _small("c2", batch=1, context=40, hadamard_block=2),
    "int4_g32_hb4": _small("c2", batch=2, context=77, hadamard_block=4),
    "int2_g128_hb8": _small("c4", batch=2, context=83, hadamard_block=8),
    "int4_g64_hb8_paged": _small("c5", batch=3, ragged=(20, 90), group_size=64, hadamard_block=8),
}


@pytest.mark.parametrize("name", list(APPEND_CASES))
def test_append_bit_exact(name):
    w = APPEND_CASES[name]
    print(f"[append] {name}: {w}", flush=True)
    p = make_pair(w, DEV, extra_tokens=2)
    append_step(p, 0, DEV)
    torch.cuda.synchronize()
    assert planes_equal(p) == []


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)


def test_append_edge_values_bit_exact():
    """Rows that stress the formula: constant groups, mixed-sign zeros, huge offsets with
    tiny ranges, fp16-subnormal scales, values near the fp16 range, one-hot outliers."""
    print("[append] edge values", flush=True)
    rng = np.random.default_rng(21)
    rows = []
    rows.append(np.full(128, 1.25))
    rows.append(np.zeros(128))
    z = np.zeros(128)
    z[::3] = -0.0
    rows.append(z)
    rows.append(-np.zeros(128))
    rows.append(1000.1 + rng.random(128) * 0.9)
    rows.append(-3.3e4 + rng.random(128) * 0.5)
    rows.append(rng.standard_normal(128) * 1e-6)       # scale in the fp16 subnormal range
    rows.append(rng.standard_normal(128) * 1e-9)       # scale rounds to 0
    rows.append(rng.standard_normal(128) * 3000.0)     # large but finite scales
    oh = np.zeros(128)
    oh[37] = 50.0
    rows.append(oh)
    rows.append(np.tile([0.5, 1.5, 2.5, 3.5], 32))     # rounding ties
    rows.append(np.arange(128) % 16)
    while len(rows) % 4:
        rows.append(rng.standard_normal(128))
    x = np.stack(rows).reshape(-1, 2, 128)             # [n][Hkv=2][d]
    n = x.shape[0]
    for bits, G, hb, mode in ((4, 32, 128, 0), (2, 128, 128, 0), (4, 64, 0, 0), (2, 32, 64, 0),
                              (4, 32, 128, 1), (2, 32, 0, 1), (4, 128, 0, 1)):
        w = wl.Workload("edge", 1, 2, 2, 128, 32, bits, G, hb)
        geo = wl.geometry(w)
        gpu = kvq.KVCache.allocate(128, 2, bits, G, hb, geo.page_size, geo.num_pages, device=DEV, quant_mode=mode)
        ref = oracle.Cache(128, 2, bits, G, hb, geo.page_size, geo.num_pages, quant_mode=mode)
        k = _bf16(x)
        v = _bf16(x[::-1].copy())
        slots = torch.arange(n, dtype=torch.int64)
        kvq.quantize_append(gpu, k.to(DEV), v.to(DEV), slots.to(DEV))
        ref.append(wl.bf16_bits(k), wl.bf16_bits(v), slots.numpy())
        torch.cuda.synchronize()
        for g, r in zip(gpu.planes(), ref.planes()):
            assert np.array_equal(g.cpu().numpy(), r), (bits, G, hb, mode)


@pytest.mark.parametrize("name", ["c1", "c4_int2_g128", "c5_paged", "int2_g64_hb32"])
def test_dequantize_bit_exact(name):
    w = APPEND_CASES[name]
    print(f"[dequantize] {name}", flush=True)
    p = make_pair(w, DEV)
    slots = torch.cat([p.geo.slots(b, 0, int(p.lens[b])) for b in range(w.batch)])
    for which in (0, 1):
        got = kvq.dequantize(p.gpu, which, slots.to(DEV)).cpu().numpy()
        want = p.ref.dequantize(which, slots.numpy())
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), which


DECODE_CASES = {
    "c1": _small("c1"),
    "c2_small": _small("c2", batch=3, context=700),
    "c3_sink_many_splits": _small("c3", context=4100),
    "c4_int2": _small("c4", batch=3, context=1000),
    "c5_paged_ragged": _small("c5", batch=6, ragged=(1, 600)),
    "gqa1": _small("c2", batch=2, num_q_heads=8, context=333),
    "gqa2": _small("c2", batch=2, num_q_heads=16, context=333),
    "int4_g128_hb0": _small("c2", batch=2, context=257, group_size=128, hadamard_block=0),
    "int2_g32_hb32": _small("c2", batch=2, context=190, bits=2, group_size=32, hadamard_block=32),
    # 48-token pages: a 32-token block's second tile often starts on the next page
    "paged48": _small("c5", batch=4, ragged=(40, 900), page_size=48),
    # pages of 17 and 256 tiles: partitions cross page boundaries at other tile offsets
    "paged272": _small("c5", batch=4, ragged=(300, 3000), page_size=272),
    "paged4096": _small("c5", batch=3, ragged=(3000, 9000), page_size=4096),
    "paged16_int2_g32": _small("c5", batch=4, ragged=(30, 700), bits=2, group_size=32),
}


PAGE_SWEEP = [32, 80, 112, 144, 496, 1008, 2032]


@pytest.mark.parametrize("page", PAGE_SWEEP)
def test_decode_page_size_sweep(page):
    """Page sizes of 2..127 tiles (the paged table walk divides tile offsets by the tiles
    per page with a rounded reciprocal and one correction): one partition per sequence and
    the balanced plan, INT4 g32 and INT2 g128 on alternate sizes, against the oracle."""
    bits, G = (4, 32) if PAGE_SWEEP.index(page) % 2 == 0 else (2, 128)
    w = _small("c5", batch=3, ragged=(900, 4100), page_size=page, bits=bits, group_size=G, seed=page)
    print(f"[decode] page sweep {page} INT{bits} g{G}", flush=True)
    p = make_pair(w, DEV)
    for ns in (1, 0):
        got, want = decode_both(p, DEV, num_splits=ns)
        err = max_err(got, want)
        record(f"decode_page_sweep/p{page}/splits={ns}", err)
        assert np.all(np.isfinite(got))
        assert err <= TOL, (page, ns, err)


LONG_PAGED_CASES = {f"p{page}_int{b}_splits{ns}": (page, b, ns)
                    for page in (16, 48, 80) for b in (4, 2) for ns in (1, 2)}


@pytest.mark.parametrize("name", list(LONG_PAGED_CASES))
def test_decode_long_partitions_over_many_pages(name):
    """Partitions spanning far more than the 64 block-table entries a wave keeps at a time
    (one or two partitions per sequence of 3000-5200 tokens in 16-, 48- and 80-token
    pages): the window of entries is refilled inside a partition, at every tile offset a
    super-block can start on."""
    page, bits, ns = LONG_PAGED_CASES[name]
    w = _small("c5", batch=2, ragged=(3000, 5200), page_size=page, bits=bits, group_size=32, seed=page + bits)
    print(f"[decode] long paged partitions {name}", flush=True)
    p = make_pair(w, DEV)
    got, want = decode_both(p, DEV, num_splits=ns)
    err = max_err(got, want)
    record(f"decode_long_paged/{name}", err)
    assert np.all(np.isfinite(got))
    assert err <= TOL


@pytest.mark.parametrize("reference", [False, True], ids=["mfma", "reference"])
@pytest.mark.parametrize("name", list(DECODE_CASES))
def test_decode_matches_oracle(name, reference):
    w = DECODE_CASES[name]
    print(f"[decode] {name} reference={reference}", flush=True)
    p = make_pair(w, DEV, extra_tokens=1)
    append_step(p, 0, DEV)
    got, want = decode_both(p, DEV, reference=reference)
    assert np.all(np.isfinite(got))
    err = max_err(got, want)
    print(f"  max-abs err {err:.3e}", flush=True)
    record(f"decode/{name}/{'reference' if reference else 'mfma'}", err)
    assert err <= TOL


def _hb_case(hb, bits, G, gqa, paged):
    """Block-diagonal rotation below head_dim (SAW-INT4, Abstract: block-diagonal
    Hadamard rotation): the decode prologue runs only the butterfly stages inside the
    block, so every block size is its own code path."""
    base = "c4" if bits == 2 else "c2"
    kw = dict(hadamard_block=hb, bits=bits, group_size=G, num_q_heads=8 * gqa, seed=hb + 7 * bits + gqa)
    if paged:
        return _small("c5", batch=4, ragged=(50, 420), **kw)
    return _small(base, batch=2, context=301, **kw)


HB_DECODE_CASES = {f"hb{hb}_int{b}_g{G}_gqa{r}": (hb, b, G, r, False)
                   for hb in (2, 4, 8, 16, 64) for (b, G) in ((4, 32), (2, 128)) for r in (4, 1)}
HB_DECODE_CASES.update({"hb8_int4_g32_gqa4_paged": (8, 4, 32, 4, True),
                        "hb64_int2_g128_gqa1_paged": (64, 2, 128, 1, True),
                        "hb16_int4_g64_gqa2_paged": (16, 4, 64, 2, True)})


@pytest.mark.parametrize("name", list(HB_DECODE_CASES))
def test_decode_hadamard_blocks(name):
    """Decode at every Hadamard block size below 128: cache bytes equal to the oracle's
    after the step's append, then the matrix-core and the plain kernels both within the
    parity bound of the fp64 oracle (whose query rotation is a dense H/sqrt(n) product)."""
    hb, bits, G, gqa, paged = HB_DECODE_CASES[name]
    w = _hb_case(hb, bits, G, gqa, paged)
    print(f"[decode] hadamard block {name}: {w}", flush=True)
    p = make_pair(w, DEV, extra_tokens=1)
    append_step(p, 0, DEV)
    torch.cuda.synchronize()
    assert planes_equal(p) == []
    for reference in (False, True):
        got, want = decode_both(p, DEV, reference=reference)
        err = max_err(got, want)
        record(f"hadamard_block/{name}/{'reference' if reference else 'mfma'}", err)
        print(f"  reference={reference} max-abs err {err:.3e}", flush=True)
        assert np.all(np.isfinite(got)) and err <= TOL


def _queries_with_magnitude(w, rng, big):
    """bf16 [B][Hq][128] queries: per head, a 32-channel block of constant sign and
    magnitude `big` (the rotation piles it into few channels, the f16 worst case) plus
    N(0,1) * big / 10 elsewhere."""
    q = rng.standard_normal((w.batch, w.num_q_heads, 128)) * (big / 10.0)
    for b in range(w.batch):
        for j in range(w.num_q_heads):
            c0 = 32 * rng.integers(0, 4)
            q[b, j, c0:c0 + 32] = big * rng.choice([-1.0, 1.0])
    return _bf16(q)


def _top2_gap(p, q, scale):
    """Smallest gap, in natural-log units, between the two largest logits of any query
    head: fp64 logits from the oracle's dequantized keys and a scipy-rotated query."""
    import scipy.linalg

    w = p.w
    hb = w.hadamard_block
    Rm = np.kron(np.eye(128 // hb), scipy.linalg.hadamard(hb) / np.sqrt(hb)) if hb else np.eye(128)
    qf = wl.bf16_bits(q).astype(np.uint32) << 16
    qf = qf.view(np.float32).astype(np.float64)
    gap = np.inf
    for b in range(w.batch):
        T = int(p.lens[b])
        k = p.ref.dequantize(0, p.geo.slots(b, 0, T).numpy()).astype(np.float64)  # [T][Hkv][d], rotated
        for j in range(w.num_q_heads):
            lg = scale * (k[:, j // w.gqa, :] @ (Rm @ qf[b, j]))
            top = np.sort(lg)[-2:]
            gap = min(gap, top[1] - top[0])
    return gap


@pytest.mark.parametrize("big,scale", [(1.0e4, 1.0), (3.0e4, 0.0), (6.0e4, 1.0), (1.0e-5, 0.0)],
                         ids=["1e4_scale1", "3e4_default", "6e4_scale1", "1e-5_default"])
def test_decode_query_magnitudes(big, scale):
    """Queries far from N(0,1): the kernel splits the rotated, scaled query into two f16
    digits after normalising each head by a power of two, so large queries (which would
    overflow f16 without it) and tiny ones (whose low digit would be an f16 subnormal)
    both match the oracle. With large queries the softmax is nearly one-hot; the test
    first checks (fp64) that no head's top two logits are within 20 units, so the
    expected output is not decided by rounding."""
    w = _small("c2", batch=2, context=300, num_q_heads=16)
    print(f"[decode] query magnitude {big:g}, softmax scale {scale:g}", flush=True)
    p = make_pair(w, DEV)
    q = _queries_with_magnitude(w, np.random.default_rng(int(big) % 1000 + 5), big)
    eff = scale if scale > 0 else 1.0 / np.sqrt(128)
    if big > 1:
        assert _top2_gap(p, q, eff) > 20.0
    for reference in (False, True):
        got, want = decode_both(p, DEV, q=q, softmax_scale=scale, reference=reference)
        err = max_err(got, want)
        record(f"query_magnitude/{big:g}/scale={scale:g}/{'reference' if reference else 'mfma'}", err)
        print(f"  reference={reference} max-abs err {err:.3e}", flush=True)
        assert np.all(np.isfinite(got)) and err <= TOL


def test_decode_zero_and_one_token_sequences():
    w = _small("c5", batch=4, ragged=(1, 100))
    print("[decode] zero/one-token sequences", flush=True)
    lens = torch.tensor([0, 1, 37, 0], dtype=torch.int32)
    p = make_pair(w, DEV, lens=lens)
    got, want = decode_both(p, DEV)
    assert np.all(got[0] == 0) and np.all(got[3] == 0)
    assert max_err(got, want) <= TOL
    # one token: the output is that token's dequantized value row for every query head
    slot = p.geo.slots(1, 0, 1)
    v0 = kvq.dequantize(p.gpu, 1, slot.to(DEV)).cpu().numpy()[0]  # [Hkv][d]
    for j in range(w.num_q_heads):
        assert np.max(np.abs(got[1, j] - v0[j // w.gqa])) <= 1e-6


# Largest deviation measured between partition counts of the case below (one full GPU
# run with KVQ_PARITY_LOG: 2.92e-6), times 4.
SPLIT_DEV_BOUND = 1.2e-5


def test_decode_split_count_independence():
    """Any partition count gives the same attention: each within the parity bound of the
    oracle, and all within SPLIT_DEV_BOUND of each other (fp32 accumulation in another
    order only; a partition-merge mistake would move outputs by far more)."""
    w = _small("c2", batch=2, context=1500)
    print("[decode] split independence", flush=True)
    p = make_pair(w, DEV)
    q = wl.queries(w)
    outs = []
    for ns in (1, 2, 7, 47, 0):
        got, want = decode_both(p, DEV, q=q, num_splits=ns)
        err = max_err(got, want)
        record(f"split_independence/oracle/splits={ns}", err)
        assert err <= TOL, ns
        outs.append(got)
    for ns, o in zip((2, 7, 47, 0), outs[1:]):
        dev = float(np.max(np.abs(o - outs[0])))
        record(f"split_independence/vs_one_split/splits={ns}", dev)
        assert dev <= SPLIT_DEV_BOUND


BALANCED_CASES = {
    # more than 64 sequences: the plan's prefix sums run over several groups of 64
    "b70_ragged_zeros": (_small("c5", batch=70, ragged=(0, 400)), None),
    "b130_short": (_small("c5", batch=130, ragged=(1, 120)), None),
    # one long sequence among short and empty ones: it takes most partitions
    "dominant": (_small("c5", batch=5, ragged=(1, 9000)), [9000, 3, 0, 40, 700]),
    # every sequence empty but one token
    "single_token": (_small("c5", batch=3, ragged=(0, 1)), [0, 1, 0]),
    # every sequence empty: no partitions at all, zero rows
    "all_empty": (_small("c5", batch=5, ragged=(0, 1)), [0, 0, 0, 0, 0]),
    # equal lengths whose partitions fill one round of waves exactly (on 256 CUs: 2 and 4
    # kv heads, 16 partitions per sequence, the last one shorter), INT4 g32 and INT2 g128
    "paired_b64_kv2": (_small("c2", batch=64, num_kv_heads=2, num_q_heads=8, context=7900), None),
    "paired_b32_kv4_int2_g128": (_small("c4", batch=32, num_kv_heads=4, num_q_heads=16, context=11982), None),
}


@pytest.mark.parametrize("name", list(BALANCED_CASES))
def test_decode_balanced_plan_ragged_batches(name):
    """Automatic partitions are planned on the device from the batch's lengths (one length
    for all sequences, each sequence's partitions found by prefix sums); the result must
    match the oracle and a fixed-partition decode of the same cache."""
    w, lens = BALANCED_CASES[name]
    lens = wl.seq_lens(w) if lens is None else torch.tensor(lens, dtype=torch.int32)
    if name == "b70_ragged_zeros":
        lens[::9] = 0
    print(f"[decode] balanced plan {name}: B={w.batch} lens sum {int(lens.sum())} max {int(lens.max())}", flush=True)
    p = make_pair(w, DEV, lens=lens)
    q = wl.queries(w)
    got, want = decode_both(p, DEV, q=q)
    err = max_err(got, want)
    record(f"balanced/{name}", err)
    print(f"  max-abs err {err:.3e}", flush=True)
    assert np.all(np.isfinite(got))
    assert err <= TOL
    assert np.all(got[lens.numpy() == 0] == 0)
    fixed, _ = decode_both(p, DEV, q=q, num_splits=3)
    dev = float(np.max(np.abs(got - fixed)))
    record(f"balanced_vs_fixed/{name}", dev)
    assert dev <= 1e-4


def test_decode_balanced_plan_random_batches():
    """Seeded random batches (2..300 sequences, lengths 0..1500 with empty ones, 16- or
    48-token pages or contiguous, INT4/INT2): the balanced plan's output equals a fixed
    partition decode of the same cache within 1e-4 (fp32 accumulation order only), and
    every third batch matches the oracle within the parity bound."""
    import random
    rnd = random.Random(11)
    for trial in range(12):
        B = rnd.choice([2, 3, 17, 64, 65, 130, 200, 300])  # 300: past the balanced cap
        hi = rnd.choice([40, 300, 1500])
        page = rnd.choice([16, 48, 0])
        bits, G = rnd.choice([(4, 32), (4, 64), (2, 128)])
        base = "c4" if bits == 2 else "c5"
        w = _small(base, batch=B, ragged=(0, hi), page_size=page, bits=bits, group_size=G, seed=100 + trial)
        lens = wl.seq_lens(w)
        lens[torch.randperm(B, generator=torch.Generator().manual_seed(trial))[: B // 7]] = 0
        with_oracle = trial % 3 == 0
        print(f"[decode] random balanced batch {trial}: B={B} max={int(lens.max())} page={page} "
              f"INT{bits} g{G} oracle={with_oracle}", flush=True)
        p = make_pair(w, DEV, lens=lens, with_oracle=with_oracle)
        q = wl.queries(w).to(DEV)
        bt, ln = p.geo.block_table.to(DEV), p.lens.to(DEV)
        maxlen = max(int(p.lens.max()), 1)
        got = kvq.decode_attention(p.gpu, q, bt, ln, maxlen).cpu().numpy().astype(np.float64)
        fixed = kvq.decode_attention(p.gpu, q, bt, ln, maxlen, num_splits=3).cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(got))
        assert np.all(got[p.lens.numpy() == 0] == 0)
        dev = float(np.max(np.abs(got - fixed)))
        record(f"balanced_vs_fixed/random{trial}", dev)
        assert dev <= 1e-4, trial
        if with_oracle:
            want = p.ref.decode(wl.bf16_bits(wl.queries(w)), p.geo.block_table.numpy(), p.lens.numpy())
            err = max_err(got, want)
            record(f"balanced/random{trial}", err)
            assert err <= TOL, (trial, err)


def test_decode_page_permutation_invariance():
    """Same logical content under two different physical page placements."""
    print("[decode] page permutation", flush=True)
    w0 = _small("c5", batch=3, ragged=(100, 300))
    outs = []
    for page_seed in (0, 5):
        # same values and lengths, only the physical page permutation differs
        w = w0.with_(page_seed=page_seed)
        lens = wl.seq_lens(w0)
        geo = wl.geometry(w, lens=lens)
        gpu = kvq.KVCache.allocate(128, 8, 4, 32, 128, 16, geo.num_pages, device=DEV)
        for b in range(w.batch):
            T = int(lens[b])
            slots = geo.slots(b, 0, T)
            kvq.quantize_append(gpu, wl.keys(w0, b, 0, T).to(DEV), wl.values(w0, b, 0, T).to(DEV), slots.to(DEV))
        out = kvq.decode_attention(gpu, wl.queries(w0).to(DEV), geo.block_table.to(DEV), lens.to(DEV),
                                   int(lens.max()))
        outs.append(out.cpu().numpy())
    assert np.array_equal(outs[0], outs[1])


def test_decode_deterministic():
    w = _small("c2", batch=2, context=900)
    print("[decode] determinism", flush=True)
    p = make_pair(w, DEV, with_oracle=False)
    q = wl.queries(w).to(DEV)
    a = kvq.decode_attention(p.gpu, q, p.geo.block_table.to(DEV), p.lens.to(DEV), 900).cpu()
    b = kvq.decode_attention(p.gpu, q, p.geo.block_table.to(DEV), p.lens.to(DEV), 900).cpu()
    assert torch.equal(a, b)



def test_decode_timed_entry_point():
    """The timed entry point gives the untimed call's exact output and records a positive
    interval around the split kernel."""
    w = _small("c2", batch=3, context=1500)
    print("[decode] timed entry point", flush=True)
    p = make_pair(w, DEV, with_oracle=False)
    q = wl.queries(w).to(DEV)
    bt, lens = p.geo.block_table.to(DEV), p.lens.to(DEV)
    plain = kvq.decode_attention(p.gpu, q, bt, lens, 1500).cpu()
    ev = EventPair()
    try:
        timed = kvq.decode_attention(p.gpu, q, bt, lens, 1500, events=ev.handles()).cpu()
        torch.cuda.synchronize()
        assert torch.equal(plain, timed)
        assert ev.elapsed_ms() > 0.0
    finally:
        ev.close()


def test_decode_custom_softmax_scale():
    w = _small("c2", batch=1, context=300)
    print("[decode] softmax scale", flush=True)
    p = make_pair(w, DEV)
    got, want = decode_both(p, DEV, softmax_scale=0.02)
    assert max_err(got, want) <= TOL


def test_sequences_longer_than_max_seq_len():
    """A sequence whose seq_lens entry exceeds max_seq_len is taken as max_seq_len long: the
    block table holds only ceil(max_seq_len / P) pages per sequence, and no kernel reads
    past that row (its own output row is undefined). The other rows match the oracle, the
    workspace and output canaries stay intact, and the fused step appends nothing for it."""
    w = _small("c5", batch=3, ragged=(1, 200))
    lens = torch.tensor([100, 100, 50], dtype=torch.int32)  # what the cache holds
    p = make_pair(w, DEV, extra_tokens=0, lens=lens)
    bt = p.geo.block_table.to(DEV)
    assert bt.shape[1] * p.geo.page_size < 150
    claimed = torch.tensor([100, 150, 50], dtype=torch.int32).to(DEV)
    q = wl.queries(w)
    want = p.ref.decode(wl.bf16_bits(q), p.geo.block_table.numpy(), lens.numpy())
    B, Hq, d = w.batch, w.num_q_heads, w.head_dim
    guard = 4096
    for name, kw in (("balanced", {}), ("fixed", {"num_splits": 2}), ("reference", {"reference": True})):
        print(f"[decode] seq_lens above max_seq_len: {name}", flush=True)
        outbuf = torch.full((B * Hq * d + 2 * guard,), 12345.0, device=DEV)
        out = outbuf[guard:guard + B * Hq * d].view(B, Hq, d)
        need = kvq.decode_workspace_bytes(p.gpu, B, Hq, 100, kw.get("num_splits", 0))
        wsbuf = torch.full((need + 2 * guard,), 0xAB, dtype=torch.uint8, device=DEV)
        kvq.decode_attention(p.gpu, q.to(DEV), bt, claimed, 100, workspace=wsbuf[guard:guard + need], out=out, **kw)
        torch.cuda.synchronize()
        assert torch.all(outbuf[:guard] == 12345.0) and torch.all(outbuf[-guard:] == 12345.0)
        assert torch.all(wsbuf[:guard] == 0xAB) and torch.all(wsbuf[-guard:] == 0xAB)
        got = out.cpu().numpy().astype(np.float64)
        assert max_err(got[[0, 2]], want[[0, 2]]) <= TOL, name
    print("[decode] seq_lens above max_seq_len: fused step", flush=True)
    before = [t.clone() for t in p.gpu.planes()]
    k, v = wl.new_tokens(w, 0)
    kvq.decode_step(p.gpu, k.to(DEV), v.to(DEV), q.to(DEV), bt, torch.tensor([101, 150, 51], dtype=torch.int32).to(DEV),
                    100)
    torch.cuda.synchronize()
    # sequence 0 (101 > 100) and sequence 1 (150) append nothing; sequence 2 writes position 50
    slot2 = int(p.geo.slots(2, 50, 1)[0])
    twin = p.gpu.clone()
    for t, b0 in zip(twin.planes(), before):
        t.copy_(b0)
    kvq.quantize_append(twin, k[2:3].to(DEV), v[2:3].to(DEV), torch.tensor([slot2], dtype=torch.int64, device=DEV))
    torch.cuda.synchronize()
    for a, b in zip(p.gpu.planes(), twin.planes()):
        assert torch.equal(a, b)


def test_output_guard_bytes_untouched():
    """Canaries around the output and workspace catch out-of-bounds writes."""
    w = _small("c5", batch=3, ragged=(1, 200))
    print("[decode] guard canaries", flush=True)
    p = make_pair(w, DEV, with_oracle=False)
    B, Hq, d = w.batch, w.num_q_heads, w.head_dim
    guard = 4096
    outbuf = torch.full((B * Hq * d + 2 * guard,), 12345.0, device=DEV)
    out = outbuf[guard:guard + B * Hq * d].view(B, Hq, d)
    ws_need = kvq.decode_workspace_bytes(p.gpu, B, Hq, int(p.lens.max()))
    wsbuf = torch.full((ws_need + 2 * guard,), 0xAB, dtype=torch.uint8, device=DEV)
    ws = wsbuf[guard:guard + ws_need]
    kvq.decode_attention(p.gpu, wl.queries(w).to(DEV), p.geo.block_table.to(DEV), p.lens.to(DEV),
                         int(p.lens.max()), workspace=ws, out=out)
    torch.cuda.synchronize()
    assert torch.all(outbuf[:guard] == 12345.0) and torch.all(outbuf[-guard:] == 12345.0)
    assert torch.all(wsbuf[:guard] == 0xAB) and torch.all(wsbuf[-guard:] == 0xAB)


@pytest.mark.parametrize("num_splits", [1, 2, 0])
def test_decode_long_paged_partitions(num_splits):
    """16-token pages, partitions of up to ~160 pages: the kernel walks its block table
    through a 64-entry window that must move forward several times per partition."""
    w = _small("c5", batch=2, ragged=(1500, 2600))
    print(f"[decode] long paged partitions, num_splits={num_splits}", flush=True)
    p = make_pair(w, DEV, extra_tokens=1)
    append_step(p, 0, DEV)
    got, want = decode_both(p, DEV, num_splits=num_splits)
    err = max_err(got, want)
    record(f"long_paged/splits={num_splits}", err)
    assert err <= TOL


@pytest.mark.parametrize("page", [0, 16, 48])
def test_decode_large_value_scales(page):
    """A few tokens with values in the thousands (value scales >= 128): the kernel's
    scaled f16 value weights would overflow, so it must fall back to unscaled weights
    for the partition and still match the oracle. Paged caches rewalk their pages for the
    second pass (with one partition of 1500 tokens in 16-token pages, the window of
    block-table entries is refilled in both passes)."""
    w = _small("c2", batch=2, context=700 if page == 0 else 1500, page_size=page)
    print(f"[decode] large value scales, page {page}", flush=True)
    lens = wl.seq_lens(w)
    geo = wl.geometry(w, lens=lens)
    gpu = kvq.KVCache.allocate(128, 8, 4, 32, 128, geo.page_size, geo.num_pages, device=DEV)
    ref = oracle.Cache(128, 8, 4, 32, 128, geo.page_size, geo.num_pages)
    for b in range(w.batch):
        T = int(lens[b])
        k = wl.keys(w, b, 0, T)
        v = wl.values(w, b, 0, T).float()
        v[400 + 37 * b] *= 4000.0          # one token per sequence, mid-partition
        v[650, :2] *= 300.0                # and a few large channels near the end
        v = v.to(torch.bfloat16)
        slots = geo.slots(b, 0, T)
        kvq.quantize_append(gpu, k.to(DEV), v.to(DEV), slots.to(DEV))
        ref.append(wl.bf16_bits(k), wl.bf16_bits(v), slots.numpy())
    q = wl.queries(w)
    for ns in (1, 0):
        out = kvq.decode_attention(gpu, q.to(DEV), geo.block_table.to(DEV), lens.to(DEV), int(lens.max()),
                                   num_splits=ns)
        got = out.cpu().numpy().astype(np.float64)
        want = ref.decode(wl.bf16_bits(q), geo.block_table.numpy(), lens.numpy())
        err = max_err(got, want)
        record(f"large_value_scales/page={page}/splits={ns}", err)
        print(f"  splits={ns}: max |o| {np.max(np.abs(want)):.1f}, max-abs err {err:.3e}", flush=True)
        assert np.all(np.isfinite(got)) and err <= TOL


def _structured_rows(rng, n, Hkv, hb):
    """Rows on which the symmetric groups win: integers in [-7, 7] and power-of-two-scaled
    ternary values for V; for K the same, mapped through the rotation's inverse (the
    rotation is its own inverse) so the rotated keys land near those grids."""
    ints = rng.integers(-7, 8, (n, Hkv, 128)).astype(np.float64)
    tern = rng.integers(-1, 2, (n, Hkv, 128)) * 2.0 ** rng.integers(-3, 4, (n, Hkv, 1))
    mix = rng.standard_normal((n, Hkv, 128))
    pick = rng.integers(0, 3, (n, Hkv, 1))
    v = np.where(pick == 0, ints, np.where(pick == 1, tern, mix))
    k = v.copy()
    if hb:
        Rm = np.kron(np.eye(128 // hb), __import__("scipy.linalg").linalg.hadamard(hb) / np.sqrt(hb))
        k = k @ Rm.T
    return _bf16(k), _bf16(v[:, ::-1].copy())


@pytest.mark.parametrize("bits,G,hb", [(4, 32, 128), (2, 32, 128), (2, 128, 128), (4, 64, 0), (2, 64, 32)])
def test_hybrid_append_and_decode(bits, G, hb):
    """quant_mode 1: every cache byte equal to the oracle's hybrid quantizer (which picks
    symmetric groups on these rows), decode within the tolerance."""
    print(f"[hybrid] bits={bits} G={G} hb={hb}", flush=True)
    rng = np.random.default_rng(61 + bits * G + hb)
    B, Hkv, Hq, T = 2, 2, 8, 300
    w = wl.Workload("hybrid", B, Hq, Hkv, 128, T, bits, G, hb, page_size=16)
    lens = torch.tensor([T, 137], dtype=torch.int32)
    geo = wl.geometry(w, lens=lens)
    gpu = kvq.KVCache.allocate(128, Hkv, bits, G, hb, geo.page_size, geo.num_pages, device=DEV, quant_mode=1)
    ref = oracle.Cache(128, Hkv, bits, G, hb, geo.page_size, geo.num_pages, quant_mode=1)
    asym = oracle.Cache(128, Hkv, bits, G, hb, geo.page_size, geo.num_pages)
    for b in range(B):
        n = int(lens[b])
        k, v = _structured_rows(rng, n, Hkv, hb)
        slots = geo.slots(b, 0, n)
        kvq.quantize_append(gpu, k.to(DEV), v.to(DEV), slots.to(DEV))
        ref.append(wl.bf16_bits(k), wl.bf16_bits(v), slots.numpy())
        asym.append(wl.bf16_bits(k), wl.bf16_bits(v), slots.numpy())
    torch.cuda.synchronize()
    for name, g, r in zip(("k_codes", "k_meta", "v_codes", "v_meta"), gpu.planes(), ref.planes()):
        gn = g.cpu().numpy()
        assert np.array_equal(gn, r), f"{name}: {int(np.sum(gn != r))} bytes differ"
    # the hybrid choice made a difference on these rows
    assert not np.array_equal(ref.v_meta, asym.v_meta)
    q = _bf16(rng.standard_normal((B, Hq, 128)))
    out = kvq.decode_attention(gpu, q.to(DEV), geo.block_table.to(DEV), lens.to(DEV), T)
    torch.cuda.synchronize()
    want = ref.decode(wl.bf16_bits(q), geo.block_table.numpy(), lens.numpy())
    err = max_err(out.cpu().numpy().astype(np.float64), want)
    record(f"hybrid_b{bits}_g{G}_hb{hb}", err)
    assert err <= TOL, err


@pytest.mark.parametrize("bits,G", [(4, 32), (2, 128)])
def test_bulk_append_tiles_and_fallback(bits, G):
    """Bulk appends go tile by tile when their rows are whole 16-token tiles and row by
    row otherwise: an aligned run, a run starting off a tile boundary, and shuffled slots,
    all bit-exact against the oracle."""
    print(f"[bulk] bits={bits} G={G}", flush=True)
    rng = np.random.default_rng(81 + bits)
    P, pages, H = 64, 24, 8
    gpu = kvq.KVCache.allocate(128, H, bits, G, 128, P, pages, device=DEV)
    ref = oracle.Cache(128, H, bits, G, 128, P, pages)
    runs = [np.arange(0, 512),                          # 8 whole pages, tile aligned
            np.arange(512 + 5, 512 + 5 + 300),         # starts 5 tokens into a tile
            rng.permutation(np.arange(832, 1536))]     # the same tokens, slots shuffled
    for slots in runs:
        n = slots.size
        k = _bf16(rng.standard_normal((n, H, 128)) * np.exp(rng.standard_normal((1, H, 128))))
        v = _bf16(rng.standard_normal((n, H, 128)))
        s = torch.from_numpy(slots.astype(np.int64))
        kvq.quantize_append(gpu, k.to(DEV), v.to(DEV), s.to(DEV))
        ref.append(wl.bf16_bits(k), wl.bf16_bits(v), slots.astype(np.int64))
    torch.cuda.synchronize()
    for name, g, r in zip(("k_codes", "k_meta", "v_codes", "v_meta"), gpu.planes(), ref.planes()):
        gn = g.cpu().numpy()
        assert np.array_equal(gn, r), f"{name}: {int(np.sum(gn != r))} bytes differ"
