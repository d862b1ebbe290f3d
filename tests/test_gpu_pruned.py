"""Query-channel pruning of key reads (Dual-QK, Abstract) on the GPU against the oracle.

Per case: the kernel ranks the 16-byte key chunks of each (sequence, kv head) by the
summed squared rotated query and keeps the top keep_chunks; it reports its choice. The
choice is checked for validity against the oracle's fp64 energies (the right number of
chunks, none pruned with clearly more energy than a kept one: the two sides round the
energies differently, so near-ties may go either way), and the decode output against
the oracle's pruned decode with that same choice, within 2e-3.
"""
import numpy as np
import pytest
import torch

import bit_kv_cache_quantize_amd as kvq
import workloads as wl
from kvq_harness import TOL, EventPair, make_pair, max_err, record

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _small(name, **kw):
    return wl.get(name).with_(**kw)


CASES = {
    "int4_g32_gqa4": _small("c2", batch=3, context=700),
    "int4_g64_gqa2_sink": _small("c3", context=2100, num_q_heads=16),
    "int2_g128": _small("c4", batch=2, context=900),
    "int2_g32_gqa1_hb0": _small("c2", batch=2, context=333, bits=2, num_q_heads=8, hadamard_block=0),
    "paged_ragged": _small("c5", batch=5, ragged=(1, 800)),
    "int4_g128_hb32": _small("c2", batch=2, context=400, group_size=128, hadamard_block=32),
    # more than 64 sequences, some empty: the balanced plan over several groups of 64
    "b70_ragged": _small("c5", batch=70, ragged=(0, 300)),
}


def check_mask(mask, energy, keep):
    """mask int32 [B][Hkv] from the GPU; energy fp64 [B][Hkv][n] from the oracle."""
    B, H, n = energy.shape
    for b in range(B):
        for h in range(H):
            kept = [j for j in range(n) if (mask[b, h] >> j) & 1]
            assert len(kept) == keep and 0 <= mask[b, h] < (1 << n), (b, h, mask[b, h])
            pruned = [j for j in range(n) if j not in kept]
            if pruned:
                e = energy[b, h]
                assert min(e[kept]) >= max(e[pruned]) * (1 - 1e-5), (b, h, e, kept)


@pytest.mark.parametrize("name", list(CASES))
def test_pruned_decode_matches_oracle(name):
    w = CASES[name]
    nch = w.bits  # head_dim * bits / 128 chunks of 128 / bits channels
    print(f"[pruned] {name}: {w}", flush=True)
    p = make_pair(w, DEV)
    q = wl.queries(w, step=3)
    bt, lens = p.geo.block_table.to(DEV), p.lens.to(DEV)
    maxlen = max(int(p.lens.max()), 1)
    energy = p.ref.prune_energy(wl.bf16_bits(q))
    plain = kvq.decode_attention(p.gpu, q.to(DEV), bt, lens, maxlen).cpu().numpy()
    for keep in range(1, nch + 1):
        mask = torch.full((w.batch, w.num_kv_heads), -1, dtype=torch.int32, device=DEV)
        out = kvq.decode_attention_pruned(p.gpu, q.to(DEV), bt, lens, maxlen, keep, chunk_mask=mask)
        torch.cuda.synchronize()
        mask_h = mask.cpu().numpy()
        live = p.lens.numpy() > 0
        check_mask(mask_h[live], energy[live], keep)
        mask_h[~live] = (1 << nch) - 1
        want = p.ref.decode_pruned(wl.bf16_bits(q), p.geo.block_table.numpy(), p.lens.numpy(), mask_h)
        got = out.cpu().numpy().astype(np.float64)
        err = max_err(got, want)
        record(f"pruned_{name}_keep{keep}", err)
        print(f"[pruned] {name} keep {keep}/{nch}: max err {err:.3e}", flush=True)
        assert err <= TOL, (keep, err)
        if keep == nch:  # nothing pruned: the plain decode's result
            dev = float(np.max(np.abs(got - plain)))
            record(f"pruned_{name}_all_vs_plain", dev)
            if w.group_size == 32:
                # the same arithmetic in both kernels: equal up to summation order
                assert dev <= 1e-6
            else:
                # with 64- or 128-channel groups the plain decode scores with int8 query
                # digits, the pruned one with f16 digits: each must match the unpruned oracle
                plain_ref = p.ref.decode(wl.bf16_bits(q), p.geo.block_table.numpy(), p.lens.numpy())
                assert np.array_equal(want, plain_ref)
                assert max_err(plain.astype(np.float64), plain_ref) <= TOL


def test_pruned_fullsize_h1_sampled():
    """H1 (B64, 32K, INT4 g32) in the benchmark's launch configuration, keep 3 and 2 of 4
    chunks: two sampled sequences recomputed by the oracle with the GPU's choice."""
    import oracle

    w = wl.get("h1")
    lens = wl.seq_lens(w)
    geo = wl.geometry(w, lens=lens)
    B, Hq, Hkv, d = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim
    print(f"[pruned] h1 full size: B={B} T={int(lens[0])}", flush=True)
    cache = kvq.KVCache.allocate(d, Hkv, w.bits, w.group_size, w.hadamard_block, geo.page_size, geo.num_pages,
                                 device=DEV)
    for b in range(B):
        T = int(lens[b])
        k, v = wl.keys(w, b, 0, T, device=DEV), wl.values(w, b, 0, T, device=DEV)
        kvq.quantize_append(cache, k, v, geo.slots(b, 0, T).to(DEV))
        del k, v
    q = wl.queries(w, step=1, device=DEV)
    bt, lens_d = geo.block_table.to(DEV), lens.to(DEV)
    T = int(lens.max())
    for keep in (3, 2):
        mask = torch.zeros((B, Hkv), dtype=torch.int32, device=DEV)
        out = kvq.decode_attention_pruned(cache, q, bt, lens_d, T, keep, chunk_mask=mask).cpu().numpy()
        mask_h = mask.cpu().numpy()
        for b in (0, B - 1):
            Tb = int(lens[b])
            ref = oracle.Cache(d, Hkv, w.bits, w.group_size, w.hadamard_block, geo.page_size, 1)
            k, v = wl.keys(w, b, 0, Tb, device=DEV), wl.values(w, b, 0, Tb, device=DEV)
            ref.append(wl.bf16_bits(k), wl.bf16_bits(v), np.arange(Tb))
            del k, v
            qb = wl.bf16_bits(q[b:b + 1])
            check_mask(mask_h[b:b + 1], ref.prune_energy(qb), keep)
            want = ref.decode_pruned(qb, np.zeros((1, 1), np.int32), np.array([Tb], np.int32), mask_h[b:b + 1])
            err = float(np.max(np.abs(out[b] - want[0])))
            record(f"pruned_h1_keep{keep}_seq{b}", err)
            print(f"[pruned] h1 keep {keep} seq {b}: max err {err:.3e}", flush=True)
            assert err <= TOL
    del cache
    torch.cuda.empty_cache()


def test_pruned_timed_events():
    """Events passed to the pruned decode give the untimed call's exact output and record a
    positive interval around the split kernel."""
    w = _small("c2", batch=3, context=700)
    print("[pruned] timed entry point", flush=True)
    p = make_pair(w, DEV, with_oracle=False)
    q = wl.queries(w, step=3).to(DEV)
    bt, lens = p.geo.block_table.to(DEV), p.lens.to(DEV)
    plain = kvq.decode_attention_pruned(p.gpu, q, bt, lens, 700, 2).cpu()
    ev = EventPair()
    try:
        timed = kvq.decode_attention_pruned(p.gpu, q, bt, lens, 700, 2, events=ev.handles()).cpu()
        torch.cuda.synchronize()
        assert torch.equal(plain, timed)
        assert ev.elapsed_ms() > 0.0
    finally:
        ev.close()
