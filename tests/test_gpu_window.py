"""High-precision windows on the GPU (through the C ABI) against the oracle.

InnerQ (Abstract): sink tokens and a recent window stay in high precision. Per case the
same generated tokens go to both sides: a prefill state (the quantized span through
the ordinary append, the window rows written directly, as a caller may), then decode
steps through the window append, each moving the token that leaves the recent window
into the cache. Bar: every byte of the four cache planes and of both bf16 window planes
equal; decode output within 2e-3 max-abs of the fp64 oracle.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import bit_kv_cache_quantize_amd as kvq
import oracle
import workloads as wl
from kvq_harness import TOL, EventPair, max_err, record

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


class WinPair:
    """The same windows + cache on the GPU and in the oracle."""

    def __init__(self, w: wl.Workload, S: int, R: int, lens: torch.Tensor, steps: int):
        self.w, self.S, self.R = w, S, R
        self.lens = lens.clone()
        self.geo = wl.geometry(w, extra_tokens=steps, lens=lens)
        g = self.geo
        self.gpu = kvq.KVCache.allocate(w.head_dim, w.num_kv_heads, w.bits, w.group_size, w.hadamard_block,
                                        g.page_size, g.num_pages, device=DEV)
        self.gwin = kvq.KVWindow.allocate(self.gpu, S, R, w.batch, device=DEV)
        self.ref = oracle.Cache(w.head_dim, w.num_kv_heads, w.bits, w.group_size, w.hadamard_block, g.page_size,
                                g.num_pages)
        self.rwin = oracle.Window(w.head_dim, w.num_kv_heads, S, R, w.batch)
        for b in range(w.batch):
            T = int(lens[b])
            if T == 0:
                continue
            k, v = wl.keys(w, b, 0, T), wl.values(w, b, 0, T)
            lo, hi = S, T - R
            if hi > lo:  # the quantized span
                slots = g.slots(b, lo, hi - lo)
                kvq.quantize_append(self.gpu, k[lo:hi].to(DEV), v[lo:hi].to(DEV), slots.to(DEV))
                self.ref.append(wl.bf16_bits(k[lo:hi]), wl.bf16_bits(v[lo:hi]), slots.numpy())
            for t in list(range(min(S, T))) + list(range(max(S, T - R), T)):
                row = self.gwin.row(t)
                self.gwin.k[b, row] = k[t].to(DEV)
                self.gwin.v[b, row] = v[t].to(DEV)
                self.rwin.k[b, row] = wl.bf16_bits(k[t])
                self.rwin.v[b, row] = wl.bf16_bits(v[t])

    def step(self, step: int, seqs: list[int] | None = None) -> None:
        """One new token for each sequence in `seqs` (default all)."""
        B = self.w.batch
        seqs = list(range(B)) if seqs is None else seqs
        kn, vn = wl.new_tokens(self.w, step)
        kn, vn = kn[seqs].contiguous(), vn[seqs].contiguous()
        pos = self.lens[seqs].clone()
        ev = torch.tensor([int(self.geo.slots(b, int(self.lens[b]) - self.R, 1)[0])
                           if int(self.lens[b]) >= self.R else 0 for b in seqs], dtype=torch.int64)
        sq = torch.tensor(seqs, dtype=torch.int32)
        kvq.window_append(self.gpu, self.gwin, kn.to(DEV), vn.to(DEV), sq.to(DEV), pos.to(DEV), ev.to(DEV))
        self.rwin.append(self.ref, wl.bf16_bits(kn), wl.bf16_bits(vn), sq.numpy(), pos.numpy(), ev.numpy())
        self.lens[seqs] += 1

    def mismatches(self) -> list[str]:
        torch.cuda.synchronize()
        bad = []
        for name, g, r in zip(("k_codes", "k_meta", "v_codes", "v_meta"), self.gpu.planes(), self.ref.planes()):
            gn = g.cpu().numpy()
            if not np.array_equal(gn, r):
                bad.append(f"{name}: {int(np.sum(gn != r))} bytes differ")
        for name, g, r in (("window k", self.gwin.k, self.rwin.k), ("window v", self.gwin.v, self.rwin.v)):
            gn = wl.bf16_bits(g)
            if not np.array_equal(gn, r):
                bad.append(f"{name}: {int(np.sum(gn != r))} elements differ")
        return bad

    def decode(self, step: int, num_splits: int = 0, softmax_scale: float = 0.0):
        q = wl.queries(self.w, step)
        maxlen = max(int(self.lens.max()), 1)
        out = kvq.decode_attention_window(self.gpu, self.gwin, q.to(DEV), self.geo.block_table.to(DEV),
                                          self.lens.to(DEV), maxlen, softmax_scale=softmax_scale,
                                          num_splits=num_splits)
        torch.cuda.synchronize()
        want = self.rwin.decode(self.ref, wl.bf16_bits(q), self.geo.block_table.numpy(), self.lens.numpy(),
                                softmax_scale)
        return out.cpu().numpy().astype(np.float64), want


def _w(name, **kw):
    return wl.get(name).with_(**kw)


# name -> (workload, sink, recent, prefill lengths, decode steps)
CASES = {
    # every token in a window: T < S, then S <= T < S + R
    "all_sink": (_w("c2", batch=2, context=20), 32, 64, [20, 7], 3),
    "sink_and_ring": (_w("c2", batch=2, context=60), 32, 64, [60, 40], 4),
    # the ring fills during the steps: the first evictions
    "first_evictions": (_w("c2", batch=3, context=95), 32, 64, [95, 94, 90], 6),
    # long spans through the split kernel, contiguous and paged
    "int4_g32_ragged": (_w("c2", batch=3, context=2000), 32, 128, [2000, 777, 161], 3),
    "paged16": (_w("c5", batch=3, ragged=None, context=3000), 64, 128, [3000, 1234, 300], 3),
    # paged narrow groups: the split kernel's span starts at the sink (48 tokens, mid-page
    # in 32-token pages) and its tiles come from the super-block table
    "paged32_int2_g128": (_w("c5", batch=2, ragged=None, context=2600, bits=2, group_size=128, page_size=32),
                          48, 64, [2600, 1000], 2),
    "paged48_int4_g64": (_w("c5", batch=2, ragged=None, context=2200, group_size=64, page_size=48),
                         16, 96, [2200, 700], 2),
    "no_sink": (_w("c2", batch=2, context=1500), 0, 96, [1500, 97], 3),
    "sink16_recent1": (_w("c2", batch=2, context=600), 16, 1, [600, 17], 3),
    "int2_g128": (_w("c4", batch=2, context=1200), 32, 128, [1200, 500], 2),
    "int4_g64_sinkkey": (_w("c3", context=3000), 32, 256, [3000], 2),
    "gqa1": (_w("c2", batch=2, context=800, num_q_heads=8), 32, 64, [800, 300], 2),
    "gqa2": (_w("c2", batch=2, context=800, num_q_heads=16), 32, 64, [800, 300], 2),
    "max_window": (_w("c2", batch=2, context=2500), 512, 512, [2500, 1100], 2),
    # more than 64 sequences: the balanced plan's prefix sums over several groups of 64
    "b70_ragged": (_w("c2", batch=70, context=700), 16, 32,
                   [(37 * b) % 700 if b % 9 else 0 for b in range(70)], 2),
}


@pytest.mark.parametrize("name", list(CASES))
def test_window_append_and_decode(name):
    w, S, R, lens, steps = CASES[name]
    print(f"[window] {name}: S={S} R={R} lens={lens} steps={steps} {w}", flush=True)
    p = WinPair(w, S, R, torch.tensor(lens, dtype=torch.int32), steps)
    got, want = p.decode(100)
    err = max_err(got, want)
    assert err <= TOL, f"{name} before steps: {err}"
    for s in range(steps):
        p.step(s)
        assert p.mismatches() == [], f"{name} step {s}"
        got, want = p.decode(s)
        err = max_err(got, want)
        record(f"window_{name}_step{s}", err)
        print(f"[window] {name} step {s}: lens={p.lens.tolist()} max err {err:.3e}", flush=True)
        assert err <= TOL, f"{name} step {s}: {err}"


def test_window_stream_from_empty():
    """Every token through the window append from position 0: sink rows, ring rows, and
    later evictions one token at a time, for sequences that join at different steps."""
    w = _w("c2", batch=3, context=200, page_size=16)
    S, R = 16, 32
    print(f"[window] stream from empty: S={S} R={R}", flush=True)
    p = WinPair(w, S, R, torch.zeros(3, dtype=torch.int32), 200)
    for s in range(130):
        seqs = [b for b in range(3) if s >= 40 * b]  # sequence b joins at step 40 b
        p.step(s, seqs)
        if s % 16 == 15 or s == 129:
            assert p.mismatches() == [], f"step {s}"
            got, want = p.decode(s)
            err = max_err(got, want)
            print(f"[window] stream step {s}: lens={p.lens.tolist()} max err {err:.3e}", flush=True)
            assert err <= TOL, f"step {s}: {err}"


def test_window_decode_explicit_splits_and_scale():
    w = _w("c2", batch=2, context=3000)
    p = WinPair(w, 32, 128, torch.tensor([3000, 2100], dtype=torch.int32), 0)
    for splits, scale in ((1, 0.0), (3, 0.0), (40, 0.05)):
        got, want = p.decode(7, num_splits=splits, softmax_scale=scale)
        err = max_err(got, want)
        print(f"[window] splits={splits} scale={scale}: max err {err:.3e}", flush=True)
        assert err <= TOL, (splits, scale, err)


def test_window_decode_many_partials():
    """More than 128 partials per (sequence, query head) plus the window partial: the
    combine's shape with four workgroups of 32 groups x 32 channels per pair."""
    w = _w("c2", batch=2, context=5200)
    p = WinPair(w, 32, 64, torch.tensor([5200, 4700], dtype=torch.int32), 0)
    for splits in (150, 0):
        got, want = p.decode(5, num_splits=splits)
        err = max_err(got, want)
        print(f"[window] many partials, splits={splits}: max err {err:.3e}", flush=True)
        assert err <= TOL, (splits, err)


def test_window_zero_length_rows():
    """seq_len 0 gives a zero row; other sequences are unaffected."""
    w = _w("c2", batch=3, context=400)
    p = WinPair(w, 32, 64, torch.tensor([400, 0, 50], dtype=torch.int32), 0)
    got, want = p.decode(3)
    assert np.all(got[1] == 0.0)
    assert max_err(got, want) <= TOL


def test_window_decode_timed_entry_point():
    """kvq_decode_attention_window_timed gives the untimed call's exact output and records
    a positive interval around the split kernel."""
    w = _w("c2", batch=2, context=3000)
    print("[window] timed entry point", flush=True)
    p = WinPair(w, 32, 128, torch.tensor([3000, 2100], dtype=torch.int32), 0)
    q = wl.queries(w, 7).to(DEV)
    bt, lens = p.geo.block_table.to(DEV), p.lens.to(DEV)
    maxlen = int(p.lens.max())
    plain = kvq.decode_attention_window(p.gpu, p.gwin, q, bt, lens, maxlen).cpu()
    ev = EventPair()
    try:
        timed = kvq.decode_attention_window(p.gpu, p.gwin, q, bt, lens, maxlen, events=ev.handles()).cpu()
        torch.cuda.synchronize()
        assert torch.equal(plain, timed)
        assert ev.elapsed_ms() > 0.0
    finally:
        ev.close()
