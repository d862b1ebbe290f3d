"""Values grouped along tokens (InnerQ, Abstract: groups along the inner dimension of the
value product) on the GPU against the oracle.

Caches with v_grouping 1: keys per token, values per (group of G tokens, channel). The
prefill appends whole groups; a bf16 residual (a window with sink 0 and a ring of G rows)
takes decode-time tokens and quantizes each group when its last token arrives. Bar:
every byte of the four cache planes and of the residual planes equal to the oracle's;
dequantized rows bit-equal; decode (matrix-core and plain split kernels, and through the
residual) within 2e-3 of the fp64 oracle.
"""
import numpy as np
import pytest
import torch

import bit_kv_cache_quantize_amd as kvq
import oracle
import workloads as wl
from kvq_harness import TOL, max_err, record

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _w(name, **kw):
    return wl.get(name).with_(**kw)


class VPair:
    """A cache with value token groups on both sides, prefilled with whole groups."""

    def __init__(self, w, lens, steps=0, mode=0, residual=False):
        self.w, self.lens = w, torch.tensor(lens, dtype=torch.int32)
        G = w.group_size
        self.geo = wl.geometry(w, extra_tokens=steps, lens=self.lens)
        g = self.geo
        self.gpu = kvq.KVCache.allocate(128, w.num_kv_heads, w.bits, G, w.hadamard_block, g.page_size, g.num_pages,
                                        device=DEV, quant_mode=mode, v_grouping=1)
        self.ref = oracle.Cache(128, w.num_kv_heads, w.bits, G, w.hadamard_block, g.page_size, g.num_pages,
                                quant_mode=mode, v_grouping=1)
        self.gwin = kvq.KVWindow.allocate(self.gpu, 0, G, w.batch, device=DEV, residual=1) if residual else None
        self.rwin = oracle.Window(128, w.num_kv_heads, 0, G, w.batch, residual=1) if residual else None
        for b in range(w.batch):
            T = int(self.lens[b])
            done = T - T % G
            k, v = wl.keys(w, b, 0, T), wl.values(w, b, 0, T)
            if done:
                slots = g.slots(b, 0, done)
                kvq.quantize_append(self.gpu, k[:done].to(DEV), v[:done].to(DEV), slots.to(DEV))
                self.ref.append(wl.bf16_bits(k[:done]), wl.bf16_bits(v[:done]), slots.numpy())
            for t in range(done, T):  # the incomplete group: residual rows t % G
                assert residual
                self.gwin.k[b, t % G] = k[t].to(DEV)
                self.gwin.v[b, t % G] = v[t].to(DEV)
                self.rwin.k[b, t % G] = wl.bf16_bits(k[t])
                self.rwin.v[b, t % G] = wl.bf16_bits(v[t])

    def step(self, s):
        G, B = self.w.group_size, self.w.batch
        kn, vn = wl.new_tokens(self.w, s)
        pos = self.lens.clone()
        first = torch.tensor([int(self.geo.slots(b, max(int(self.lens[b]) - G + 1, 0), 1)[0]) for b in range(B)],
                             dtype=torch.int64)
        seqs = torch.arange(B, dtype=torch.int32)
        kvq.window_append(self.gpu, self.gwin, kn.to(DEV), vn.to(DEV), seqs.to(DEV), pos.to(DEV), first.to(DEV))
        self.rwin.append(self.ref, wl.bf16_bits(kn), wl.bf16_bits(vn), seqs.numpy(), pos.numpy(), first.numpy())
        self.lens += 1

    def mismatches(self):
        torch.cuda.synchronize()
        bad = []
        for name, g, r in zip(("k_codes", "k_meta", "v_codes", "v_meta"), self.gpu.planes(), self.ref.planes()):
            gn = g.cpu().numpy()
            if not np.array_equal(gn, r):
                bad.append(f"{name}: {int(np.sum(gn != r))} bytes differ")
        if self.gwin is not None:
            for name, g, r in (("residual k", self.gwin.k, self.rwin.k), ("residual v", self.gwin.v, self.rwin.v)):
                if not np.array_equal(wl.bf16_bits(g), r):
                    bad.append(name)
        return bad

    def decode(self, step, reference=False, num_splits=0):
        q = wl.queries(self.w, step)
        maxlen = max(int(self.lens.max()), 1)
        bt, lens = self.geo.block_table, self.lens
        if self.gwin is not None:
            out = kvq.decode_attention_window(self.gpu, self.gwin, q.to(DEV), bt.to(DEV), lens.to(DEV), maxlen,
                                              num_splits=num_splits)
            want = self.rwin.decode(self.ref, wl.bf16_bits(q), bt.numpy(), lens.numpy())
        else:
            out = kvq.decode_attention(self.gpu, q.to(DEV), bt.to(DEV), lens.to(DEV), maxlen, num_splits=num_splits,
                                       reference=reference)
            want = self.ref.decode(wl.bf16_bits(q), bt.numpy(), lens.numpy())
        torch.cuda.synchronize()
        return out.cpu().numpy().astype(np.float64), want


# name -> (workload, whole-group lengths)
CASES = {
    "int4_g32": (_w("c2", batch=3, context=2048, page_size=128), [2048, 640, 32]),
    "int4_g64_gqa2": (_w("c2", batch=2, context=1024, page_size=256, group_size=64, num_q_heads=16), [1024, 448]),
    "int4_g128_hb0": (_w("c2", batch=2, context=768, page_size=256, group_size=128, hadamard_block=0), [768, 256]),
    "int2_g128": (_w("c4", batch=2, context=1280, page_size=128), [1280, 384]),
    "int2_g32_gqa1": (_w("c2", batch=2, context=512, page_size=64, bits=2, num_q_heads=8), [512, 96]),
    "int4_g32_sink_outliers": (_w("c3", context=4096, group_size=32, page_size=512), [4096]),
    # more than 64 sequences: the balanced plan over several groups of 64
    "b66_int4_g32": (_w("c2", batch=66, context=256, page_size=64), [32 * (1 + (5 * b) % 8) for b in range(66)]),
}


@pytest.mark.parametrize("mode", [0, 1], ids=["minmax", "hybrid"])
@pytest.mark.parametrize("name", list(CASES))
def test_vgroup_append_dequantize_decode(name, mode):
    w, lens = CASES[name]
    print(f"[vgroup] {name} mode={mode}: lens={lens}", flush=True)
    p = VPair(w, lens, mode=mode)
    assert p.mismatches() == []
    slots = torch.cat([p.geo.slots(b, 0, lens[b]) for b in range(w.batch)])
    got = kvq.dequantize(p.gpu, 1, slots.to(DEV)).cpu().numpy()
    assert np.array_equal(got.view(np.uint32), p.ref.dequantize(1, slots.numpy()).view(np.uint32))
    for reference in (False, True):
        out, want = p.decode(step=2, reference=reference)
        err = max_err(out, want)
        record(f"vgroup_{name}_m{mode}_{'ref' if reference else 'mfma'}", err)
        print(f"[vgroup] {name} mode={mode} reference={reference}: max err {err:.3e}", flush=True)
        assert err <= TOL, (reference, err)


def test_vgroup_split_counts():
    w, lens = CASES["int4_g32"]
    p = VPair(w, lens)
    for splits in (1, 3, 17):
        out, want = p.decode(step=4, num_splits=splits)
        err = max_err(out, want)
        print(f"[vgroup] splits={splits}: max err {err:.3e}", flush=True)
        assert err <= TOL


@pytest.mark.parametrize("name,steps,mode", [("int4_g32", 70, 0), ("int2_g128", 140, 0), ("int4_g64_gqa2", 70, 0),
                                             ("int4_g32", 40, 1)])
def test_vgroup_residual_stream(name, steps, mode):
    """Decode-time tokens through the residual: groups complete and are quantized as the
    stream crosses multiples of G; planes bit-exact and decode within tolerance at
    several points (residual empty, partly and almost full)."""
    w, lens = CASES[name]
    G = w.group_size
    lens = [n + (5 if i == 0 else G - 3) for i, n in enumerate(lens)]  # start with a partial group
    print(f"[vgroup] residual {name}: lens={lens} steps={steps} mode={mode}", flush=True)
    p = VPair(w, lens, steps=steps, mode=mode, residual=True)
    for s in range(steps):
        p.step(s)
        if s % 23 == 0 or s == steps - 1 or int(p.lens[0]) % G == 0:
            assert p.mismatches() == [], f"step {s}"
            out, want = p.decode(step=s)
            err = max_err(out, want)
            record(f"vgroup_residual_{name}_s{s}", err)
            print(f"[vgroup] residual {name} step {s}: lens={p.lens.tolist()} max err {err:.3e}", flush=True)
            assert err <= TOL, (s, err)


def test_residual_channel_groups():
    """The residual also serves caches with per-token value groups (each completed group
    is quantized row by row)."""
    w = _w("c2", batch=2, context=300, page_size=32)  # a group of R tokens within one page
    G, R = 32, 32
    B = w.batch
    lens = torch.tensor([300, 77], dtype=torch.int32)
    geo = wl.geometry(w, extra_tokens=40, lens=lens)
    gpu = kvq.KVCache.allocate(128, 8, 4, G, 128, geo.page_size, geo.num_pages, device=DEV)
    ref = oracle.Cache(128, 8, 4, G, 128, geo.page_size, geo.num_pages)
    gw = kvq.KVWindow.allocate(gpu, 0, R, B, device=DEV, residual=1)
    rw = oracle.Window(128, 8, 0, R, B, residual=1)
    for b in range(B):
        T = int(lens[b])
        done = T - T % R
        k, v = wl.keys(w, b, 0, T), wl.values(w, b, 0, T)
        slots = geo.slots(b, 0, done)
        kvq.quantize_append(gpu, k[:done].to(DEV), v[:done].to(DEV), slots.to(DEV))
        ref.append(wl.bf16_bits(k[:done]), wl.bf16_bits(v[:done]), slots.numpy())
        for t in range(done, T):
            gw.k[b, t % R], gw.v[b, t % R] = k[t].to(DEV), v[t].to(DEV)
            rw.k[b, t % R], rw.v[b, t % R] = wl.bf16_bits(k[t]), wl.bf16_bits(v[t])
    for s in range(40):
        kn, vn = wl.new_tokens(w, s)
        first = torch.tensor([int(geo.slots(b, max(int(lens[b]) - R + 1, 0), 1)[0]) for b in range(B)])
        seqs = torch.arange(B, dtype=torch.int32)
        kvq.window_append(gpu, gw, kn.to(DEV), vn.to(DEV), seqs.to(DEV), lens.to(DEV), first.to(DEV))
        rw.append(ref, wl.bf16_bits(kn), wl.bf16_bits(vn), seqs.numpy(), lens.numpy(), first.numpy())
        lens += 1
    torch.cuda.synchronize()
    for g, r in zip(gpu.planes(), ref.planes()):
        assert np.array_equal(g.cpu().numpy(), r)
    q = wl.queries(w, 9)
    out = kvq.decode_attention_window(gpu, gw, q.to(DEV), geo.block_table.to(DEV), lens.to(DEV), int(lens.max()))
    want = rw.decode(ref, wl.bf16_bits(q), geo.block_table.numpy(), lens.numpy())
    err = max_err(out.cpu().numpy().astype(np.float64), want)
    print(f"[vgroup] residual with channel groups: max err {err:.3e}", flush=True)
    assert err <= TOL
