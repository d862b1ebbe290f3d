"""The fused decode step (kvq_decode_step: append + decode in one split-K launch) against
the two calls it fuses and against the oracle, through the C ABI.

Bar: after the step every byte of the four cache planes equals what kvq_quantize_append
of the same rows at the slots of positions seq_lens[b] - 1 leaves, and equals the
oracle's planes after the same append; the output equals kvq_decode_attention's on that
cache bit for bit, and lies within TOL of the fp64 oracle. Cases cover the balanced
plan (batch > 1) and fixed partitions (batch 1, explicit split counts), INT4/INT2 and
the three group sizes, GQA 1/2/4, paged ragged batches, hybrid groups, a rotation block
below the head size, and new tokens that open a partition, a 32-token block or a page,
that close one, and that are a sequence's only token, next to empty sequences.
"""
import numpy as np
import pytest
import torch

import bit_kv_cache_quantize_amd as kvq
import workloads as wl
from kvq_harness import TOL, EventPair, make_pair, max_err, planes_equal

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _small(name, **kw):
    return wl.get(name).with_(**kw)


def _lens(*v):
    return torch.tensor(v, dtype=torch.int32)


# name -> (workload, sequence lengths after the step or None for the workload's, num_splits, quant_mode)
CASES = {
    "c2_balanced": (_small("c2", batch=3, context=700), None, 0, 0),
    "c2_fixed_splits": (_small("c2", batch=3, context=700), None, 3, 0),
    "c3_batch1_g64": (_small("c3", context=1000), None, 0, 0),
    "c4_int2_g128": (_small("c4", batch=2, context=333), None, 0, 0),
    "c5_paged_ragged": (_small("c5", batch=5, ragged=(1, 300)), None, 0, 0),
    "gqa1_int4_g128": (_small("c2", batch=2, context=257, num_q_heads=8, group_size=128), None, 0, 0),
    "gqa2_int2_g32": (_small("c2", batch=2, context=129, num_q_heads=16, bits=2, group_size=32), None, 0, 0),
    "hybrid_int4_g32": (_small("c2", batch=2, context=300), None, 0, 1),
    "hybrid_int2_g64_hb16": (_small("c2", batch=2, context=200, bits=2, group_size=64, hadamard_block=16),
                             None, 0, 1),
    # 1: the only token; 33: opens a 32-token block; 256: closes a 256-token partition
    # unit; 257: opens the next; 0: nothing to append
    "boundaries_balanced": (_small("c2", batch=6, context=300), _lens(1, 33, 256, 257, 0, 32), 0, 0),
    "boundaries_fixed": (_small("c2", batch=6, context=300), _lens(1, 33, 256, 257, 0, 32), 4, 0),
    # pages of 16 tokens: 17 opens a page, 48 closes one
    "boundaries_paged": (_small("c5", batch=4, ragged=(1, 100)), _lens(17, 48, 1, 97), 0, 0),
    # paged narrow groups (the super-block tile table read as wave-uniform rows): INT2 g128
    # and INT4 g64 in 16- and 48-token pages, one sequence in a single partition of 60+
    # pages (the block-table window refilled after the append)
    "paged_int2_g128": (_small("c5", batch=4, ragged=(1, 900), bits=2, group_size=128), None, 0, 0),
    "paged48_int4_g64": (_small("c5", batch=3, ragged=(30, 700), page_size=48, group_size=64), None, 0, 0),
    "paged_int2_g128_one_partition": (_small("c5", batch=2, ragged=(1100, 1500), bits=2, group_size=128),
                                      None, 1, 0),
}


def _run_case(name):
    w, lens, num_splits, qm = CASES[name]
    if lens is None:
        lens = wl.seq_lens(w)
    print(f"[step] {name}: {w} lens={lens.tolist()} splits={num_splits} quant_mode={qm}", flush=True)
    has_new = lens > 0
    before = lens - has_new.to(torch.int32)
    p = make_pair(w, DEV, extra_tokens=1, lens=before, quant_mode=qm)
    twin = p.gpu.clone()
    k, v = wl.new_tokens(w, 0)
    q = wl.queries(w, 1)
    bt = p.geo.block_table.to(DEV)
    maxlen = max(int(lens.max()), 1)
    lens_d = lens.to(DEV)

    out_f = kvq.decode_step(p.gpu, k.to(DEV), v.to(DEV), q.to(DEV), bt, lens_d, maxlen, num_splits=num_splits)

    sel = [b for b in range(w.batch) if bool(has_new[b])]
    slots = torch.stack([p.geo.slots(b, int(before[b]), 1)[0] for b in sel])
    kvq.quantize_append(twin, k[sel].to(DEV), v[sel].to(DEV), slots.to(DEV))
    out_u = kvq.decode_attention(twin, q.to(DEV), bt, lens_d, maxlen, num_splits=num_splits)
    torch.cuda.synchronize()

    for i, (a, b) in enumerate(zip(p.gpu.planes(), twin.planes())):
        assert torch.equal(a, b), f"{name}: plane {i} differs from the separate append"
    assert torch.equal(out_f, out_u), f"{name}: output differs from append + decode"

    p.ref.append(wl.bf16_bits(k[sel]), wl.bf16_bits(v[sel]), slots.numpy())
    assert planes_equal(p) == []
    want = p.ref.decode(wl.bf16_bits(q), p.geo.block_table.numpy(), lens.numpy(), 0.0)
    got = out_f.cpu().numpy().astype(np.float64)
    err = max_err(got, want)
    print(f"[step] {name}: max_abs_err {err:.3g}", flush=True)
    assert err <= TOL
    for b in range(w.batch):
        if int(lens[b]) == 0:
            assert np.all(got[b] == 0)


@pytest.mark.parametrize("name", list(CASES))
def test_decode_step_matches_append_then_decode(name):
    _run_case(name)


def test_decode_step_repeated_steps():
    """Three steps in a row on one cache, each appending the next token: the cache and the
    outputs track the unfused sequence of calls."""
    w = _small("c5", batch=4, ragged=(5, 120))
    lens0 = wl.seq_lens(w)
    print(f"[step] repeated: {w} lens0={lens0.tolist()}", flush=True)
    p = make_pair(w, DEV, extra_tokens=3, lens=lens0, with_oracle=False)
    twin = p.gpu.clone()
    bt = p.geo.block_table.to(DEV)
    lens = lens0.clone()
    for step in range(3):
        k, v = wl.new_tokens(w, step)
        q = wl.queries(w, step)
        slots = torch.stack([p.geo.slots(b, int(lens[b]), 1)[0] for b in range(w.batch)])
        lens += 1
        maxlen = int(lens.max())
        out_f = kvq.decode_step(p.gpu, k.to(DEV), v.to(DEV), q.to(DEV), bt, lens.to(DEV), maxlen)
        kvq.quantize_append(twin, k.to(DEV), v.to(DEV), slots.to(DEV))
        out_u = kvq.decode_attention(twin, q.to(DEV), bt, lens.to(DEV), maxlen)
        torch.cuda.synchronize()
        assert torch.equal(out_f, out_u), f"step {step}"
        for a, b in zip(p.gpu.planes(), twin.planes()):
            assert torch.equal(a, b), f"step {step}"


def test_decode_step_timed_and_errors():
    w = _small("c2", batch=2, context=100)
    p = make_pair(w, DEV, extra_tokens=1, with_oracle=False)
    k, v = wl.new_tokens(w, 0)
    lens = (p.lens + 1).to(DEV)
    q = wl.queries(w).to(DEV)
    bt = p.geo.block_table.to(DEV)
    ev = EventPair()
    twin = p.gpu.clone()
    out_t = kvq.decode_step(p.gpu, k.to(DEV), v.to(DEV), q, bt, lens, int(lens.max()), events=ev.handles())
    out_p = kvq.decode_step(twin, k.to(DEV), v.to(DEV), q, bt, lens, int(lens.max()))
    torch.cuda.synchronize()
    assert ev.elapsed_ms() > 0
    ev.close()
    assert torch.equal(out_t, out_p)
    with pytest.raises(ValueError):
        kvq.decode_step(p.gpu, k[:1].to(DEV), v.to(DEV), q, bt, lens, int(lens.max()))
