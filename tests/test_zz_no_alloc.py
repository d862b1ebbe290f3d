"""kvq_decode_attention_noalloc (the decode call whose workspace is a device array the
library owns) against kvq_decode_attention, through the C ABI: two calls in a row, the
second on a smaller input, each bit-equal to the workspace-taking call on the same cache
and query (same kernels, same partition plan), and within the parity bound of the oracle.
A call whose workspace would not fit the array is refused before any launch."""
import numpy as np
import pytest
import torch

import bit_kv_cache_quantize_amd as kvq
import workloads as wl
from kvq_harness import TOL, decode_both, make_pair, max_err

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _call_both(p, q):
    bt, lens = p.geo.block_table.to(DEV), p.lens.to(DEV)
    maxlen = int(p.lens.max())
    B, Hq = q.shape[0], q.shape[1]
    want = kvq.decode_attention(p.gpu, q, bt, lens, maxlen)
    out = torch.full((B, Hq, 128), float("nan"), dtype=torch.float32, device=DEV)
    got = kvq.decode_attention_noalloc(p.gpu, q, bt, lens, maxlen, out)
    torch.cuda.synchronize()
    return got.cpu(), want.cpu()


def test_noalloc_matches_workspace_call_twice():
    cases = [("c5 paged ragged, balanced partitions", wl.get("c5").with_(batch=24, ragged=(200, 3000))),
             ("c2 shape, one sequence, fixed partitions", wl.get("c2").with_(batch=1, context=700))]
    for label, w in cases:
        print(f"[noalloc] {label}: {w}", flush=True)
        p = make_pair(w, DEV)
        q = wl.queries(w)
        got, want = _call_both(p, q.to(DEV))
        assert torch.equal(got, want), label
        _, ref = decode_both(p, DEV, q=q)
        assert max_err(got.numpy().astype(np.float64), ref) <= TOL, label


def test_noalloc_refuses_oversized_workspace():
    """B = 1 with 32768 fixed partitions would need 32 heads x 32768 x 520 B of partials,
    past the 32 MiB array: KVQ_ERR_WORKSPACE, returned on the host before any launch."""
    w = wl.get("c2").with_(batch=1, context=64)
    p = make_pair(w, DEV, with_oracle=False)
    q = wl.queries(w).to(DEV)
    out = torch.empty((1, 32, 128), dtype=torch.float32, device=DEV)
    bt = torch.zeros((1, 1 << 16), dtype=torch.int32, device=DEV)
    lens = p.lens.to(DEV)
    with pytest.raises(kvq.KVQError) as e:
        kvq.decode_attention_noalloc(p.gpu, q, bt, lens, 1 << 20, out, num_splits=1 << 15)
    assert e.value.status == kvq.ERR_WORKSPACE
