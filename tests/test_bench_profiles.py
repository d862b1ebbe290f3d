"""The benchmark's `roofline.traffic` comes only from counter runs of the same split-kernel
configuration on the same kernel source (CPU; reads the committed profiles)."""
from __future__ import annotations

import argparse
import glob
import json
import os

import bench


def _args(**kw):
    base = dict(workload="h1", prune=0, window="", vgroup=False, hybrid=False, hadamard_block=-1, num_splits=0,
                unfused=False, page_size=-1)
    base.update(kw)
    return argparse.Namespace(**base)


def test_profile_keys_name_every_variant():
    assert bench.profile_key(_args()) == "h1"
    assert bench.profile_key(_args(workload="c5")) == "c5"
    assert bench.profile_key(_args(prune=2)) == "h1_prune2"
    assert bench.profile_key(_args(window="32,128")) == "h1_window32x128"
    assert bench.profile_key(_args(vgroup=True)) == "h1_vgroup"
    assert bench.profile_key(_args(hybrid=True)) == "h1_hybrid"
    assert bench.profile_key(_args(hadamard_block=32)) == "h1_hb32"
    assert bench.profile_key(_args(num_splits=8)) == "h1_splits8"
    assert bench.profile_key(_args(prune=3, num_splits=16)) == "h1_prune3_splits16"
    assert bench.profile_key(_args(unfused=True)) == "h1_unfused"
    assert bench.profile_key(_args(workload="c2", unfused=True)) == "c2_unfused"
    assert bench.profile_key(_args(workload="c4", page_size=16)) == "c4_p16"


def test_traffic_only_from_matching_profiles():
    sha = bench.kernel_source_sha()
    paths = glob.glob(os.path.join(bench.ROOT, "profiles", "decode_split_*_traffic.json"))
    assert paths, "no committed traffic profiles"
    for path in paths:
        key = os.path.basename(path)[len("decode_split_"):-len("_traffic.json")]
        with open(path) as f:
            t = json.load(f)
        assert t["workload"] == key
        want = t["hbm_bytes_per_launch"] if t["kernel_source_sha"] == sha else None
        assert bench.traffic_from_profile(key) == want
        if want is not None:
            # counters within a few percent of the algorithmic bytes; the widest case is
            # INT2 g128 on 16-token pages (c4_p16), where a tile's 64-byte {scale, zero}
            # block fills half a 128-byte line (8 B of 72 B per token read twice over)
            assert 0.99 < t["traffic_over_algorithmic"] < 1.13, (key, t["traffic_over_algorithmic"])
    # a configuration without its own counter runs reports none (never another's figure)
    assert bench.traffic_from_profile("h1_prune1") is None
    assert bench.traffic_from_profile("h1_splits8") is None
