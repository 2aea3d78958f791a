"""Host logic of bench.py (CPU only).

`value` is the split attention's useful work per step over the step time; its
numerator comes from bench.attended_pairs, which counts (query, key) pairs from
the plan's segment lengths.  Here that count is checked against the oracle's
(itself pinned by brute force over the visibility rule) on the seeded batches
the bench runs, built and packed by the oracle; and a request for more than
one GPU is refused before anything touches a device.
"""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import bench
import oracle
from workloads import WORKLOADS, make_batch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench_info(info):
    """The fields bench.attended_pairs reads, in the binding's form (tensors)."""
    out = {
        "G": info["G"],
        "prompt_len": torch.tensor(np.asarray(info["prompt_len"], dtype=np.int32)),
        "resp_len": torch.tensor(np.asarray(info["resp_len"], dtype=np.int32)),
        "group_of": torch.tensor(np.asarray(info["group_of"], dtype=np.int32)),
    }
    if info.get("prefix_len", 0):
        out["prefix_len"] = info["prefix_len"]
    return out


@pytest.mark.parametrize("name,share_prefix", [
    ("long_2x8_p32768_r256to1024_unpad", False),
    ("qwen3_0p6b_2x8_p8192_r512", False),
    ("redundancy_1x10_p10240_r1024", False),
    ("bwd_4x8_p4096_r1024", False),
    ("prefix_4x8_s4096_p5120_r512", False),
    ("prefix_4x8_s4096_p5120_r512", True),
])
def test_flop_count_matches_oracle(name, share_prefix):
    w = WORKLOADS[name]
    bt = make_batch(w)
    groups, uniq = oracle.find_prompt_groups(bt.input_ids, bt.response_length)
    lp = oracle.find_shared_prefix(bt.input_ids, bt.response_length, groups) if share_prefix else 0
    _, _, info = oracle.create_deduplicated_batch(bt.input_ids, bt.position_ids, bt.response_length, groups, uniq,
                                                  attention_mask=bt.attention_mask, use_unpad=w.use_unpad,
                                                  prefix_len=lp)
    if share_prefix:
        assert info["prefix_len"] > 0
    dedup, plain = oracle.attended_pairs(info)
    assert bench.attended_pairs(_bench_info(info)) == dedup
    assert dedup < plain


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
