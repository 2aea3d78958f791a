"""Shared helpers for the GPU parity tests: run the HIP path through the
binding and the oracle on the same seeded inputs, and compare."""
from __future__ import annotations

import sys

import numpy as np

import oracle
from workloads import Workload, make_attn_inputs, make_batch

# Tolerances for floating point, per dtype: max |gpu - oracle| and relative L2.
TOL = {"f32": dict(max_abs=1e-5, rel_l2=None), "bf16": dict(max_abs=2e-2, rel_l2=5e-3)}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_numpy(t):
    import torch
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


def oracle_plan(bt, use_unpad):
    groups, uniq = oracle.find_prompt_groups(bt.input_ids, bt.response_length)
    dids, dpos, info = oracle.create_deduplicated_batch(
        bt.input_ids, bt.position_ids, bt.response_length, groups, uniq,
        attention_mask=bt.attention_mask, use_unpad=use_unpad)
    return groups, uniq, dids, dpos, info


def gpu_plan(bt, use_unpad, mask_dtype=None, device="cuda"):
    import torch
    import shared_prompt_dedup_amd as spd
    ids = torch.from_numpy(bt.input_ids).to(device)
    pos = torch.from_numpy(bt.position_ids).to(device)
    mask = torch.from_numpy(bt.attention_mask).to(device)
    if mask_dtype is not None:
        mask = mask.to(mask_dtype)
    groups, uniq = spd.find_prompt_groups(ids, bt.response_length)
    dids, dpos, info = spd.create_deduplicated_batch(ids, pos, bt.response_length, groups, uniq,
                                                     attention_mask=mask if use_unpad else None,
                                                     use_unpad=use_unpad)
    return groups, uniq, dids, dpos, info


def attn_inputs(w: Workload, T: int, device="cuda"):
    """(numpy AttnInputs, torch q, k, v, dout) with the GPU tensors bit-equal to the numpy values."""
    import torch
    x = make_attn_inputs(w, T)
    if w.dtype == "bf16":
        conv = lambda bits: torch.from_numpy(bits.view(np.int16)).to(device).view(torch.bfloat16)
        return x, conv(x.q_bits), conv(x.k_bits), conv(x.v_bits), conv(x.do_bits)
    conv = lambda a: torch.from_numpy(a).to(device)
    return x, conv(x.q), conv(x.k), conv(x.v), conv(x.do)


def compare(name, got, ref, dtype, where="", max_abs_tol=None):
    """Assert the per-dtype tolerance; returns (max_abs, rel_l2)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{name}: non-finite values {where}"
    diff = got - ref
    max_abs = float(np.max(np.abs(diff))) if diff.size else 0.0
    den = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(diff) / den) if den > 0 else float(np.linalg.norm(diff))
    tol = dict(TOL[dtype])
    if max_abs_tol is not None:
        tol["max_abs"] = max_abs_tol
    say(f"  {name}{where}: max_abs={max_abs:.3e} rel_l2={rel:.3e}")
    assert max_abs <= tol["max_abs"], f"{name}{where}: max_abs {max_abs} > {tol['max_abs']}"
    if tol["rel_l2"] is not None:
        assert rel <= tol["rel_l2"], f"{name}{where}: rel_l2 {rel} > {tol['rel_l2']}"
    return max_abs, rel
