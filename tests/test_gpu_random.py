"""Randomised GPU parity: small batches drawn from a seeded generator -- group
count, rollouts, prompt and response lengths, padded, unpadded or padded with
a mask, a shared prompt prefix or none, GQA ratio, head dimension, bf16 or
fp32; every fourth also in standard (full-batch) mode -- each
checked end to end against the oracle: plan arrays and packed ids bit-exact,
row moves bit-exact, attention forward and backward within the per-dtype
tolerances (the non-deduplicated per-sample definition)."""
import numpy as np
import pytest

import oracle
from helpers import attn_inputs, compare, say, to_numpy
from workloads import WORKLOADS, make_batch

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

HEADS = [(2, 1, 64), (4, 2, 128), (4, 4, 64), (8, 2, 128), (3, 1, 128), (16, 1, 64), (4, 1, 128)]
SEEDS = list(range(64))


def _config(seed):
    rng = np.random.default_rng(10_000 + seed)
    G = int(rng.integers(1, 5))
    n = int(rng.integers(1, 5))
    P = int(rng.integers(1, 260))
    R = int(rng.integers(1, 90))
    hq, hkv, d = HEADS[int(rng.integers(len(HEADS)))]
    dtype = "f32" if rng.random() < 0.2 else "bf16"
    if dtype == "f32":
        # the fp32 bound (max-abs 1e-5) is for small problems: fp32 rounding of a sum grows with its terms, and a
        # key read by hundreds of rows and several query heads sums thousands of them
        G, n, P, R = min(G, 2), min(n, 4), min(P, 128), min(R, 64)
        hq, hkv, d = HEADS[int(rng.integers(3))]
    # packed format: padded without a mask, unpadded, or padded with a mask (pads kept, no part in attention)
    fmt = ("padded", "unpad", "padded_mask")[int(rng.choice(3, p=[0.35, 0.35, 0.3]))]
    prefix = int(rng.integers(1, P + 1)) if (G >= 2 and rng.random() < 0.35) else 0
    w = WORKLOADS["tiny_fp32"].scaled(
        name=f"random_{seed}", num_prompts=G, rollout_n=n, prompt_len=P, response_len=R, num_q_heads=hq,
        num_kv_heads=hkv, head_dim=d, dtype=dtype, sigma=0.5 if dtype == "bf16" else 1.0,
        resp_len_range=None if fmt == "padded" else (0, R), shared_prefix=prefix, seed=20_000 + seed)
    return w, fmt, prefix > 0


def _config_medium(seed):
    """Larger bf16 batches: prompts of hundreds to thousands of tokens, so key tiles are read by more rows than
    a CU's share and the backward splits them into chunks."""
    rng = np.random.default_rng(30_000 + seed)
    G = int(rng.integers(1, 4))
    n = int(rng.integers(2, 13 // G + 1))
    P = int(rng.integers(400, 2600))
    R = int(rng.integers(40, 500))
    hq, hkv, d = [(2, 1, 128), (4, 2, 64), (4, 1, 128), (2, 2, 128)][int(rng.integers(4))]
    fmt = ("padded", "unpad", "padded_mask")[seed % 3]
    prefix = int(rng.integers(1, P)) if (G >= 2 and rng.random() < 0.5) else 0
    w = WORKLOADS["tiny_fp32"].scaled(
        name=f"random_medium_{seed}", num_prompts=G, rollout_n=n, prompt_len=P, response_len=R, num_q_heads=hq,
        num_kv_heads=hkv, head_dim=d, dtype="bf16", sigma=0.5, vocab=151936,
        resp_len_range=None if fmt == "padded" else (R // 4, R), shared_prefix=prefix, seed=40_000 + seed)
    return w, fmt, prefix > 0


@pytest.mark.parametrize("seed", SEEDS)
def test_random_batch_end_to_end(seed):
    _end_to_end(seed, *_config(seed))


@pytest.mark.parametrize("seed", range(6))
def test_random_medium_batch_end_to_end(seed):
    _end_to_end(seed, *_config_medium(seed))


def _end_to_end(seed, w, fmt, share):
    import shared_prompt_dedup_amd as spd
    unpad = fmt == "unpad"
    say(f"[random {seed}] G={w.num_prompts} n={w.rollout_n} P={w.prompt_len} R={w.response_len} "
        f"{fmt} prefix={w.shared_prefix} heads={w.num_q_heads}/{w.num_kv_heads}/{w.head_dim} {w.dtype}")
    bt = make_batch(w, permute=True)
    groups, uniq = oracle.find_prompt_groups(bt.input_ids, bt.response_length)
    L0 = oracle.find_shared_prefix(bt.input_ids, bt.response_length, groups) if share else 0
    odids, odpos, oinfo = oracle.create_deduplicated_batch(bt.input_ids, bt.position_ids, bt.response_length, groups,
                                                           uniq, attention_mask=bt.attention_mask,
                                                           use_unpad=unpad, prefix_len=L0)
    ids, pos, mask = (torch.from_numpy(a).cuda() for a in (bt.input_ids, bt.position_ids, bt.attention_mask))
    gg, gu = spd.find_prompt_groups(ids, bt.response_length)
    assert [list(x) for x in gg] == [list(x) for x in groups]
    gmask = None if fmt == "padded" else mask
    gdids, gdpos, ginfo = spd.create_deduplicated_batch(ids, pos, bt.response_length, gg, gu, attention_mask=gmask,
                                                        use_unpad=unpad, share_prefix=share)
    T = oinfo["T"]
    assert ginfo["T"] == T and ginfo["G"] == oinfo["G"] and ginfo["prefix_len"] == oinfo["prefix_len"]
    np.testing.assert_array_equal(gdids.cpu().numpy(), odids)
    np.testing.assert_array_equal(gdpos.cpu().numpy(), odpos)
    p = ginfo.plan
    for f in ("group_of", "resp_off", "resp_len", "dst"):
        np.testing.assert_array_equal(getattr(p, f).cpu().numpy(), oinfo[f], err_msg=f)
    for f in ("src", "seg_start"):
        np.testing.assert_array_equal(getattr(p, f)[:T].cpu().numpy(), oinfo[f], err_msg=f)
    # row moves, bit-exact
    rng = np.random.default_rng(seed)
    B, S = oinfo["B"], oinfo["S"]
    x = rng.integers(-2**31, 2**31 - 1, size=(T, 4), dtype=np.int64).astype(np.int32)
    np.testing.assert_array_equal(spd.reconstruct(torch.from_numpy(x).cuda(), ginfo).cpu().numpy(),
                                  oracle.reconstruct_sequences(x, oinfo))
    np.testing.assert_array_equal(spd.pack_rows_bwd(torch.from_numpy(x).cuda(), ginfo).cpu().numpy(),
                                  oracle.pack_rows_backward(x, oinfo))
    rows = rng.integers(-2**31, 2**31 - 1, size=(B, S, 4), dtype=np.int64).astype(np.int32)
    np.testing.assert_array_equal(spd.pack_rows(torch.from_numpy(rows).cuda(), ginfo).cpu().numpy(),
                                  oracle.pack_rows(rows, oinfo))
    if T == 0:
        return
    # attention, forward and backward; with the padded format and a mask, pad rows are no keys and output 0
    valid = bt.attention_mask.reshape(-1)[oinfo["src"]] != 0 if fmt == "padded_mask" else None
    xa, q, k, v, do = attn_inputs(w, T)
    o, lse = spd.split_attn_fwd(q, k, v, ginfo)
    dq, dk, dv = spd.split_attn_bwd(q, k, v, o, lse, do, ginfo)
    ro, rlse = oracle.split_attention_forward(xa.q, xa.k, xa.v, oinfo, valid=valid)
    rgrads = oracle.split_attention_backward(xa.q, xa.k, xa.v, xa.do, oinfo, valid=valid)
    compare("o", to_numpy(o), ro, w.dtype)
    compare("lse", lse.cpu().numpy(), rlse if valid is None else rlse[:, valid], w.dtype)
    for key, got, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), rgrads):
        compare(key, to_numpy(got), ref, w.dtype)
    if seed % 4 == 0:       # standard mode (attention on the full batch) on the same plan: same function
        full = spd.create_full_batch(ids, pos, bt.response_length, attention_mask=gmask, use_unpad=unpad)[2]
        qg, kg, vg = (t.clone().requires_grad_() for t in (q, k, v))
        so = spd.standard_attention(qg, kg, vg, ginfo, full)
        so.backward(do)
        compare("standard o", to_numpy(so.detach()), ro, w.dtype)
        for key, got, ref in zip(("dq", "dk", "dv"), (qg.grad, kg.grad, vg.grad), rgrads):
            compare(f"standard {key}", to_numpy(got), ref, w.dtype)
