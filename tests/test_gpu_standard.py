"""GPU parity for the standard (non-split) QKV mode -- Phase 2, "Standard QKV
Optimization": Q, K, V of the deduplicated batch reconstructed to the full
batch, standard per-sample causal attention there, the output brought back.

* the full-batch plan (every sample its own group) is bit-exact with the
  oracle's packing of singleton groups;
* moving rows between the two layouts is bit-exact with the oracle's
  reconstruct-then-pack, and its transpose matches the oracle's transposes;
* the attention result equals split attention's, so it is checked against the
  same oracle (the non-deduplicated per-sample definition) at the same
  tolerances.
"""
import numpy as np
import pytest

import oracle
from helpers import attn_inputs, compare, gpu_plan, oracle_plan, say, to_numpy
from workloads import WORKLOADS, make_batch

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

_base = WORKLOADS["tiny_fp32"]
PLAN_CASES = [
    _base,
    _base.scaled(name="ragged_unpad", num_prompts=3, rollout_n=5, prompt_len=300, response_len=77,
                 resp_len_range=(0, 77), seed=21),
    _base.scaled(name="singletons", num_prompts=7, rollout_n=1, prompt_len=5, response_len=3, seed=22),
    WORKLOADS["qwen3_0p6b_2x8_p8192_r512"],
    WORKLOADS["long_2x8_p32768_r256to1024_unpad"],
]
ATTN_CASES = {
    "tiny_fp32": _base,
    "bf16_gqa2_ragged_unpad": _base.scaled(name="bf16_gqa2_ragged_unpad", num_prompts=2, rollout_n=3, prompt_len=300,
                                           response_len=77, num_q_heads=4, num_kv_heads=2, head_dim=128,
                                           dtype="bf16", sigma=0.5, resp_len_range=(0, 77), seed=32),
    "bf16_mid_2x4_p2048_r512": _base.scaled(name="bf16_mid_2x4_p2048_r512", num_prompts=2, rollout_n=4,
                                            prompt_len=2048, response_len=512, num_q_heads=16, num_kv_heads=8,
                                            head_dim=128, dtype="bf16", sigma=0.5, vocab=151936, seed=39),
}


def _oracle_full(bt, use_unpad):
    B, P = bt.input_ids.shape[0], bt.input_ids.shape[1] - bt.response_length
    return oracle.create_deduplicated_batch(bt.input_ids, bt.position_ids, bt.response_length,
                                            [[b] for b in range(B)], bt.input_ids[:, :P],
                                            attention_mask=bt.attention_mask, use_unpad=use_unpad)


def _gpu_full(bt, use_unpad):
    import shared_prompt_dedup_amd as spd
    ids = torch.from_numpy(bt.input_ids).cuda()
    pos = torch.from_numpy(bt.position_ids).cuda()
    mask = torch.from_numpy(bt.attention_mask).cuda()
    return spd.create_full_batch(ids, pos, bt.response_length, attention_mask=mask if use_unpad else None,
                                 use_unpad=use_unpad)


@pytest.mark.parametrize("w", PLAN_CASES, ids=[w.name for w in PLAN_CASES])
def test_full_batch_plan_bit_exact(w):
    say(f"[standard] full-batch plan {w.name}")
    bt = make_batch(w, permute=True)
    oids, opos, oinfo = _oracle_full(bt, w.use_unpad)
    gids, gpos, ginfo = _gpu_full(bt, w.use_unpad)
    assert ginfo["G"] == oinfo["G"] == w.batch and ginfo["T"] == oinfo["T"]
    np.testing.assert_array_equal(gids.cpu().numpy(), oids)
    np.testing.assert_array_equal(gpos.cpu().numpy(), opos)
    p, T = ginfo.plan, oinfo["T"]
    for f in ("group_of", "rep", "prompt_off", "prompt_len", "resp_off", "resp_len", "dst"):
        np.testing.assert_array_equal(getattr(p, f).cpu().numpy(), oinfo[f], err_msg=f)
    for f in ("src", "seg_start"):
        np.testing.assert_array_equal(getattr(p, f)[:T].cpu().numpy(), oinfo[f], err_msg=f)
    np.testing.assert_array_equal(p.grp_off.cpu().numpy(), np.arange(w.batch + 1))
    np.testing.assert_array_equal(p.grp_idx.cpu().numpy(), np.arange(w.batch))


@pytest.mark.parametrize("w", PLAN_CASES, ids=[w.name for w in PLAN_CASES])
def test_repack_rows_both_ways(w):
    """Rows between the deduplicated and the full layout, and the transposes."""
    import shared_prompt_dedup_amd as spd
    say(f"[standard] repack rows {w.name}")
    bt = make_batch(w, permute=True)
    _, _, _, _, od = oracle_plan(bt, w.use_unpad)
    _, _, of = _oracle_full(bt, w.use_unpad)
    _, _, _, _, gd = gpu_plan(bt, w.use_unpad)
    _, _, gf = _gpu_full(bt, w.use_unpad)
    rng = np.random.default_rng(3)
    W = 12
    # forward, bytes: dedup -> full and full -> dedup
    x = rng.integers(-2**31, 2**31 - 1, size=(od["T"], W), dtype=np.int64).astype(np.int32)
    got = spd.repack_rows(torch.from_numpy(x).cuda(), gf, gd).cpu().numpy()
    np.testing.assert_array_equal(got, oracle.pack_rows(oracle.reconstruct_sequences(x, od), of))
    y = rng.integers(-2**31, 2**31 - 1, size=(of["T"], W), dtype=np.int64).astype(np.int32)
    got = spd.repack_rows(torch.from_numpy(y).cuda(), gd, gf).cpu().numpy()
    np.testing.assert_array_equal(got, oracle.pack_rows(oracle.reconstruct_sequences(y, of), od))
    # transposes, fp32 and bf16 (full -> dedup sums each prompt row over the members' copies)
    nmax = w.rollout_n
    for dt in (torch.float32, torch.bfloat16):
        gfull = rng.standard_normal((of["T"], 16)).astype(np.float32)
        gfull = torch.from_numpy(gfull).to(dt).float().numpy()
        got = spd.repack_rows_bwd(torch.from_numpy(gfull).to("cuda", dt), gf, gd).float().cpu().numpy()
        ref = oracle.reconstruct_backward(oracle.pack_rows_backward(gfull, of), od)
        absum = oracle.reconstruct_backward(oracle.pack_rows_backward(np.abs(gfull), of), od)
        bound = (nmax - 1) * 2.0**-24 * absum + (2.0**-8 * np.abs(ref) if dt == torch.bfloat16 else 0.0)
        assert (np.abs(got - ref) <= bound + 1e-30).all()
        gded = torch.from_numpy(rng.standard_normal((od["T"], 16)).astype(np.float32)).to(dt)
        got = spd.repack_rows_bwd(gded.cuda(), gd, gf).float().cpu().numpy()
        ref = oracle.reconstruct_backward(oracle.pack_rows_backward(gded.float().numpy(), od), of)
        np.testing.assert_array_equal(got, ref)   # one term per row: exact


@pytest.mark.parametrize("name", list(ATTN_CASES))
def test_standard_attention_matches_oracle_and_split(name):
    import shared_prompt_dedup_amd as spd
    w = ATTN_CASES[name]
    say(f"[standard] attention {name} dtype={w.dtype}")
    bt = make_batch(w, permute=True)
    _, _, _, _, oinfo = oracle_plan(bt, w.use_unpad)
    _, _, _, _, ginfo = gpu_plan(bt, w.use_unpad)
    _, _, finfo = _gpu_full(bt, w.use_unpad)
    x, q, k, v, do = attn_inputs(w, oinfo["T"])
    qg, kg, vg = (t.clone().requires_grad_() for t in (q, k, v))
    o = spd.standard_attention(qg, kg, vg, ginfo, finfo)
    o.backward(do)
    ro, _ = oracle.split_attention_forward(x.q, x.k, x.v, oinfo)
    rdq, rdk, rdv = oracle.split_attention_backward(x.q, x.k, x.v, x.do, oinfo)
    for key, got, ref in (("o", o.detach(), ro), ("dq", qg.grad, rdq), ("dk", kg.grad, rdk), ("dv", vg.grad, rdv)):
        compare(f"standard {key}", to_numpy(got), ref, w.dtype)
    # the split path on the same inputs: same forward output for every row
    so, _ = spd.split_attn_fwd(q, k, v, ginfo)
    compare("standard o vs split o", to_numpy(o.detach()), to_numpy(so), w.dtype)
