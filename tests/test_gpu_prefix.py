"""GPU parity for prefix sharing (Key Limitations & Future Work: prefix caching
for partially overlapping prompts): the prompts' common prefix is packed once,
ahead of every group.  Plans and row moves bit-exact with the oracle;
attention (forward and backward) against the same non-deduplicated oracle and
tolerances as split attention."""
import numpy as np
import pytest

import oracle
from helpers import attn_inputs, compare, say, to_numpy
from workloads import WORKLOADS, make_batch

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

_base = WORKLOADS["tiny_fp32"]
PLAN_CASES = [
    _base.scaled(name="px_small", num_prompts=3, rollout_n=2, prompt_len=40, response_len=12, shared_prefix=23,
                 seed=71),
    _base.scaled(name="px_unpad", num_prompts=4, rollout_n=3, prompt_len=300, response_len=77, shared_prefix=129,
                 resp_len_range=(0, 77), seed=72),
    _base.scaled(name="px_one_group", num_prompts=1, rollout_n=4, prompt_len=30, response_len=10, seed=73),
    _base.scaled(name="px_none", num_prompts=3, rollout_n=2, prompt_len=30, response_len=10, seed=74),
    WORKLOADS["prefix_4x8_s4096_p5120_r512"],
]
ATTN_CASES = {
    "px_f32": _base.scaled(name="px_f32", num_prompts=3, rollout_n=2, prompt_len=150, response_len=45, shared_prefix=70,
                           num_q_heads=4, num_kv_heads=2, head_dim=128, resp_len_range=(0, 45), seed=75),
    "px_bf16": _base.scaled(name="px_bf16", num_prompts=3, rollout_n=3, prompt_len=420, response_len=100,
                            shared_prefix=300, num_q_heads=4, num_kv_heads=2, head_dim=128, dtype="bf16", sigma=0.5,
                            resp_len_range=(1, 100), seed=76),
    "px_bf16_d64": _base.scaled(name="px_bf16_d64", num_prompts=2, rollout_n=4, prompt_len=200, response_len=70,
                                shared_prefix=129, num_q_heads=8, num_kv_heads=2, head_dim=64, dtype="bf16",
                                sigma=0.5, seed=77),
}


def _plans(bt, use_unpad):
    import shared_prompt_dedup_amd as spd
    groups, uniq = oracle.find_prompt_groups(bt.input_ids, bt.response_length)
    L0 = oracle.find_shared_prefix(bt.input_ids, bt.response_length, groups)
    odids, odpos, oinfo = oracle.create_deduplicated_batch(bt.input_ids, bt.position_ids, bt.response_length, groups,
                                                           uniq, attention_mask=bt.attention_mask,
                                                           use_unpad=use_unpad, prefix_len=L0)
    ids, pos, mask = (torch.from_numpy(a).cuda() for a in (bt.input_ids, bt.position_ids, bt.attention_mask))
    gg, gu = spd.find_prompt_groups(ids, bt.response_length)
    gdids, gdpos, ginfo = spd.create_deduplicated_batch(ids, pos, bt.response_length, gg, gu,
                                                        attention_mask=mask if use_unpad else None,
                                                        use_unpad=use_unpad, share_prefix=True)
    return (odids, odpos, oinfo), (gdids, gdpos, ginfo), (ids, pos, mask)


@pytest.mark.parametrize("w", PLAN_CASES, ids=[w.name for w in PLAN_CASES])
def test_prefix_plan_bit_exact(w):
    say(f"[prefix] plan {w.name}")
    bt = make_batch(w, permute=True)
    (odids, odpos, oinfo), (gdids, gdpos, ginfo), _ = _plans(bt, w.use_unpad)
    assert ginfo["L0"] == oinfo["L0"] and ginfo["prefix_len"] == oinfo["prefix_len"]
    assert ginfo["G"] == oinfo["G"] and ginfo["T"] == oinfo["T"]
    if w.shared_prefix and w.num_prompts > 1:
        assert oinfo["L0"] == w.shared_prefix
    np.testing.assert_array_equal(gdids.cpu().numpy(), odids)
    np.testing.assert_array_equal(gdpos.cpu().numpy(), odpos)
    p, G, T = ginfo.plan, oinfo["G"], oinfo["T"]
    for f in ("prompt_off", "prompt_len", "rep"):
        np.testing.assert_array_equal(getattr(p, f)[:G].cpu().numpy(), oinfo[f], err_msg=f)
    for f in ("group_of", "resp_off", "resp_len", "dst"):
        np.testing.assert_array_equal(getattr(p, f).cpu().numpy(), oinfo[f], err_msg=f)
    for f in ("src", "seg_start"):
        np.testing.assert_array_equal(getattr(p, f)[:T].cpu().numpy(), oinfo[f], err_msg=f)


@pytest.mark.parametrize("L0,P,R", [(1500, 2600, 900), (1024, 1300, 2000)], ids=["prefix_mid_chunk", "prefix_aligned"])
def test_prefix_plan_across_column_chunks(L0, P, R):
    """The shared prefix, the group prompts and the responses packed from
    masks with holes, with the prefix's end inside a column chunk or on its
    boundary: plans bit-exact with the oracle."""
    from test_gpu_dedup import _holey_batch
    bt = _holey_batch(P, R, 3, 2, seed=L0 + P, prefix=L0)
    say(f"[prefix] plan across column chunks L0={L0} P={P}")
    (odids, odpos, oinfo), (gdids, gdpos, ginfo), _ = _plans(bt, True)
    assert oinfo["L0"] >= L0 and ginfo["L0"] == oinfo["L0"] and ginfo["T"] == oinfo["T"]
    np.testing.assert_array_equal(gdids.cpu().numpy(), odids)
    np.testing.assert_array_equal(gdpos.cpu().numpy(), odpos)
    p, G, T = ginfo.plan, oinfo["G"], oinfo["T"]
    for f in ("prompt_off", "prompt_len", "rep"):
        np.testing.assert_array_equal(getattr(p, f)[:G].cpu().numpy(), oinfo[f], err_msg=f)
    for f in ("group_of", "resp_off", "resp_len", "dst"):
        np.testing.assert_array_equal(getattr(p, f).cpu().numpy(), oinfo[f], err_msg=f)
    for f in ("src", "seg_start"):
        np.testing.assert_array_equal(getattr(p, f)[:T].cpu().numpy(), oinfo[f], err_msg=f)


@pytest.mark.parametrize("w", PLAN_CASES[:2] + PLAN_CASES[-1:], ids=[w.name for w in PLAN_CASES[:2] + PLAN_CASES[-1:]])
def test_prefix_rows(w):
    import shared_prompt_dedup_amd as spd
    say(f"[prefix] rows {w.name}")
    bt = make_batch(w, permute=True)
    (_, _, oinfo), (_, _, ginfo), _ = _plans(bt, w.use_unpad)
    B, S, T = oinfo["B"], oinfo["S"], oinfo["T"]
    rng = np.random.default_rng(6)
    x = rng.integers(-2**31, 2**31 - 1, size=(T, 8), dtype=np.int64).astype(np.int32)
    np.testing.assert_array_equal(spd.reconstruct(torch.from_numpy(x).cuda(), ginfo).cpu().numpy(),
                                  oracle.reconstruct_sequences(x, oinfo))
    rows = rng.integers(-2**31, 2**31 - 1, size=(B, S, 8), dtype=np.int64).astype(np.int32)
    np.testing.assert_array_equal(spd.pack_rows(torch.from_numpy(rows).cuda(), ginfo).cpu().numpy(),
                                  oracle.pack_rows(rows, oinfo))
    np.testing.assert_array_equal(spd.pack_rows_bwd(torch.from_numpy(x).cuda(), ginfo).cpu().numpy(),
                                  oracle.pack_rows_backward(x, oinfo))
    vals = rng.standard_normal((B, S, 16)).astype(np.float32)
    got = spd.reconstruct_bwd(torch.from_numpy(vals).cuda(), ginfo).cpu().numpy()
    ref = oracle.reconstruct_backward(vals, oinfo)
    bound = (B - 1) * 2.0**-24 * oracle.reconstruct_backward(np.abs(vals), oinfo)
    assert (np.abs(got - ref) <= bound + 1e-30).all()


@pytest.mark.parametrize("name", list(ATTN_CASES))
def test_prefix_attention_small(name):
    import shared_prompt_dedup_amd as spd
    w = ATTN_CASES[name]
    say(f"[prefix] attention {name} dtype={w.dtype}")
    bt = make_batch(w, permute=True)
    (_, _, oinfo), (_, _, ginfo), (ids, pos, mask) = _plans(bt, w.use_unpad)
    assert oinfo["prefix_len"] > 0
    x, q, k, v, do = attn_inputs(w, oinfo["T"])
    o, lse = spd.split_attn_fwd(q, k, v, ginfo)
    dq, dk, dv = spd.split_attn_bwd(q, k, v, o, lse, do, ginfo)
    ro, rlse = oracle.split_attention_forward(x.q, x.k, x.v, oinfo)
    rg = oracle.split_attention_backward(x.q, x.k, x.v, x.do, oinfo)
    compare("o", to_numpy(o), ro, w.dtype)
    compare("lse", lse.cpu().numpy(), rlse, w.dtype)
    for key, got, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), rg):
        compare(key, to_numpy(got), ref, w.dtype)
    # standard mode on top of the prefix plan: same function
    full = spd.create_full_batch(ids, pos, bt.response_length, attention_mask=mask if w.use_unpad else None,
                                 use_unpad=w.use_unpad)[2]
    qg, kg, vg = (t.clone().requires_grad_() for t in (q, k, v))
    so = spd.standard_attention(qg, kg, vg, ginfo, full)
    so.backward(do)
    compare("standard o", to_numpy(so.detach()), ro, w.dtype)
    for key, got, ref in zip(("dq", "dk", "dv"), (qg.grad, kg.grad, vg.grad), rg):
        compare(f"standard {key}", to_numpy(got), ref, w.dtype)


def test_prefix_attention_full_sampled():
    """The 4 x 8 workload whose prompts share 4096 of 5120 tokens: sampled rows and keys, including prefix keys
    read by every sample."""
    import shared_prompt_dedup_amd as spd
    w = WORKLOADS["prefix_4x8_s4096_p5120_r512"]
    bt = make_batch(w)
    (_, _, oinfo), (_, _, ginfo), _ = _plans(bt, False)
    T, Lp = oinfo["T"], oinfo["prefix_len"]
    say(f"[prefix] full: T={T} prefix rows={Lp}")
    x, q, k, v, do = attn_inputs(w, T)
    o, lse = spd.split_attn_fwd(q, k, v, ginfo)
    dq, dk, dv = spd.split_attn_bwd(q, k, v, o, lse, do, ginfo)
    torch.cuda.synchronize()
    f64 = {n: getattr(x, n).astype(np.float64) for n in ("q", "k", "v", "do")}
    rng = np.random.default_rng(3)
    rows = sorted(set([0, 1, Lp // 2, Lp - 1, Lp, Lp + 1] + [int(oinfo["prompt_off"][g]) for g in range(oinfo["G"])]
                      + [int(oinfo["resp_off"][b]) for b in range(3)] + rng.choice(T, 20, replace=False).tolist()))
    heads = [0, w.num_q_heads - 1]
    ro, rl = oracle.forward_rows(f64["q"], f64["k"], f64["v"], oinfo, rows, heads)
    compare("o", to_numpy(o)[rows][:, heads], ro, "bf16")
    rdq = oracle.dq_rows(f64["q"], f64["k"], f64["v"], f64["do"], oinfo, rows[:12], heads)
    compare("dq", to_numpy(dq)[rows[:12]][:, heads], rdq, "bf16")
    # a prefix key is read by all 32 samples: one of them (and a response key) on one kv head keeps the oracle
    # at a few seconds
    keys = [Lp - 1, int(oinfo["resp_off"][0])]
    kvh = [w.num_kv_heads - 1]
    rdk, rdv = oracle.dkdv_rows(f64["q"], f64["k"], f64["v"], f64["do"], oinfo, keys, kvh)
    compare("dk", to_numpy(dk)[keys][:, kvh], rdk, "bf16")
    compare("dv", to_numpy(dv)[keys][:, kvh], rdv, "bf16")
