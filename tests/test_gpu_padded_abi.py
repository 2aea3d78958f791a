"""The padded format with an attention mask at the C ABI (How Prompt Deduplication Works -- Working with
Packed/Unpacked Sequences: pads stay in the packed sequence and take no part in attention).

Raw ctypes calls only, no binding logic: spd_pack marks such a plan (padded_with_mask = 1) and both attention
calls refuse it; the documented path -- the same groups packed without pads (a second plan), rows moved by
spd_repack_rows, attention there, rows moved back -- matches the oracle's masked definition.
"""
import ctypes
import dataclasses
import math

import numpy as np
import pytest

import oracle
from helpers import attn_inputs, compare, say, to_numpy
from workloads import WORKLOADS, make_batch

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

OK, UNSUPPORTED = 0, -2
FIELDS = ("group_of", "grp_off", "grp_idx", "rep", "prompt_off", "prompt_len", "resp_off", "resp_len", "src", "dst",
          "seg_start", "counts")


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


class RawPlan:
    """Caller-owned plan arrays (capacities from B and S only) and the spd_plan struct that points at them."""

    def __init__(self, B, S, P, lib_mod):
        i32 = dict(dtype=torch.int32, device="cuda")
        n = B * S
        sizes = dict(group_of=B, grp_off=B + 1, grp_idx=B, rep=B, prompt_off=B, prompt_len=B, resp_off=B,
                     resp_len=B, src=n, dst=n, seg_start=n, counts=8)
        self.t = {f: torch.zeros(sizes[f], **i32) for f in FIELDS}
        self.c = lib_mod.SpdPlan(B, S, P, *[self.t[f].data_ptr() for f in FIELDS])


def test_raw_c_calls_on_padded_plan_with_mask():
    from shared_prompt_dedup_amd import _lib as L
    lib = L.lib
    w = WORKLOADS["tiny_fp32"].scaled(name="padded_abi", num_prompts=2, rollout_n=3, prompt_len=300,
                                      response_len=77, num_q_heads=4, num_kv_heads=2, head_dim=128, dtype="bf16",
                                      sigma=0.5, resp_len_range=(0, 77), seed=32)
    bt = make_batch(w, permute=True)
    groups, uniq = oracle.find_prompt_groups(bt.input_ids, bt.response_length)
    mask = bt.attention_mask.copy()
    mask[groups[0], :4] = 0                      # left pads on group 0's prompt, right pads in the responses
    bt = dataclasses.replace(bt, attention_mask=mask)
    _, _, oinfo = oracle.create_deduplicated_batch(bt.input_ids, bt.position_ids, bt.response_length, groups, uniq,
                                                   attention_mask=mask, use_unpad=False)
    valid = mask.reshape(-1)[oinfo["src"]] != 0
    B, S = bt.input_ids.shape
    R = bt.response_length
    P = S - R
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    ids, pos, m = (torch.from_numpy(a).cuda() for a in (bt.input_ids, bt.position_ids, mask))

    plan = RawPlan(B, S, P, L)
    gws = torch.empty(lib.spd_group_workspace_bytes(B, S), dtype=torch.uint8, device="cuda")
    assert lib.spd_group(_p(ids), B, S, R, ctypes.byref(plan.c), None, _p(gws), gws.numel(), st) == OK
    pws = torch.empty(lib.spd_pack_workspace_bytes(B, S), dtype=torch.uint8, device="cuda")
    dids = torch.empty(B * S, dtype=torch.int64, device="cuda")
    dpos = torch.empty(B * S, dtype=torch.int64, device="cuda")
    assert lib.spd_pack(_p(ids), _p(pos), _p(m), 8, 0, ctypes.byref(plan.c), _p(dids), _p(dpos), _p(pws),
                        pws.numel(), st) == OK
    assert plan.c.padded_with_mask == 1
    counts = plan.t["counts"].cpu().tolist()
    T, kept = counts[1], counts[3]
    say(f"[padded abi] T={T} kept pads={kept} (oracle: T={oinfo['T']}, pads={int((~valid).sum())})")
    assert T == oinfo["T"] and kept == int((~valid).sum()) > 4

    x, q, k, v, do = attn_inputs(w, T)
    Hq, Hkv, d = w.num_q_heads, w.num_kv_heads, w.head_dim
    desc = L.SpdAttnDesc(Hq, Hkv, d, L.SPD_BF16, 1.0 / math.sqrt(d))
    o = torch.empty_like(q)
    lse = torch.empty((Hq, T), dtype=torch.float32, device="cuda")
    fws = torch.empty(lib.spd_attn_fwd_workspace_bytes(ctypes.byref(desc), B, T), dtype=torch.uint8, device="cuda")
    bws = torch.empty(lib.spd_attn_workspace_bytes(ctypes.byref(desc), B, T), dtype=torch.uint8, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    # the padded plan is refused: its pads would be attended as tokens
    assert lib.spd_split_attn_fwd(ctypes.byref(desc), ctypes.byref(plan.c), T, _p(q), _p(k), _p(v), _p(o), _p(lse),
                                  _p(fws), fws.numel(), st) == UNSUPPORTED
    assert lib.spd_split_attn_bwd(ctypes.byref(desc), ctypes.byref(plan.c), T, _p(q), _p(k), _p(v), _p(o), _p(lse),
                                  _p(do), _p(dq), _p(dk), _p(dv), _p(bws), bws.numel(), st) == UNSUPPORTED

    # the same groups packed without the pads
    twin = RawPlan(B, S, P, L)
    for f in ("group_of", "grp_off", "grp_idx", "rep"):
        twin.t[f].copy_(plan.t[f])
    twin.t["counts"][0] = plan.t["counts"][0]
    tids = torch.empty(B * S, dtype=torch.int64, device="cuda")
    tpos = torch.empty(B * S, dtype=torch.int64, device="cuda")
    assert lib.spd_pack(_p(ids), _p(pos), _p(m), 8, 1, ctypes.byref(twin.c), _p(tids), _p(tpos), _p(pws),
                        pws.numel(), st) == OK
    assert twin.c.padded_with_mask == 0
    Tu = int(twin.t["counts"][1].item())
    assert Tu == int(valid.sum())

    def move(src, to, t_to, fr, t_fr):
        out = torch.empty((t_to,) + tuple(src.shape[1:]), dtype=src.dtype, device="cuda")
        rb = src[0].numel() * src.element_size()
        assert lib.spd_repack_rows(ctypes.byref(to.c), t_to, ctypes.byref(fr.c), t_fr, _p(src), rb, _p(out),
                                   st) == OK
        return out

    qu, ku, vu, dou = (move(t, twin, Tu, plan, T) for t in (q, k, v, do))
    ou = torch.empty_like(qu)
    lu = torch.empty((Hq, Tu), dtype=torch.float32, device="cuda")
    fws = torch.empty(lib.spd_attn_fwd_workspace_bytes(ctypes.byref(desc), B, Tu), dtype=torch.uint8, device="cuda")
    bws = torch.empty(lib.spd_attn_workspace_bytes(ctypes.byref(desc), B, Tu), dtype=torch.uint8, device="cuda")
    assert lib.spd_split_attn_fwd(ctypes.byref(desc), ctypes.byref(twin.c), Tu, _p(qu), _p(ku), _p(vu), _p(ou),
                                  _p(lu), _p(fws), fws.numel(), st) == OK
    dqu, dku, dvu = torch.empty_like(qu), torch.empty_like(ku), torch.empty_like(vu)
    assert lib.spd_split_attn_bwd(ctypes.byref(desc), ctypes.byref(twin.c), Tu, _p(qu), _p(ku), _p(vu), _p(ou),
                                  _p(lu), _p(dou), _p(dqu), _p(dku), _p(dvu), _p(bws), bws.numel(), st) == OK
    o = move(ou, plan, T, twin, Tu)
    grads = [move(g, plan, T, twin, Tu) for g in (dqu, dku, dvu)]
    torch.cuda.synchronize()

    ro, _ = oracle.split_attention_forward(x.q, x.k, x.v, oinfo, valid=valid)
    rgrads = oracle.split_attention_backward(x.q, x.k, x.v, x.do, oinfo, valid=valid)
    compare("o", to_numpy(o), ro, "bf16")
    for name, g, r in zip(("dq", "dk", "dv"), grads, rgrads):
        compare(name, to_numpy(g), r, "bf16")
    pads = torch.from_numpy(~valid).cuda()
    assert not o[pads].any() and not any(g[pads].any() for g in grads)
