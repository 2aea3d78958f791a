"""spd_split_attn_fwd_noalloc (the forward with the library's fixed device scratch instead of a workspace),
called through the C ABI, against spd_split_attn_fwd on the same inputs: bitwise equal outputs and LSE (the
same kernels on the same tile list).  Three calls in a row on one device, each smaller than the one before, so
later calls run on a scratch that still holds the earlier, larger call's tile list."""
import ctypes
import math

import pytest

from helpers import attn_inputs, gpu_plan, say
from workloads import WORKLOADS, make_batch

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

_base = WORKLOADS["tiny_fp32"]
SEQUENCE = [
    # 2 prompts x 4 responses, prompt 2048, response 512, GQA 16/8/128: 58 query tiles x 8 head groups
    _base.scaled(name="noalloc_mid", num_prompts=2, rollout_n=4, prompt_len=2048, response_len=512,
                 num_q_heads=16, num_kv_heads=8, head_dim=128, dtype="bf16", sigma=0.5, vocab=151936, seed=39),
    # smaller, ragged unpadded responses
    _base.scaled(name="noalloc_small", num_prompts=2, rollout_n=3, prompt_len=300, response_len=77, num_q_heads=4,
                 num_kv_heads=2, head_dim=128, dtype="bf16", sigma=0.5, resp_len_range=(0, 77), seed=32),
    # smallest, the fp32 path
    _base,
]


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def test_noalloc_forward_matches_workspace_forward():
    from shared_prompt_dedup_amd import _lib as L
    lib = L.lib
    prev_T = None
    for w in SEQUENCE:
        bt = make_batch(w, permute=True)
        *_, ginfo = gpu_plan(bt, w.use_unpad)
        T = ginfo["T"]
        assert prev_T is None or T < prev_T
        prev_T = T
        _, q, k, v, _ = attn_inputs(w, T)
        Hq, Hkv, d = w.num_q_heads, w.num_kv_heads, w.head_dim
        desc = L.SpdAttnDesc(Hq, Hkv, d, L.SPD_BF16 if w.dtype == "bf16" else L.SPD_F32, 1.0 / math.sqrt(d))
        st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        plan = ctypes.byref(ginfo.plan.c)
        say(f"[noalloc] {w.name}: T={T} Hq/Hkv/d={Hq}/{Hkv}/{d} {w.dtype}")
        # the existing entry point, with its workspace
        ws = torch.empty(lib.spd_attn_fwd_workspace_bytes(ctypes.byref(desc), ginfo["B"], T), dtype=torch.uint8,
                         device="cuda")
        o_ref, lse_ref = torch.empty_like(q), torch.empty((Hq, T), dtype=torch.float32, device="cuda")
        assert lib.spd_split_attn_fwd(ctypes.byref(desc), plan, T, _p(q), _p(k), _p(v), _p(o_ref), _p(lse_ref),
                                      _p(ws), ws.numel(), st) == 0
        # the workspace-free entry point, outputs pre-filled with NaN so that a row it misses shows
        o = torch.full_like(q, float("nan"))
        lse = torch.full((Hq, T), float("nan"), dtype=torch.float32, device="cuda")
        assert lib.spd_split_attn_fwd_noalloc(ctypes.byref(desc), plan, T, _p(q), _p(k), _p(v), _p(o), _p(lse),
                                              st) == 0
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), f"{w.name}: outputs differ"
        assert torch.equal(lse, lse_ref), f"{w.name}: lse differs"
