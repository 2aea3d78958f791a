"""GPU parity for the variable-length parameters (How Prompt Deduplication
Works -- Flash Attention Integration): bit-exact with the oracle's
definitions, on block-diagonal masks of every alignment, on malformed and
empty masks, and on the plans of every workload."""
import numpy as np
import pytest

import oracle
from helpers import gpu_plan, oracle_plan, say
from workloads import WORKLOADS, make_batch

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _block_mask(q_lens, k_lens, style):
    Tq, Tk = sum(q_lens), sum(k_lens)
    m = np.zeros((Tq, Tk), bool)
    r0 = c0 = 0
    for ql, kl in zip(q_lens, k_lens):
        for i in range(ql):
            hi = kl if style == "full" else (i + 1 if style == "causal" else kl - ql + i + 1)
            if hi > 0:
                m[r0 + i, c0:c0 + min(hi, kl)] = True
        r0, c0 = r0 + ql, c0 + kl
    return m


def _check(mask_np, dtype=torch.bool):
    import shared_prompt_dedup_amd as spd
    ref = oracle.attention_mask_to_flash_attn_params(mask_np)
    got = spd.attention_mask_to_flash_attn_params(torch.from_numpy(mask_np).to("cuda", dtype))
    np.testing.assert_array_equal(got["cu_seqlens_q"].cpu().numpy(), ref["cu_seqlens_q"])
    np.testing.assert_array_equal(got["cu_seqlens_k"].cpu().numpy(), ref["cu_seqlens_k"])
    for key in ("max_seqlen_q", "max_seqlen_k", "num_seqs", "mismatched_rows"):
        assert got[key] == ref[key], key
    return got


@pytest.mark.parametrize("style", ["full", "causal", "bottom_right"])
@pytest.mark.parametrize("dtype", [torch.bool, torch.int32, torch.int64])
@pytest.mark.parametrize("row_align", [1, 16], ids=["any_row_bytes", "row_bytes_16x"])
def test_block_masks(style, dtype, row_align):
    """row_bytes_16x pads trailing all-zero key columns so each row is a multiple of 16 bytes (the 16-byte read
    path); any_row_bytes keeps odd row lengths (the byte path)."""
    rng = np.random.default_rng(51)
    esz = torch.tensor([], dtype=dtype).element_size()
    for n, hi in ((1, 9), (6, 40), (40, 90)):
        k_lens = rng.integers(1, hi, n).tolist()
        q_lens = list(k_lens) if style == "causal" else rng.integers(1, hi, n).tolist()
        m = _block_mask(q_lens, k_lens, style)
        if row_align == 16:
            m = np.pad(m, ((0, 0), (0, (-m.shape[1]) % max(1, 16 // esz))))
        elif (m.shape[1] * esz) % 16 == 0:
            m = np.pad(m, ((0, 0), (0, 1)))
        say(f"[varlen] {style} {dtype} blocks={n} rows={sum(q_lens)} cols={m.shape[1]}")
        got = _check(m, dtype)
        assert got["num_seqs"] == n and got["mismatched_rows"] == 0


@pytest.mark.parametrize("style", ["full", "bottom_right"])
def test_block_masks_many_rows(style):
    """More rows than one pass of the scans covers (16,384), with blocks and rows that see nothing straddling the
    pass boundaries."""
    rng = np.random.default_rng(53)
    n = 300
    q_lens = rng.integers(1, 140, n).tolist()
    k_lens = rng.integers(1, 16, n).tolist()
    m = _block_mask(q_lens, k_lens, style)
    say(f"[varlen] many rows: {style} blocks={n} rows={m.shape[0]} cols={m.shape[1]}")
    assert m.shape[0] > 16384
    got = _check(m)
    assert got["num_seqs"] == n and got["mismatched_rows"] == 0
    _check(np.pad(m, ((0, 0), (0, (-m.shape[1]) % 16))))


def test_malformed_and_empty_masks():
    rng = np.random.default_rng(52)
    m = _block_mask([300, 500, 700], [400, 400, 900], "bottom_right")
    m[350, 10] = True                                   # a row of block 1 also sees a key of block 0
    m[1200, 1500] = False
    m[rng.integers(0, 1500, 20), rng.integers(0, 1700, 20)] = True
    got = _check(m)
    assert got["mismatched_rows"] > 0
    _check(np.zeros((1300, 20), bool))
    _check(np.ones((5, 1), bool))


@pytest.mark.parametrize("name", ["tiny_fp32", "qwen3_0p6b_2x8_p8192_r512", "long_2x8_p32768_r256to1024_unpad",
                                  "bwd_4x8_p4096_r1024"])
def test_plan_varlen_params(name):
    import shared_prompt_dedup_amd as spd
    w = WORKLOADS[name]
    bt = make_batch(w, permute=True)
    _, _, _, _, oinfo = oracle_plan(bt, w.use_unpad)
    _, _, _, _, ginfo = gpu_plan(bt, w.use_unpad)
    ref = oracle.varlen_params(oinfo)
    got = spd.flash_attn_params(ginfo)
    for key in ("cu_seqlens_prompt", "cu_seqlens_q", "cu_seqlens_k"):
        np.testing.assert_array_equal(got[key].cpu().numpy(), ref[key], err_msg=key)
    for key in ("max_seqlen_prompt", "max_seqlen_q", "max_seqlen_k"):
        assert got[key] == ref[key], key
