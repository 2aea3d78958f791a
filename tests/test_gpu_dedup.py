"""GPU parity: grouping, packing, row packing and reconstruction are bit-exact
with the oracle, on every workload at full size and on edge cases."""
import numpy as np
import pytest

import oracle
from helpers import gpu_plan, oracle_plan, say
from workloads import WORKLOADS, Workload, make_batch

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SMALL = [
    WORKLOADS["tiny_fp32"],
    WORKLOADS["tiny_fp32"].scaled(name="ragged_unpad", num_prompts=3, rollout_n=5, prompt_len=300,
                                  response_len=77, resp_len_range=(0, 77), seed=21),
    WORKLOADS["tiny_fp32"].scaled(name="singletons", num_prompts=7, rollout_n=1, prompt_len=5,
                                  response_len=3, seed=22),
    WORKLOADS["tiny_fp32"].scaled(name="one_sample", num_prompts=1, rollout_n=1, prompt_len=9,
                                  response_len=4, seed=23),
    WORKLOADS["tiny_fp32"].scaled(name="many_rows", num_prompts=40, rollout_n=30, prompt_len=17,
                                  response_len=5, vocab=3, seed=24),
]
CASES = [(w, p) for w in SMALL for p in (False, True)] + \
        [(WORKLOADS[n], False) for n in WORKLOADS if n != "tiny_fp32"]


def _ids(w, p):
    return f"{w.name}{'-perm' if p else ''}"


def _check_plan(bt, use_unpad, mask_dtype=None):
    og, ou, odids, odpos, oinfo = oracle_plan(bt, use_unpad)
    gg, gu, gdids, gdpos, ginfo = gpu_plan(bt, use_unpad, mask_dtype)
    assert list(gg) == og
    np.testing.assert_array_equal(gu.cpu().numpy(), ou)
    assert ginfo["G"] == oinfo["G"] and ginfo["T"] == oinfo["T"]
    np.testing.assert_array_equal(gdids.cpu().numpy(), odids)
    np.testing.assert_array_equal(gdpos.cpu().numpy(), odpos)
    G, B, T = oinfo["G"], oinfo["B"], oinfo["T"]
    p = ginfo.plan
    np.testing.assert_array_equal(p.group_of.cpu().numpy(), oinfo["group_of"])
    np.testing.assert_array_equal(p.rep[:G].cpu().numpy(), oinfo["rep"])
    np.testing.assert_array_equal(p.prompt_off[:G].cpu().numpy(), oinfo["prompt_off"])
    np.testing.assert_array_equal(p.prompt_len[:G].cpu().numpy(), oinfo["prompt_len"])
    np.testing.assert_array_equal(p.resp_off.cpu().numpy(), oinfo["resp_off"])
    np.testing.assert_array_equal(p.resp_len.cpu().numpy(), oinfo["resp_len"])
    np.testing.assert_array_equal(p.src[:T].cpu().numpy(), oinfo["src"])
    np.testing.assert_array_equal(p.dst.cpu().numpy(), oinfo["dst"])
    np.testing.assert_array_equal(p.seg_start[:T].cpu().numpy(), oinfo["seg_start"])
    off = [0]
    for m in og:
        off.append(off[-1] + len(m))
    np.testing.assert_array_equal(p.grp_off[:G + 1].cpu().numpy(), off)
    np.testing.assert_array_equal(p.grp_idx.cpu().numpy(), sum(og, []))
    return oinfo, ginfo


@pytest.mark.parametrize("w,permute", CASES, ids=[_ids(*c) for c in CASES])
def test_plan_bit_exact(w, permute):
    say(f"[dedup plan] {w.name} permute={permute} B={w.batch} S={w.seq_len} unpad={w.use_unpad}")
    _check_plan(make_batch(w, permute=permute), w.use_unpad)


@pytest.mark.parametrize("mask_dtype", ["bool", "int32", "int64"])
def test_mask_dtypes(mask_dtype):
    w = SMALL[1]
    say(f"[dedup plan] mask dtype {mask_dtype}")
    _check_plan(make_batch(w, permute=True), True, getattr(torch, mask_dtype))


def test_padded_mode_ignores_mask_and_prompt_padding():
    """use_unpad=False keeps every token; use_unpad=True drops left-padded prompt tokens too."""
    rng = np.random.default_rng(9)
    B, P, R = 9, 40, 12
    ids = rng.integers(1, 50, size=(B, P + R))
    ids[:5, :P] = ids[0, :P]
    ids[5:, :P] = ids[5, :P]
    mask = np.ones_like(ids)
    mask[:5, :7] = 0
    mask[2, P + 3:] = 0
    mask[6, P:] = 0
    pos = np.cumsum(mask, 1) - 1
    from workloads import Batch
    bt = Batch(ids, pos, mask, R, None, None)
    for unpad in (False, True):
        say(f"[dedup plan] handmade padding unpad={unpad}")
        _check_plan(bt, unpad)


def test_response_length_extremes():
    w = SMALL[0]
    bt = make_batch(w)
    from workloads import Batch
    for R in (0, w.seq_len, 1):
        say(f"[dedup plan] response_length={R}")
        _check_plan(Batch(bt.input_ids, bt.position_ids, bt.attention_mask, R, None, None), False)



@pytest.mark.parametrize("S,R", [(5001, 3), (4100, 3), (6146, 2)], ids=["odd_S", "odd_P", "whole_chunks"])
def test_grouping_across_hash_chunks(S, R):
    """Prompts longer than one 2048-token hashing block: rows that differ in one
    token on either side of a block boundary, in the first or last token, or by
    two tokens swapped across a boundary never group together; exact copies do.
    Odd S takes the 8-byte load path, odd P the odd tail of the 16-byte one."""
    P = S - R
    rng = np.random.default_rng(S)
    base = rng.integers(0, 1000, size=P)
    base[2047], base[2048] = 5, 7          # distinct, so swapping them changes the prompt
    rows = []
    for change in (None, P - 1, None, 2047, 2048, 0, None, 2049, 2047, P - 2, "swap"):
        r = base.copy()
        if change == "swap":
            r[2047], r[2048] = r[2048], r[2047]
        elif change is not None:
            r[change] = r[change] + 1
        rows.append(r)
    B = len(rows)
    ids = np.concatenate([np.stack(rows), rng.integers(0, 1000, size=(B, R))], axis=1).astype(np.int64)
    pos = np.tile(np.arange(S, dtype=np.int64), (B, 1))
    from workloads import Batch
    bt = Batch(ids, pos, np.ones_like(ids), R, None, None)
    say(f"[dedup plan] hash chunks S={S} P={P}")
    oinfo, _ = _check_plan(bt, False)
    assert oinfo["G"] == 8          # {0, 2, 6} and {3, 8} group; the other six rows stand alone


def _holey_batch(P, R, G, n, seed, prefix=0):
    """G groups of n samples (members interleaved): prompts identical within a
    group, with left pads and random holes in the prompt mask (the same for every
    member); responses of random tokens with random holes.  With prefix > 0,
    every prompt starts with the same prefix tokens and prefix mask."""
    from workloads import Batch
    rng = np.random.default_rng(seed)
    S, B = P + R, G * n
    prompts = rng.integers(1, 1000, size=(G, P))
    pmask = (rng.random((G, P)) > 0.2).astype(np.int64)
    pmask[:, :37] = 0
    if prefix:
        prompts[:, :prefix] = prompts[0, :prefix]
        pmask[:, :prefix] = pmask[0, :prefix]
    order = rng.permutation(B)
    ids = np.zeros((B, S), dtype=np.int64)
    mask = np.zeros((B, S), dtype=np.int64)
    for b in range(B):
        g = order[b] % G
        ids[b, :P], mask[b, :P] = prompts[g], pmask[g]
        ids[b, P:] = rng.integers(1, 1000, size=R)
        mask[b, P:] = rng.random(R) > 0.3
    pos = np.maximum(np.cumsum(mask, axis=1) - 1, 0).astype(np.int64)
    return Batch(ids, pos, mask, R, None, None)


@pytest.mark.parametrize("P,R", [(2500, 1500), (1023, 1026), (3072, 5)], ids=["mid_chunk", "edge_chunk", "aligned"])
def test_unpad_pack_across_column_chunks(P, R):
    """Unpadded packing counts kept columns per column chunk of each row: the
    prompt/response boundary inside a chunk, one column before a chunk
    boundary, and on one; masks with holes in prompts and responses."""
    bt = _holey_batch(P, R, 3, 3, seed=P + R)
    say(f"[dedup plan] unpad across column chunks P={P} R={R}")
    oinfo, _ = _check_plan(bt, True)
    assert oinfo["G"] == 3 and 0 < oinfo["T"] < bt.input_ids.size


def test_maximum_batch_size():
    """B = 65,536 rows, the largest batch the C ABI takes, of 3-token prompts over a
    3-token vocabulary: all 27 prompts occur, each group with thousands of members."""
    rng = np.random.default_rng(65536)
    B, P, R = 65536, 3, 1
    ids = rng.integers(0, 3, size=(B, P + R)).astype(np.int64)
    pos = np.tile(np.arange(P + R, dtype=np.int64), (B, 1))
    from workloads import Batch
    say(f"[dedup plan] maximum batch B={B}")
    oinfo, _ = _check_plan(Batch(ids, pos, np.ones_like(ids), R, None, None), False)
    assert oinfo["G"] == 27

ROW_CASES = [(SMALL[0], 512), (SMALL[1], 48), (SMALL[4], 16), (WORKLOADS["qwen3_0p6b_2x8_p8192_r512"], 4096),
             (WORKLOADS["long_2x8_p32768_r256to1024_unpad"], 64), (WORKLOADS["bwd_4x8_p4096_r1024"], 160)]


@pytest.mark.parametrize("w,row_bytes", ROW_CASES, ids=[f"{w.name}-{r}B" for w, r in ROW_CASES])
def test_pack_rows_and_reconstruct_bit_exact(w, row_bytes):
    import shared_prompt_dedup_amd as spd
    say(f"[rows] {w.name} row_bytes={row_bytes}")
    bt = make_batch(w, permute=True)
    _, _, _, _, oinfo = oracle_plan(bt, w.use_unpad)
    _, _, _, _, ginfo = gpu_plan(bt, w.use_unpad)
    rng = np.random.default_rng(5)
    B, S, T = oinfo["B"], oinfo["S"], oinfo["T"]
    W = row_bytes // 4
    # reconstruct: packed rows -> batch
    packed = rng.integers(-2**31, 2**31 - 1, size=(T, W), dtype=np.int64).astype(np.int32)
    out = spd.reconstruct_sequences(torch.from_numpy(packed).cuda()[None], ginfo)
    ref = oracle.reconstruct_sequences(packed[None], oinfo)
    np.testing.assert_array_equal(out.cpu().numpy(), ref)
    del out
    # pack_rows: batch rows -> packed (prompt rows equal within a group)
    rows = rng.integers(-2**31, 2**31 - 1, size=(B, S, W), dtype=np.int64).astype(np.int32)
    got = spd.pack_rows(torch.from_numpy(rows).cuda(), ginfo)
    np.testing.assert_array_equal(got.cpu().numpy(), oracle.pack_rows(rows, oinfo))


def test_reconstruct_bf16_hidden_shape():
    """The pages' shape contract: [1, T, H] in, [B, S, H] out, for an H of hidden size."""
    import shared_prompt_dedup_amd as spd
    w = WORKLOADS["tiny_fp32"]
    bt = make_batch(w)
    _, _, _, _, oinfo = oracle_plan(bt, False)
    _, _, _, _, ginfo = gpu_plan(bt, False)
    H = 1024
    x = torch.randn(1, oinfo["T"], H, dtype=torch.bfloat16, device="cuda")
    y = spd.reconstruct_sequences(x, ginfo)
    assert tuple(y.shape) == (w.batch, w.seq_len, H)
    ref = oracle.reconstruct_sequences(x.float().cpu().numpy(), oinfo)
    np.testing.assert_array_equal(y.float().cpu().numpy(), ref)


def test_repeat_calls_are_identical():
    import shared_prompt_dedup_amd as spd
    w = SMALL[1]
    bt = make_batch(w, permute=True)
    a = gpu_plan(bt, True)
    b = gpu_plan(bt, True)
    T = a[4]["T"]
    assert T == b[4]["T"]
    for f in ("src", "seg_start"):     # capacity B*S; the first T entries are defined
        assert torch.equal(getattr(a[4].plan, f)[:T], getattr(b[4].plan, f)[:T])
    for f in ("dst", "resp_off", "resp_len", "group_of", "grp_idx"):
        assert torch.equal(getattr(a[4].plan, f), getattr(b[4].plan, f))


# ---------------------------------------------------------------- every row move at the workloads' own width

FULL_WIDTH = ["redundancy_1x10_p10240_r1024", "long_2x8_p32768_r256to1024_unpad", "bwd_4x8_p4096_r1024",
              "prefix_4x8_s4096_p5120_r512"]


def _bf16_bits(rng, shape):
    """Seeded normal values rounded to bf16: (uint16 bit patterns, float32 values); drawn one leading row at a
    time to bound host memory."""
    from workloads import round_to_bf16
    bits = np.empty(shape, dtype=np.uint16)
    for i in range(shape[0]):
        bits[i] = round_to_bf16(rng.standard_normal(shape[1:], dtype=np.float32))[0]
    return bits


def _as_f32(bits):
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


@pytest.mark.parametrize("name", FULL_WIDTH)
def test_row_moves_at_full_width(name):
    """pack_rows, reconstruct and both backwards on the attention output's own rows (Hq * d bf16 = 4096 bytes):
    the whole batch on the GPU in one call each, compared with the oracle on column blocks (each block of a row
    move is the same move at a narrower width), so host memory stays bounded.  The 32K-prompt batch's
    reconstruct writes 2.2 GB: byte offsets past 2^31.  Byte moves bit-exact; reconstruct_bwd within the
    fp32-accumulation bound of test_rows_backward."""
    import shared_prompt_dedup_amd as spd
    w = WORKLOADS[name]
    say(f"[rows full width] {name}")
    bt = make_batch(w, permute=True)
    groups, uniq = oracle.find_prompt_groups(bt.input_ids, bt.response_length)
    L0 = oracle.find_shared_prefix(bt.input_ids, bt.response_length, groups) if w.shared_prefix else 0
    _, _, oinfo = oracle.create_deduplicated_batch(bt.input_ids, bt.position_ids, bt.response_length, groups, uniq,
                                                   attention_mask=bt.attention_mask, use_unpad=w.use_unpad,
                                                   prefix_len=L0)
    ids, pos, mask = (torch.from_numpy(a).cuda() for a in (bt.input_ids, bt.position_ids, bt.attention_mask))
    gg, gu = spd.find_prompt_groups(ids, bt.response_length)
    _, _, ginfo = spd.create_deduplicated_batch(ids, pos, bt.response_length, gg, gu,
                                                attention_mask=mask if w.use_unpad else None,
                                                use_unpad=w.use_unpad, share_prefix=bool(w.shared_prefix))
    assert ginfo["prefix_len"] == oinfo["prefix_len"] and (oinfo["prefix_len"] > 0) == bool(w.shared_prefix)
    B, S, T = oinfo["B"], oinfo["S"], oinfo["T"]
    assert ginfo["T"] == T
    W = w.num_q_heads * w.head_dim          # bf16 elements per row: 4096 bytes
    nmax = B if oinfo["prefix_len"] else max(len(m) for m in groups)   # terms summed into one packed row
    blocks = [(c, c + 256) for c in range(0, W, 256)]
    rng = np.random.default_rng(17)

    # forward pair: reconstruct [T, W] -> [B, S, W]; pack_rows [B, S, W] -> [T, W]
    packed = _bf16_bits(rng, (T, W))
    out = spd.reconstruct_sequences(torch.from_numpy(packed.view(np.int16)).cuda().view(torch.bfloat16)[None], ginfo)
    say(f"  reconstruct: {out.numel() * 2 / 1e9:.2f} GB written")
    for c0, c1 in blocks:
        ref = oracle.reconstruct_sequences(packed[:, c0:c1][None], oinfo)
        got = out[:, :, c0:c1].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        np.testing.assert_array_equal(got, ref)
    del out
    rows = _bf16_bits(rng, (B, S, W))
    rows_t = torch.from_numpy(rows.view(np.int16)).cuda().view(torch.bfloat16)
    got = spd.pack_rows(rows_t, ginfo).view(torch.int16).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(got, oracle.pack_rows(rows, oinfo))
    del got
    # backward pair: pack_rows_bwd [T, W] -> [B, S, W]; reconstruct_bwd [B, S, W] -> [T, W]
    back = spd.pack_rows_bwd(torch.from_numpy(packed.view(np.int16)).cuda().view(torch.bfloat16), ginfo)
    for c0, c1 in blocks:
        ref = oracle.pack_rows_backward(packed[:, c0:c1], oinfo)
        got = back[:, :, c0:c1].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        np.testing.assert_array_equal(got, ref)
    del back
    gsum = spd.reconstruct_bwd(rows_t, ginfo).float().cpu().numpy()
    del rows_t
    worst = 0.0
    for c0, c1 in blocks:
        vals = _as_f32(rows[:, :, c0:c1])
        ref = oracle.reconstruct_backward(vals, oinfo)
        absum = oracle.reconstruct_backward(np.abs(vals), oinfo)
        bound = (nmax - 1) * 2.0**-24 * absum + 2.0**-8 * np.abs(ref)
        err = np.abs(gsum[:, c0:c1] - ref)
        worst = max(worst, float((err / (bound + 1e-30)).max()) if err.size else 0.0)
        assert (err <= bound + 1e-30).all()
    say(f"  reconstruct_bwd: worst err / bound = {worst:.3f}")


# ---------------------------------------------------------------- backward of reconstruct / pack_rows

BWD_ROW_CASES = [(SMALL[0], 512), (SMALL[1], 48), (SMALL[2], 32), (SMALL[4], 16),
                 (WORKLOADS["qwen3_0p6b_2x8_p8192_r512"], 256), (WORKLOADS["redundancy_1x10_p10240_r1024"], 128),
                 (WORKLOADS["long_2x8_p32768_r256to1024_unpad"], 64), (WORKLOADS["bwd_4x8_p4096_r1024"], 160)]


def _bf16_round(a):
    """float32 -> nearest bfloat16 (ties to even), as float32."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16).float().numpy()


@pytest.mark.parametrize("w,row_bytes", BWD_ROW_CASES, ids=[f"{w.name}-{r}B" for w, r in BWD_ROW_CASES])
def test_rows_backward(w, row_bytes):
    """pack_rows_bwd is a byte scatter: bit-exact.  reconstruct_bwd sums each packed row's readers in fp32 and
    rounds once: within (n - 1) 2^-24 sum|x| (fp32 accumulation of n terms) plus half a bf16 ulp of the exact
    sum (bf16 keeps 8 significant bits: at most 2^-8 |sum|)."""
    import shared_prompt_dedup_amd as spd
    say(f"[rows bwd] {w.name} row_bytes={row_bytes}")
    bt = make_batch(w, permute=True)
    groups, _, _, _, oinfo = oracle_plan(bt, w.use_unpad)
    _, _, _, _, ginfo = gpu_plan(bt, w.use_unpad)
    rng = np.random.default_rng(9)
    B, S, T = oinfo["B"], oinfo["S"], oinfo["T"]
    nmax = max(len(m) for m in groups)
    # pack_rows backward
    W = row_bytes // 4
    dp = rng.integers(-2**31, 2**31 - 1, size=(T, W), dtype=np.int64).astype(np.int32)
    got = spd.pack_rows_bwd(torch.from_numpy(dp).cuda(), ginfo)
    np.testing.assert_array_equal(got.cpu().numpy(), oracle.pack_rows_backward(dp, oinfo))
    del got
    # reconstruct backward, bf16 and fp32 rows
    for dt, elt in ((torch.bfloat16, 2), (torch.float32, 4)):
        W = row_bytes // elt
        vals = rng.standard_normal((B, S, W)).astype(np.float32)
        if dt == torch.bfloat16:
            vals = _bf16_round(vals)
        got = spd.reconstruct_bwd(torch.from_numpy(vals).to("cuda", dt), ginfo).float().cpu().numpy()
        ref = oracle.reconstruct_backward(vals, oinfo)
        absum = oracle.reconstruct_backward(np.abs(vals), oinfo)
        bound = (nmax - 1) * 2.0**-24 * absum + (2.0**-8 * np.abs(ref) if dt == torch.bfloat16 else 0.0)
        err = np.abs(got - ref)
        say(f"  reconstruct_bwd {dt}: max_err={err.max() if err.size else 0:.3e} "
            f"exact={np.mean(got == (_bf16_round(ref) if dt == torch.bfloat16 else ref.astype(np.float32))):.6f}")
        assert (err <= bound + 1e-30).all()


def test_rows_autograd():
    """reconstruct_sequences and pack_rows are differentiable through the library's backward calls."""
    import shared_prompt_dedup_amd as spd
    w = SMALL[1]
    bt = make_batch(w, permute=True)
    _, _, _, _, oinfo = oracle_plan(bt, True)
    _, _, _, _, ginfo = gpu_plan(bt, True)
    T, B, S, H = oinfo["T"], oinfo["B"], oinfo["S"], 64
    x = torch.randn(T, H, dtype=torch.bfloat16, device="cuda", requires_grad=True)
    gy = torch.randn(B, S, H, dtype=torch.bfloat16, device="cuda")
    y = spd.reconstruct_sequences(x[None], ginfo)
    (y * gy).sum().backward()
    np.testing.assert_array_equal(x.grad.float().cpu().numpy(),
                                  spd.reconstruct_bwd(gy, ginfo).float().cpu().numpy())
    ref = oracle.reconstruct_backward(gy.float().cpu().numpy(), oinfo)
    assert (np.abs(x.grad.float().cpu().numpy() - ref) <= 2.0**-8 * np.abs(ref) + 1e-6).all()
    rows = torch.randn(B, S, H, dtype=torch.float32, device="cuda", requires_grad=True)
    gp = torch.randn(T, H, dtype=torch.float32, device="cuda")
    (spd.pack_rows(rows, ginfo) * gp).sum().backward()
    np.testing.assert_array_equal(rows.grad.cpu().numpy(), oracle.pack_rows_backward(gp.cpu().numpy(), oinfo))
