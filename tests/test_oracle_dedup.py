"""Pins for the oracle's grouping, packing and reconstruction (CPU only).

Each check ties the oracle to something other than itself: the pages'
worked examples (tests/golden/), brute force with an independent
equivalence-class construction, token arithmetic, and round trips.
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle
from workloads import WORKLOADS, make_batch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _classes_by_dict(ids, P):
    """Independent grouping: bucket rows by the tuple of their prompt tokens,
    order buckets by their smallest member."""
    buckets = {}
    for b in range(ids.shape[0]):
        buckets.setdefault(tuple(ids[b, :P].tolist()), []).append(b)
    return sorted(buckets.values(), key=lambda m: m[0])


def test_page_grouping_example():
    g = _golden("find_prompt_groups_example.json")
    rng = np.random.default_rng(0)
    P, R = 6, 3
    prompts = rng.integers(0, 50, size=(2, P))
    ids = np.concatenate([prompts[g["prompt_of_sample"]], rng.integers(0, 50, size=(g["batch"], R))], 1)
    groups, uniq = oracle.find_prompt_groups(ids, R)
    assert groups == g["prompt_groups"]
    assert uniq.shape == (2, P)
    np.testing.assert_array_equal(uniq, prompts)


@pytest.mark.parametrize("B,P", [(1, 1), (3, 2), (4, 2), (5, 2), (6, 2), (4, 3)])
def test_grouping_exhaustive_binary(B, P):
    """Every batch of B rows over the vocabulary {0, 1} with prompt length P."""
    R = 1
    for bits in itertools.product([0, 1], repeat=B * P):
        prm = np.array(bits, dtype=np.int64).reshape(B, P)
        ids = np.concatenate([prm, np.arange(B)[:, None] % 2], 1)
        groups, uniq = oracle.find_prompt_groups(ids, R)
        assert groups == _classes_by_dict(ids, P)
        for g, m in enumerate(groups):
            np.testing.assert_array_equal(uniq[g], prm[m[0]])


def test_grouping_adversarial():
    P, R = 8, 4
    base = np.arange(P) + 10
    rows = [base.copy() for _ in range(7)]
    rows[1][0] += 1          # differs only in the first prompt token
    rows[2][-1] += 1         # differs only in the last prompt token
    rows[4] = rows[1].copy()  # interleaved member of row 1's group
    ids = np.stack([np.concatenate([r, np.full(R, i)]) for i, r in enumerate(rows)])
    groups, _ = oracle.find_prompt_groups(ids, R)
    # rows 0,3,5,6 share the base prompt (their responses differ); 1 and 4 share one; 2 alone
    assert groups == [[0, 3, 5, 6], [1, 4], [2]]
    # a response token equal to a prompt token never matters
    groups_all_resp, _ = oracle.find_prompt_groups(ids, 0)
    assert groups_all_resp == [[i] for i in range(7)]
    # response_length == seq_len: empty prompts, one group
    groups_empty, uniq = oracle.find_prompt_groups(ids, P + R)
    assert groups_empty == [list(range(7))] and uniq.shape == (1, 0)


def test_concatenation_order_example():
    g = _golden("concatenation_example.json")
    tok = {"A": [1, 2, 3], "B": [4, 5, 6], "R1": [11, 12], "R2": [21, 22], "R3": [31, 32], "R4": [41, 42]}
    ids = np.array([tok[p] + tok[r] for p, r in g["samples"]], dtype=np.int64)
    pos = np.tile(np.arange(ids.shape[1]), (ids.shape[0], 1))
    groups, uniq = oracle.find_prompt_groups(ids, 2)
    assert groups == [[0, 1], [2, 3]]
    dids, dpos, info = oracle.create_deduplicated_batch(ids, pos, 2, groups, uniq)
    expect = sum((tok[x] for x in g["packed"]), [])
    assert dids.shape == (1, len(expect))
    assert dids[0].tolist() == expect
    # positions are gathered: prompt 0..2, each response 3..4
    assert dpos[0].tolist() == [0, 1, 2, 3, 4, 3, 4, 0, 1, 2, 3, 4, 3, 4]


def test_redundancy_example_arithmetic():
    g = _golden("redundancy_example.json")
    P, n, R = g["prompt_len"], g["num_responses"], g["response_len"]
    ids = np.zeros((n, P + R), dtype=np.int64)
    ids[:, P:] = np.arange(n)[:, None]
    pos = np.tile(np.arange(P + R), (n, 1))
    groups, uniq = oracle.find_prompt_groups(ids, R)
    _, _, info = oracle.create_deduplicated_batch(ids, pos, R, groups, uniq)
    total, unique, red = oracle.redundancy_counts(info)
    assert total == g["total_tokens"]
    assert unique == g["unique_tokens"]
    assert round(100 * red) == g["redundancy_percent_rounded"]


def test_redundancy_workload_tokens():
    """The 10240/1024 workload: 110Ki total, 20Ki unique, 82% redundant."""
    w = WORKLOADS["redundancy_1x10_p10240_r1024"]
    bt = make_batch(w)
    groups, uniq = oracle.find_prompt_groups(bt.input_ids, bt.response_length)
    _, _, info = oracle.create_deduplicated_batch(bt.input_ids, bt.position_ids, bt.response_length,
                                                  groups, uniq)
    total, unique, red = oracle.redundancy_counts(info)
    assert (total, unique) == (112640, 20480)
    assert round(100 * red) == 82


def _check_plan(ids, pos, mask, R, use_unpad, groups, uniq):
    dids, dpos, info = oracle.create_deduplicated_batch(ids, pos, R, groups, uniq,
                                                        attention_mask=mask, use_unpad=use_unpad)
    B, S = ids.shape
    P = S - R
    keep = (mask != 0) if use_unpad else np.ones_like(ids, dtype=bool)
    # token count: each group's first-member prompt once plus every kept response token
    T = sum(int(keep[m[0], :P].sum()) for m in groups) + int(keep[:, P:].sum())
    assert info["T"] == T == dids.shape[1]
    flat_ids, flat_pos = ids.reshape(-1), pos.reshape(-1)
    np.testing.assert_array_equal(dids[0], flat_ids[info["src"]])
    np.testing.assert_array_equal(dpos[0], flat_pos[info["src"]])
    # segments tile [0, T) in the concatenation order
    cursor = 0
    for g, m in enumerate(groups):
        assert info["prompt_off"][g] == cursor
        cursor += info["prompt_len"][g]
        for b in m:
            assert info["resp_off"][b] == cursor
            cursor += info["resp_len"][b]
    assert cursor == T
    # dst inverts src on the rows that were packed; prompt copies map to the first member's rows
    for j, s in enumerate(info["src"]):
        assert info["dst"][s] == j
    for b in range(B):
        g = info["group_of"][b]
        r = groups[g][0]
        for t in range(S):
            j = info["dst"][b * S + t]
            if t < P:
                assert j == info["dst"][r * S + t]
                assert (j >= 0) == bool(keep[r, t])
            else:
                assert (j >= 0) == bool(keep[b, t])
    return info


@pytest.mark.parametrize("use_unpad", [False, True])
@pytest.mark.parametrize("permute", [False, True])
def test_pack_tiny_workload(use_unpad, permute):
    w = WORKLOADS["tiny_fp32"]
    if use_unpad:
        w = w.scaled(resp_len_range=(0, 32))
    bt = make_batch(w, permute=permute)
    groups, uniq = oracle.find_prompt_groups(bt.input_ids, bt.response_length)
    assert groups == _classes_by_dict(bt.input_ids, w.prompt_len)
    _check_plan(bt.input_ids, bt.position_ids, bt.attention_mask, bt.response_length, use_unpad,
                groups, uniq)


def test_pack_unpad_prompt_padding():
    """Left-padded prompts: masked prompt tokens are dropped for the whole group."""
    rng = np.random.default_rng(5)
    B, P, R = 6, 10, 5
    ids = rng.integers(1, 9, size=(B, P + R))
    ids[:3, :P] = ids[0, :P]
    ids[3:, :P] = ids[0, :P] + 10   # a second, different prompt
    mask = np.ones_like(ids)
    mask[:3, :4] = 0      # left pads on group 0's prompt
    mask[1, P + 2:] = 0    # short response
    mask[4, P:] = 0        # all-pad response
    pos = np.cumsum(mask, 1) - 1
    groups, uniq = oracle.find_prompt_groups(ids, R)
    info = _check_plan(ids, pos, mask, R, True, groups, uniq)
    assert info["prompt_len"].tolist() == [6, 10]
    assert info["resp_len"].tolist() == [5, 2, 5, 5, 0, 5]


def test_reconstruct_round_trip():
    rng = np.random.default_rng(7)
    w = WORKLOADS["tiny_fp32"].scaled(resp_len_range=(0, 32))
    bt = make_batch(w, permute=True)
    groups, uniq = oracle.find_prompt_groups(bt.input_ids, bt.response_length)
    _, _, info = oracle.create_deduplicated_batch(bt.input_ids, bt.position_ids, bt.response_length,
                                                  groups, uniq, attention_mask=bt.attention_mask,
                                                  use_unpad=True)
    B, S, W = w.batch, w.seq_len, 5
    X = rng.standard_normal((B, S, W))
    P = w.prompt_len
    for m in groups:      # prompt rows identical within a group, as for real hidden states
        X[m, :P] = X[m[0], :P]
    packed = oracle.pack_rows(X, info)
    assert packed.shape == (info["T"], W)
    Y = oracle.reconstruct_sequences(packed[None], info)
    keep = bt.attention_mask != 0
    np.testing.assert_array_equal(Y[keep], X[keep])
    assert not Y[~keep].any()
    # 2-D input is accepted too and gives the same
    np.testing.assert_array_equal(oracle.reconstruct_sequences(packed, info), Y)


# ---------------------------------------------------------------- backward of reconstruct / pack_rows
# Correctness & Gradients: gradients flow back through the reconstruction and
# the deduplication.  Both maps are linear, so their gradients are pinned by
# the adjoint identity <F(x), y> = <x, F^T(y)>, by torch autograd through an
# independent formulation (a gather by dst), and by closed forms.

def _info(use_unpad, permute=True, resp_len_range=(0, 32)):
    w = WORKLOADS["tiny_fp32"].scaled(resp_len_range=resp_len_range)
    bt = make_batch(w, permute=permute)
    groups, uniq = oracle.find_prompt_groups(bt.input_ids, bt.response_length)
    _, _, info = oracle.create_deduplicated_batch(bt.input_ids, bt.position_ids, bt.response_length,
                                                  groups, uniq, attention_mask=bt.attention_mask,
                                                  use_unpad=use_unpad)
    return w, bt, groups, info


def _adjoint_gap(fwd, bwd, x, y):
    lhs = float(np.sum(fwd(x) * y))
    rhs = float(np.sum(x * bwd(y)))
    return abs(lhs - rhs), float(np.sum(np.abs(fwd(x) * y)))


@pytest.mark.parametrize("use_unpad", [False, True])
def test_reconstruct_backward_is_the_adjoint(use_unpad):
    w, bt, groups, info = _info(use_unpad)
    rng = np.random.default_rng(21)
    for _ in range(4):
        x = rng.standard_normal((info["T"], 3))
        y = rng.standard_normal((w.batch, w.seq_len, 3))
        gap, scale = _adjoint_gap(lambda a: oracle.reconstruct_sequences(a, info),
                                  lambda a: oracle.reconstruct_backward(a, info), x, y)
        assert gap <= 1e-12 * scale


@pytest.mark.parametrize("use_unpad", [False, True])
def test_pack_rows_backward_is_the_adjoint(use_unpad):
    w, bt, groups, info = _info(use_unpad)
    rng = np.random.default_rng(22)
    for _ in range(4):
        x = rng.standard_normal((w.batch, w.seq_len, 3))
        y = rng.standard_normal((info["T"], 3))
        gap, scale = _adjoint_gap(lambda a: oracle.pack_rows(a, info),
                                  lambda a: oracle.pack_rows_backward(a, info), x, y)
        assert gap <= 1e-12 * scale


def test_reconstruct_backward_matches_autograd_gather():
    """torch autograd through reconstruct written as a gather by dst (zero row for dst = -1)."""
    torch = pytest.importorskip("torch")
    w, bt, groups, info = _info(True)
    rng = np.random.default_rng(23)
    x = torch.tensor(rng.standard_normal((info["T"], 4)), dtype=torch.float64, requires_grad=True)
    y = torch.tensor(rng.standard_normal((w.batch * w.seq_len, 4)), dtype=torch.float64)
    dst = torch.tensor(np.asarray(info["dst"]), dtype=torch.int64)
    padded = torch.cat([x, torch.zeros((1, 4), dtype=torch.float64)])
    out = padded[torch.where(dst >= 0, dst, torch.full_like(dst, info["T"]))]
    (out * y).sum().backward()
    ref = oracle.reconstruct_backward(y.numpy().reshape(w.batch, w.seq_len, 4), info)
    np.testing.assert_allclose(x.grad.numpy(), ref, rtol=0, atol=1e-13)


@pytest.mark.parametrize("use_unpad", [False, True])
def test_reconstruct_backward_ones_count_readers(use_unpad):
    """All-ones output gradient: a prompt row collects one per member, a response row one."""
    w, bt, groups, info = _info(use_unpad)
    g = oracle.reconstruct_backward(np.ones((w.batch, w.seq_len)), info)
    for gi, members in enumerate(groups):
        po, pl = info["prompt_off"][gi], info["prompt_len"][gi]
        assert (g[po:po + pl] == len(members)).all()
        for b in members:
            ro, rl = info["resp_off"][b], info["resp_len"][b]
            assert (g[ro:ro + rl] == 1).all()
    # every packed row is a prompt row or a response row
    assert g.sum() == sum(len(m) * info["prompt_len"][i] for i, m in enumerate(groups)) + info["resp_len"].sum()


@pytest.mark.parametrize("use_unpad", [False, True])
def test_pack_rows_backward_marks_sources(use_unpad):
    """All-ones packed gradient lands exactly on the first member's prompt and every response."""
    w, bt, groups, info = _info(use_unpad)
    d = oracle.pack_rows_backward(np.ones(info["T"], dtype=np.int64), info)
    P = w.prompt_len
    keep = bt.attention_mask != 0 if use_unpad else np.ones((w.batch, w.seq_len), bool)
    expect = np.zeros((w.batch, w.seq_len), np.int64)
    for members in groups:
        expect[members[0], :P] = keep[members[0], :P]
        for b in members:
            expect[b, P:] = keep[b, P:]
    np.testing.assert_array_equal(d, expect)
    assert d.sum() == info["T"]


def test_planted_mistake_in_reconstruct_backward_is_caught():
    """A backward that forgets the non-first members fails the adjoint identity."""
    w, bt, groups, info = _info(False, resp_len_range=None)

    def wrong(dout, info):
        out = oracle.reconstruct_backward(dout, info)
        for gi, members in enumerate(groups):
            po, pl = info["prompt_off"][gi], info["prompt_len"][gi]
            out[po:po + pl] = np.asarray(dout)[members[0], info["prompt_cols"][members[0]]]
        return out

    rng = np.random.default_rng(24)
    x = rng.standard_normal((info["T"], 3))
    y = rng.standard_normal((w.batch, w.seq_len, 3))
    gap, scale = _adjoint_gap(lambda a: oracle.reconstruct_sequences(a, info), lambda a: wrong(a, info), x, y)
    assert gap > 1e-3 * scale


@pytest.mark.parametrize("use_unpad", [False, True])
def test_full_batch_layout_is_samples_concatenated(use_unpad):
    """Standard QKV Optimization: with every sample its own group the packed layout is the full batch,
    sample after sample, each its kept prompt then its kept response tokens."""
    w = WORKLOADS["tiny_fp32"].scaled(resp_len_range=(0, 32))
    bt = make_batch(w, permute=True)
    P = w.prompt_len
    groups = [[b] for b in range(w.batch)]
    ids, pos, info = oracle.create_deduplicated_batch(bt.input_ids, bt.position_ids, bt.response_length, groups,
                                                      bt.input_ids[:, :P], attention_mask=bt.attention_mask,
                                                      use_unpad=use_unpad)
    keep = bt.attention_mask != 0 if use_unpad else np.ones(bt.input_ids.shape, bool)
    np.testing.assert_array_equal(np.asarray(ids).ravel(), bt.input_ids[keep])
    np.testing.assert_array_equal(np.asarray(pos).ravel(), bt.position_ids[keep])
    assert info["T"] == keep.sum()


# ---------------------------------------------------------------- Flash Attention Integration: varlen parameters

def _block_mask(q_lens, k_lens, style, rng):
    Tq, Tk = sum(q_lens), sum(k_lens)
    m = np.zeros((Tq, Tk), bool)
    r0 = c0 = 0
    for ql, kl in zip(q_lens, k_lens):
        for i in range(ql):
            if style == "full":
                hi = kl
            elif style == "causal":            # top-left aligned
                hi = min(kl, i + 1)
            else:                              # bottom-right aligned: the last query sees every key
                hi = kl - ql + i + 1
            if hi > 0:
                m[r0 + i, c0:c0 + hi] = True
        r0, c0 = r0 + ql, c0 + kl
    return m


@pytest.mark.parametrize("style", ["full", "causal", "bottom_right"])
def test_mask_to_flash_params_round_trip(style):
    rng = np.random.default_rng(31)
    for _ in range(5):
        n = int(rng.integers(1, 7))
        k_lens = rng.integers(1, 12, n).tolist()
        q_lens = rng.integers(1, 12, n).tolist()
        if style == "causal":
            # square blocks: with fewer queries than keys no query would see the last block's trailing keys,
            # and the mask could not fix that block's key length
            q_lens = list(k_lens)
        p = oracle.attention_mask_to_flash_attn_params(_block_mask(q_lens, k_lens, style, rng))
        np.testing.assert_array_equal(p["cu_seqlens_q"], np.concatenate([[0], np.cumsum(q_lens)]))
        np.testing.assert_array_equal(p["cu_seqlens_k"], np.concatenate([[0], np.cumsum(k_lens)]))
        assert p["max_seqlen_q"] == max(q_lens) and p["max_seqlen_k"] == max(k_lens)
        assert p["num_seqs"] == n and p["mismatched_rows"] == 0


def test_varlen_params_match_the_masks_of_the_two_calls():
    """Prompt-to-prompt and response-to-full masks built from the plan's definition convert to varlen_params."""
    w = WORKLOADS["tiny_fp32"].scaled(num_prompts=3, rollout_n=3, resp_len_range=(1, 32), seed=41)
    bt = make_batch(w, permute=True)
    groups, uniq = oracle.find_prompt_groups(bt.input_ids, bt.response_length)
    _, _, info = oracle.create_deduplicated_batch(bt.input_ids, bt.position_ids, bt.response_length, groups, uniq,
                                                  attention_mask=bt.attention_mask, use_unpad=True)
    vp = oracle.varlen_params(info)
    pl, rl, gof = info["prompt_len"], info["resp_len"], info["group_of"]
    # prompt-to-prompt: each prompt causally over itself
    tot = int(sum(pl))
    mp = np.zeros((tot, tot), bool)
    o = 0
    for g in range(info["G"]):
        for i in range(pl[g]):
            mp[o + i, o:o + i + 1] = True
        o += pl[g]
    p = oracle.attention_mask_to_flash_attn_params(mp)
    np.testing.assert_array_equal(p["cu_seqlens_q"], vp["cu_seqlens_prompt"])
    np.testing.assert_array_equal(p["cu_seqlens_k"], vp["cu_seqlens_prompt"])
    # response-to-full: response row i of sample b sees its prompt and its own keys 0..i
    Tq, Tk = int(sum(rl)), int(sum(pl[gof[b]] + rl[b] for b in range(info["B"])))
    mr = np.zeros((Tq, Tk), bool)
    qo = ko = 0
    for b in range(info["B"]):
        P = pl[gof[b]]
        for i in range(rl[b]):
            mr[qo + i, ko:ko + P + i + 1] = True
        qo, ko = qo + rl[b], ko + P + rl[b]
    p = oracle.attention_mask_to_flash_attn_params(mr)
    np.testing.assert_array_equal(p["cu_seqlens_q"], vp["cu_seqlens_q"])
    np.testing.assert_array_equal(p["cu_seqlens_k"], vp["cu_seqlens_k"])
    assert p["max_seqlen_q"] == vp["max_seqlen_q"] and p["max_seqlen_k"] == vp["max_seqlen_k"]
    assert vp["cu_seqlens_k"][-1] == sum(pl[gof[b]] + rl[b] for b in range(info["B"]))


def test_mask_to_flash_params_reports_non_block_masks():
    m = _block_mask([3, 3], [4, 4], "full", None)
    m[4, 1] = True                    # a row of block 1 also sees a key of block 0
    assert oracle.attention_mask_to_flash_attn_params(m)["mismatched_rows"] >= 1
    p = oracle.attention_mask_to_flash_attn_params(np.zeros((3, 5), bool))
    assert p["num_seqs"] == 0 and p["cu_seqlens_q"].tolist() == [0]


# ---------------------------------------------------------------- shared prefix (prefix caching)

def _prefix_batch(G=3, n=2, L=11, P=20, R=6, seed=61, vocab=9, unpad=False):
    """G distinct prompts sharing their first L columns (and differing at column L), n responses each."""
    rng = np.random.default_rng(seed)
    B, S = G * n, P + R
    ids = rng.integers(1, vocab, size=(B, S))
    common = rng.integers(1, vocab, size=L)
    tails = []
    for g in range(G):
        t = rng.integers(1, vocab, size=P - L)
        if L < P:
            t[0] = (g % (vocab - 1)) + 1          # column L differs between groups
        tails.append(t)
    for b in range(B):
        ids[b, :L] = common
        ids[b, L:P] = tails[b // n]
    pos = np.tile(np.arange(S), (B, 1))
    mask = np.ones((B, S), np.int64)
    if unpad:
        for b in range(B):
            mask[b, P + int(rng.integers(0, R + 1)):] = 0
    return ids, pos, mask, R


@pytest.mark.parametrize("L", [0, 1, 7, 19, 20])
def test_find_shared_prefix_planted(L):
    ids, pos, mask, R = _prefix_batch(L=L)
    groups, _ = oracle.find_prompt_groups(ids, R)
    got = oracle.find_shared_prefix(ids, R, groups)
    P = ids.shape[1] - R
    # brute force over all pairs of samples
    def lcp(a, b):
        k = 0
        while k < P and ids[a, k] == ids[b, k]:
            k += 1
        return k
    brute = min(lcp(a, b) for a in range(len(ids)) for b in range(len(ids))) if len(groups) > 1 else 0
    assert got == brute
    if L < P:
        assert got == L


@pytest.mark.parametrize("unpad", [False, True])
def test_prefix_layout_and_round_trip(unpad):
    ids, pos, mask, R = _prefix_batch(unpad=unpad)
    groups, uniq = oracle.find_prompt_groups(ids, R)
    L0 = oracle.find_shared_prefix(ids, R, groups)
    dids, dpos, info = oracle.create_deduplicated_batch(ids, pos, R, groups, uniq, attention_mask=mask,
                                                        use_unpad=unpad, prefix_len=L0)
    P = ids.shape[1] - R
    keep = mask != 0
    # [prefix once][suffix of g][responses of g] ...
    expect = list(ids[0, :L0])
    for m in groups:
        expect += list(ids[m[0], L0:P])
        for b in m:
            expect += list(ids[b, P:][keep[b, P:]])
    np.testing.assert_array_equal(np.asarray(dids).ravel(), expect)
    assert info["prefix_len"] == L0 and info["T"] == L0 + sum(P - L0 for _ in groups) + keep[:, P:].sum()
    X = np.random.default_rng(3).standard_normal((ids.shape[0], ids.shape[1], 4))
    X[:, :L0] = X[0, :L0]
    for m in groups:
        X[m, :P] = X[m[0], :P]
    Y = oracle.reconstruct_sequences(oracle.pack_rows(X, info), info)
    np.testing.assert_array_equal(Y[keep], X[keep])
    # backward of reconstruct: a prefix row collects every sample
    g = oracle.reconstruct_backward(np.ones(ids.shape), info)
    assert (g[:L0] == ids.shape[0]).all()
    x = np.random.default_rng(4).standard_normal((info["T"], 3))
    y = np.random.default_rng(5).standard_normal(ids.shape + (3,))
    lhs = np.sum(oracle.reconstruct_sequences(x, info) * y)
    rhs = np.sum(x * oracle.reconstruct_backward(y, info))
    assert abs(lhs - rhs) <= 1e-12 * np.abs(y).sum() * np.abs(x).max()
