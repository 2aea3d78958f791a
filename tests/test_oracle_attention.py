"""Pins for the oracle's split attention (CPU only).

The oracle is tied to things other than itself:
  * a library attention routine (torch scaled_dot_product_attention, fp64,
    causal) run per sample, and torch.autograd through the packed-output
    function built from it;
  * special cases that reduce to plain causal attention;
  * closed forms (constant V, zero Q, the first row);
  * fp64 central finite differences;
  * exact invariants of softmax attention gradients;
  * brute-force pair counting.
A few tests plant a mistake in the oracle (monkeypatched, CPU only) and check
that the pins catch it.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import oracle.attention as oatt
from workloads import WORKLOADS, make_attn_inputs, make_batch


def _setup(w, permute=False, seed=None):
    bt = make_batch(w, permute=permute)
    groups, uniq = oracle.find_prompt_groups(bt.input_ids, bt.response_length)
    _, _, info = oracle.create_deduplicated_batch(
        bt.input_ids, bt.position_ids, bt.response_length, groups, uniq,
        attention_mask=bt.attention_mask, use_unpad=w.use_unpad)
    x = make_attn_inputs(w, info["T"])
    return info, x


SMALL = {
    "tiny": WORKLOADS["tiny_fp32"],
    "gqa_ragged_unpad": WORKLOADS["tiny_fp32"].scaled(
        name="gqa_ragged_unpad", num_prompts=3, rollout_n=3, prompt_len=37, response_len=21,
        num_q_heads=4, num_kv_heads=2, head_dim=16, resp_len_range=(0, 21), seed=77),
    "mha": WORKLOADS["tiny_fp32"].scaled(name="mha", num_q_heads=3, num_kv_heads=3, head_dim=8,
                                         prompt_len=20, response_len=9, seed=78),
}


def _sdpa_packed(q, k, v, info, scale):
    """Packed output assembled from per-sample torch SDPA (fp64, causal, kv heads repeated)."""
    T, Hq, d = q.shape
    ratio = Hq // k.shape[1]
    outs = []
    for b in range(info["B"]):
        idx = torch.as_tensor(oracle.sample_rows(info, b))
        Q = q[idx].transpose(0, 1)
        K = k[idx].repeat_interleave(ratio, dim=1).transpose(0, 1)
        V = v[idx].repeat_interleave(ratio, dim=1).transpose(0, 1)
        outs.append((idx, F.scaled_dot_product_attention(Q, K, V, is_causal=True, scale=scale)
                     .transpose(0, 1)))
    o = torch.zeros_like(q)
    out_rows = [None] * T
    for b, (idx, ob) in enumerate(outs):
        g = info["group_of"][b]
        pl = int(info["prompt_len"][g])
        for i, j in enumerate(idx.tolist()):
            if i >= pl or b == info["rep"][g]:
                out_rows[j] = ob[i]
    return torch.stack(out_rows) if T else o


@pytest.mark.parametrize("name", list(SMALL))
def test_forward_matches_library_sdpa(name):
    info, x = _setup(SMALL[name], permute=True)
    scale = 1.0 / math.sqrt(SMALL[name].head_dim)
    o, lse = oracle.split_attention_forward(x.q, x.k, x.v, info)
    ref = _sdpa_packed(*(torch.from_numpy(a.astype(np.float64)) for a in (x.q, x.k, x.v)), info, scale)
    np.testing.assert_allclose(o, ref.numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("name", list(SMALL))
def test_backward_matches_autograd(name):
    info, x = _setup(SMALL[name], permute=True)
    scale = 1.0 / math.sqrt(SMALL[name].head_dim)
    q, k, v = (torch.from_numpy(a.astype(np.float64)).requires_grad_() for a in (x.q, x.k, x.v))
    out = _sdpa_packed(q, k, v, info, scale)
    (out * torch.from_numpy(x.do.astype(np.float64))).sum().backward()
    dq, dk, dv = oracle.split_attention_backward(x.q, x.k, x.v, x.do, info)
    for got, ref in ((dq, q.grad), (dk, k.grad), (dv, v.grad)):
        np.testing.assert_allclose(got, ref.numpy(), rtol=0, atol=1e-11)


def test_single_response_is_plain_causal():
    w = SMALL["mha"].scaled(num_prompts=1, rollout_n=1, seed=9)
    info, x = _setup(w)
    o, lse = oracle.split_attention_forward(x.q, x.k, x.v, info)
    Q, K, V = (torch.from_numpy(a.astype(np.float64)).transpose(0, 1) for a in (x.q, x.k, x.v))
    ref = F.scaled_dot_product_attention(Q, K, V, is_causal=True).transpose(0, 1)
    np.testing.assert_allclose(o, ref.numpy(), atol=1e-12, rtol=0)
    # the log-sum-exp, by direct definition on the same single sequence
    s = (Q @ K.transpose(1, 2)) / math.sqrt(w.head_dim)
    s = s.masked_fill(torch.triu(torch.ones(info["T"], info["T"], dtype=torch.bool), 1), -math.inf)
    np.testing.assert_allclose(lse, torch.logsumexp(s, -1).numpy(), atol=1e-12, rtol=0)


def test_empty_responses_reduce_to_prompt_attention():
    w = SMALL["mha"].scaled(num_prompts=1, rollout_n=2, resp_len_range=(0, 0), seed=10)
    info, x = _setup(w)
    assert info["T"] == w.prompt_len
    o, _ = oracle.split_attention_forward(x.q, x.k, x.v, info)
    Q, K, V = (torch.from_numpy(a.astype(np.float64)).transpose(0, 1) for a in (x.q, x.k, x.v))
    ref = F.scaled_dot_product_attention(Q, K, V, is_causal=True).transpose(0, 1)
    np.testing.assert_allclose(o, ref.numpy(), atol=1e-12, rtol=0)


def test_closed_forms():
    w = SMALL["gqa_ragged_unpad"]
    info, x = _setup(w)
    x.v = x.v.astype(np.float64)
    T, Hq, d = x.q.shape
    # constant V rows -> every output is that constant
    v_const = np.broadcast_to(np.linspace(-1, 1, d), x.v.shape).copy()
    o, _ = oracle.split_attention_forward(x.q, x.k, v_const, info)
    np.testing.assert_allclose(o, np.broadcast_to(np.linspace(-1, 1, d), o.shape), atol=1e-13)
    # Q = 0 -> uniform softmax: output is the mean of the visible V rows, LSE = log(#visible)
    o, lse = oracle.split_attention_forward(np.zeros_like(x.q), x.k, x.v, info)
    ratio = Hq // x.k.shape[1]
    for g in range(info["G"]):
        po, pl = info["prompt_off"][g], info["prompt_len"][g]
        for i in range(pl):            # prompt row i: prefix mean of its own prompt
            vis = np.arange(po, po + i + 1)
            for h in range(Hq):
                np.testing.assert_allclose(o[po + i, h], x.v[vis, h // ratio].mean(0), atol=1e-13)
                assert abs(lse[h, po + i] - math.log(len(vis))) < 1e-13
        for b in info["groups"][g]:
            ro, rl = info["resp_off"][b], info["resp_len"][b]
            for i in range(rl):        # response row i: all prompt keys plus own keys 0..i
                vis = np.concatenate([np.arange(po, po + pl), np.arange(ro, ro + i + 1)])
                for h in range(Hq):
                    np.testing.assert_allclose(o[ro + i, h], x.v[vis, h // ratio].mean(0), atol=1e-13)
                    assert abs(lse[h, ro + i] - math.log(len(vis))) < 1e-13
    # first prompt row sees only itself
    o, _ = oracle.split_attention_forward(x.q, x.k, x.v, info)
    for g in range(info["G"]):
        po = info["prompt_off"][g]
        for h in range(Hq):
            np.testing.assert_allclose(o[po, h], x.v[po, h // ratio], atol=1e-14)


def test_finite_differences():
    w = WORKLOADS["tiny_fp32"].scaled(prompt_len=12, response_len=5, head_dim=8, seed=11)
    info, x = _setup(w, permute=True)
    rng = np.random.default_rng(3)
    q, k, v, do = (a.astype(np.float64) for a in (x.q, x.k, x.v, x.do))
    dq, dk, dv = oracle.split_attention_backward(q, k, v, do, info)

    def loss(q_, k_, v_):
        o, _ = oracle.split_attention_forward(q_, k_, v_, info)
        return float((o * do).sum())

    h = 1e-6
    for _ in range(3):
        eq, ek, ev = (rng.standard_normal(a.shape) for a in (q, k, v))
        fd = (loss(q + h * eq, k + h * ek, v + h * ev) - loss(q - h * eq, k - h * ek, v - h * ev)) / (2 * h)
        an = (dq * eq).sum() + (dk * ek).sum() + (dv * ev).sum()
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (fd, an)


@pytest.mark.parametrize("name", ["tiny", "gqa_ragged_unpad"])
def test_gradient_invariants(name):
    info, x = _setup(SMALL[name], permute=True)
    dq, dk, dv = oracle.split_attention_backward(x.q, x.k, x.v, x.do, info)
    Hq, Hkv = x.q.shape[1], x.k.shape[1]
    ratio = Hq // Hkv
    do = x.do.astype(np.float64)
    for j in range(Hkv):
        # softmax rows sum to 1: the values' gradient sums to the output gradient
        np.testing.assert_allclose(dv[:, j].sum(0), do[:, j * ratio:(j + 1) * ratio].sum((0, 1)),
                                   atol=1e-11)
        # rows of dS sum to 0: the keys' gradient sums to 0
        np.testing.assert_allclose(dk[:, j].sum(0), 0.0, atol=1e-11)


def test_sampled_rows_match_full():
    w = SMALL["gqa_ragged_unpad"]
    info, x = _setup(w, permute=True)
    o, lse = oracle.split_attention_forward(x.q, x.k, x.v, info)
    dq, dk, dv = oracle.split_attention_backward(x.q, x.k, x.v, x.do, info)
    rows = np.random.default_rng(1).choice(info["T"], 12, replace=False)
    heads = [0, 3]
    o_s, lse_s = oracle.forward_rows(x.q, x.k, x.v, info, rows, heads)
    np.testing.assert_allclose(o_s, o[rows][:, heads], atol=1e-13)
    np.testing.assert_allclose(lse_s, lse[heads][:, rows].T, atol=1e-13)
    dq_s = oracle.dq_rows(x.q, x.k, x.v, x.do, info, rows, heads)
    np.testing.assert_allclose(dq_s, dq[rows][:, heads], atol=1e-12)
    dk_s, dv_s = oracle.dkdv_rows(x.q, x.k, x.v, x.do, info, rows, [0, 1])
    np.testing.assert_allclose(dk_s, dk[rows], atol=1e-12)
    np.testing.assert_allclose(dv_s, dv[rows], atol=1e-12)
    # every key at once, in a scrambled order: the keys of a sample share one pass over its rows
    every = np.random.default_rng(2).permutation(info["T"])
    dk_a, dv_a = oracle.dkdv_rows(x.q, x.k, x.v, x.do, info, every, [1, 0])
    np.testing.assert_allclose(dk_a, dk[every][:, [1, 0]], atol=1e-12)
    np.testing.assert_allclose(dv_a, dv[every][:, [1, 0]], atol=1e-12)


def test_sampled_keys_match_full_across_row_blocks():
    """Sequences of several 512-row blocks: a key read by later blocks only, keys in every block."""
    w = WORKLOADS["tiny_fp32"].scaled(name="blocks", num_prompts=2, rollout_n=2, prompt_len=700, response_len=400,
                                      num_q_heads=2, num_kv_heads=1, head_dim=8, resp_len_range=(100, 400), seed=77)
    info, x = _setup(w, permute=True)
    _, dk, dv = oracle.split_attention_backward(x.q, x.k, x.v, x.do, info)
    keys = np.random.default_rng(6).permutation(info["T"])[:300]
    keys = np.concatenate([keys, [int(info["prompt_off"][0]), int(info["prompt_off"][1]) + 650]])
    dk_s, dv_s = oracle.dkdv_rows(x.q, x.k, x.v, x.do, info, keys, [0])
    np.testing.assert_allclose(dk_s, dk[keys], atol=1e-11)
    np.testing.assert_allclose(dv_s, dv[keys], atol=1e-11)


def test_sampled_keys_match_full_with_shared_prefix():
    """Prefix keys are read by every sample; the batched key pass must collect all of them."""
    _, _, info = _prefix_setup()
    q, k, v, do = _qkv(info["T"])
    _, dk, dv = oracle.split_attention_backward(q, k, v, do, info)
    keys = np.random.default_rng(4).permutation(info["T"])
    dk_s, dv_s = oracle.dkdv_rows(q, k, v, do, info, keys, [0, 1])
    np.testing.assert_allclose(dk_s, dk[keys], atol=1e-12)
    np.testing.assert_allclose(dv_s, dv[keys], atol=1e-12)


def test_attended_pairs_brute_force():
    for name in SMALL:
        info, _ = _setup(SMALL[name], permute=True)
        pairs = set()
        plain = 0
        for b in range(info["B"]):
            idx = oracle.sample_rows(info, b)
            plain += len(idx) * (len(idx) + 1) // 2
            for i in range(len(idx)):
                for kk in range(i + 1):
                    pairs.add((int(idx[i]), int(idx[kk])))
        assert oracle.attended_pairs(info) == (len(pairs), plain)


# --- planted mistakes: each must be caught by one of the pins above -------------------------

def _planted_causal_block_off_by_one(Qs, Ks, Vs, i0, i1, scale, dOs=None):
    s = scale * (Qs[i0:i1] @ Ks[:i1].T)
    future = np.arange(i1)[None, :] >= np.arange(i0, i1)[:, None]   # drops the diagonal key
    future[:, 0] = False
    s[future] = -np.inf
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    p = e / l
    o = p @ Vs[:i1]
    lse = (m + np.log(l))[:, 0]
    if dOs is None:
        return p, o, lse, None
    dO = dOs[i0:i1]
    dS = p * (dO @ Vs[:i1].T - (dO * o).sum(axis=1, keepdims=True))
    return p, o, lse, dS


def test_planted_mask_mistake_is_caught(monkeypatch):
    monkeypatch.setattr(oatt, "_causal_block", _planted_causal_block_off_by_one)
    with pytest.raises(AssertionError):
        test_forward_matches_library_sdpa("tiny")


def test_planted_gqa_mistake_is_caught(monkeypatch):
    monkeypatch.setattr(oatt, "_kv_head", lambda h, Hq, Hkv: h % Hkv)
    with pytest.raises(AssertionError):
        test_forward_matches_library_sdpa("gqa_ragged_unpad")


def test_planted_sibling_leak_is_caught(monkeypatch):
    """A response that also saw its siblings' rows must fail the pins."""
    real = oracle.dedup.sample_rows

    def leaky(info, b):
        g = info["group_of"][b]
        first = info["groups"][g][0]
        idx = real(info, b)
        if b != first:
            extra = real(info, first)[info["prompt_len"][g]:]
            pl = info["prompt_len"][g]
            idx = np.concatenate([idx[:pl], extra, idx[pl:]])
        return idx

    monkeypatch.setattr(oatt, "sample_rows", leaky)
    with pytest.raises(AssertionError):
        test_closed_forms()


def test_planted_prompt_grad_mistake_is_caught(monkeypatch):
    """Counting prompt rows' dO once per member (not once) must fail the autograd pin."""
    real = oatt.split_attention_backward

    def doubled(q, k, v, dout, info, scale=None):
        q_, k_, v_, T, Hq, Hkv, d, scale = oatt._prep(q, k, v, scale)
        dq = np.zeros_like(q_)
        dk = np.zeros_like(k_)
        dv = np.zeros_like(v_)
        for b in range(info["B"]):
            idx = oracle.sample_rows(info, b)
            for h in range(Hq):
                j = h // (Hq // Hkv)
                L = len(idx)
                p, _, _, dS = oatt._causal_block(q_[idx, h], k_[idx, j], v_[idx, j], 0, L, scale,
                                                 np.asarray(dout, np.float64)[idx, h])
                dv[idx, j] += p.T @ np.asarray(dout, np.float64)[idx, h]
                dq[idx, h] += scale * dS @ k_[idx, j]
                dk[idx, j] += scale * dS.T @ q_[idx, h]
        return dq, dk, dv

    monkeypatch.setattr(oracle, "split_attention_backward", doubled)
    with pytest.raises(AssertionError):
        test_backward_matches_autograd("tiny")
    assert real is not doubled


# ---------------------------------------------------------------- padded format with an attention mask
# Working with Packed/Unpacked Sequences: in the padded format the pads stay
# in the packed sequence; the reading here is that they take no part in
# attention (no sample's key; their outputs and gradients are 0).

def _padded_with_mask(seed=81):
    w = SMALL["gqa_ragged_unpad"].scaled(seed=seed)
    bt = make_batch(w, permute=True)
    mask = bt.attention_mask.copy()
    groups, uniq = oracle.find_prompt_groups(bt.input_ids, bt.response_length)
    mask[groups[0], :4] = 0          # left pads on group 0's prompt (every member)
    _, _, info = oracle.create_deduplicated_batch(bt.input_ids, bt.position_ids, bt.response_length, groups, uniq,
                                                  attention_mask=mask, use_unpad=False)
    x = make_attn_inputs(w, info["T"])
    valid = mask.reshape(-1)[info["src"]] != 0
    return w, bt, mask, groups, uniq, info, x, valid


def _sdpa_packed_masked(q, k, v, info, scale, valid):
    """Per sample: SDPA over all its rows with keys masked to (key <= query) and valid, for its valid query
    rows; pad rows are 0."""
    T, Hq, d = q.shape
    ratio = Hq // k.shape[1]
    rows = [None] * T
    for b in range(info["B"]):
        idx = np.asarray(oracle.sample_rows(info, b))
        g = info["group_of"][b]
        pl = int(info["prompt_len"][g])
        L = len(idx)
        vk = torch.as_tensor(valid[idx])
        allowed = torch.tril(torch.ones(L, L, dtype=torch.bool)) & vk[None, :]
        qrows = np.nonzero(valid[idx])[0]
        if len(qrows) == 0:
            continue
        ti = torch.as_tensor(idx)
        Q = q[ti[qrows]].transpose(0, 1)
        K = k[ti].repeat_interleave(ratio, dim=1).transpose(0, 1)
        V = v[ti].repeat_interleave(ratio, dim=1).transpose(0, 1)
        ob = F.scaled_dot_product_attention(Q, K, V, attn_mask=allowed[qrows], scale=scale).transpose(0, 1)
        for n, i in enumerate(qrows.tolist()):
            if i >= pl or b == info["rep"][g]:
                rows[idx[i]] = ob[n]
    zero = torch.zeros((Hq, d), dtype=q.dtype)
    return torch.stack([r if r is not None else zero for r in rows])


def test_padded_with_mask_matches_library_sdpa():
    w, bt, mask, groups, uniq, info, x, valid = _padded_with_mask()
    assert (~valid).sum() > 4          # pads in prompts and responses
    scale = 1.0 / math.sqrt(w.head_dim)
    o, _ = oracle.split_attention_forward(x.q, x.k, x.v, info, valid=valid)
    ref = _sdpa_packed_masked(*(torch.from_numpy(a.astype(np.float64)) for a in (x.q, x.k, x.v)), info, scale, valid)
    np.testing.assert_allclose(o, ref.numpy(), rtol=0, atol=1e-12)
    assert not o[~valid].any()


def test_padded_with_mask_backward_matches_autograd():
    w, bt, mask, groups, uniq, info, x, valid = _padded_with_mask()
    scale = 1.0 / math.sqrt(w.head_dim)
    q, k, v = (torch.from_numpy(a.astype(np.float64)).requires_grad_() for a in (x.q, x.k, x.v))
    out = _sdpa_packed_masked(q, k, v, info, scale, valid)
    (out * torch.from_numpy(x.do.astype(np.float64))).sum().backward()
    dq, dk, dv = oracle.split_attention_backward(x.q, x.k, x.v, x.do, info, valid=valid)
    for got, ref in ((dq, q.grad), (dk, k.grad), (dv, v.grad)):
        np.testing.assert_allclose(got, ref.numpy(), rtol=0, atol=1e-11)
    for gr in (dq, dk, dv):
        assert not gr[~valid].any()


def test_padded_with_mask_equals_unpadded():
    """The valid rows of the padded format give what the unpadded format gives for the same tokens."""
    w, bt, mask, groups, uniq, info, x, valid = _padded_with_mask()
    _, _, info_u = oracle.create_deduplicated_batch(bt.input_ids, bt.position_ids, bt.response_length, groups, uniq,
                                                    attention_mask=mask, use_unpad=True)
    rows = np.nonzero(valid)[0]
    urows = np.asarray(info_u["dst"])[np.asarray(info["src"])[rows]]
    assert (urows >= 0).all() and len(urows) == info_u["T"]
    order = np.argsort(urows)
    src_rows = rows[order]                   # padded row of each unpadded row
    o, _ = oracle.split_attention_forward(x.q, x.k, x.v, info, valid=valid)
    ou, _ = oracle.split_attention_forward(x.q[src_rows], x.k[src_rows], x.v[src_rows], info_u)
    np.testing.assert_allclose(o[src_rows], ou, rtol=0, atol=1e-12)
    g = oracle.split_attention_backward(x.q, x.k, x.v, x.do, info, valid=valid)
    gu = oracle.split_attention_backward(x.q[src_rows], x.k[src_rows], x.v[src_rows], x.do[src_rows], info_u)
    for a, b in zip(g, gu):
        np.testing.assert_allclose(a[src_rows], b, rtol=0, atol=1e-11)


def test_planted_pad_key_leak_is_caught():
    """Treating the kept pads as keys (ignoring the mask) disagrees with the masked library pin."""
    w, bt, mask, groups, uniq, info, x, valid = _padded_with_mask()
    scale = 1.0 / math.sqrt(w.head_dim)
    wrong, _ = oracle.split_attention_forward(x.q, x.k, x.v, info)
    ref = _sdpa_packed_masked(*(torch.from_numpy(a.astype(np.float64)) for a in (x.q, x.k, x.v)), info, scale, valid)
    assert np.abs(wrong[valid] - ref.numpy()[valid]).max() > 1e-3


# ---------------------------------------------------------------- shared prefix (prefix caching)

def _prefix_setup(prefix=True, seed=91):
    import importlib
    tod = importlib.import_module("test_oracle_dedup")
    ids, pos, mask, R = tod._prefix_batch(G=3, n=2, L=13, P=24, R=9, seed=seed, unpad=True)
    groups, uniq = oracle.find_prompt_groups(ids, R)
    L0 = oracle.find_shared_prefix(ids, R, groups) if prefix else 0
    _, _, info = oracle.create_deduplicated_batch(ids, pos, R, groups, uniq, attention_mask=mask, use_unpad=True,
                                                  prefix_len=L0)
    return ids, mask, info


def _qkv(T, seed=5, Hq=4, Hkv=2, d=16):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal(s) * 0.7 for s in ((T, Hq, d), (T, Hkv, d), (T, Hkv, d), (T, Hq, d))]


def _sdpa_owner(q, k, v, info):
    """Per-sample torch SDPA over each sample's rows; each packed row from the sample it was packed from."""
    T, Hq, d = q.shape
    ratio = Hq // k.shape[1]
    owner = np.asarray(info["src"]) // info["S"]
    rows = [None] * T
    for b in range(info["B"]):
        idx = oracle.sample_rows(info, b)
        ti = torch.as_tensor(idx)
        Q = q[ti].transpose(0, 1)
        K = k[ti].repeat_interleave(ratio, dim=1).transpose(0, 1)
        V = v[ti].repeat_interleave(ratio, dim=1).transpose(0, 1)
        ob = F.scaled_dot_product_attention(Q, K, V, is_causal=True).transpose(0, 1)
        for i, j in enumerate(idx.tolist()):
            if owner[j] == b:
                rows[j] = ob[i]
    return torch.stack(rows)


def test_prefix_forward_backward_match_library():
    ids, mask, info = _prefix_setup()
    assert info["prefix_len"] == 13
    q, k, v, do = _qkv(info["T"])
    o, _ = oracle.split_attention_forward(q, k, v, info)
    tq, tk, tv = (torch.from_numpy(a).requires_grad_() for a in (q, k, v))
    ref = _sdpa_owner(tq, tk, tv, info)
    np.testing.assert_allclose(o, ref.detach().numpy(), rtol=0, atol=1e-12)
    (ref * torch.from_numpy(do)).sum().backward()
    for got, want in zip(oracle.split_attention_backward(q, k, v, do, info), (tq.grad, tk.grad, tv.grad)):
        np.testing.assert_allclose(got, want.numpy(), rtol=0, atol=1e-11)


def test_prefix_sharing_equals_exact_dedup_per_cell():
    """Packing the shared prefix once changes the layout, not the function: per (sample, column) outputs
    agree with the layout without it; a prefix key's gradient is the sum of the groups' copies."""
    ids, mask, pinfo = _prefix_setup(prefix=True)
    _, _, ninfo = _prefix_setup(prefix=False)
    B, S = ids.shape
    rng = np.random.default_rng(8)
    cells = {n: rng.standard_normal((B, S, 4, 16)) * 0.7 for n in ("q", "do")}
    kvc = {n: rng.standard_normal((B, S, 2, 16)) * 0.7 for n in ("k", "v")}
    # the same per-cell inputs (identical copies across the cells a packed row stands for)
    L0, P = pinfo["L0"], pinfo["P"]
    for a in list(cells.values()) + list(kvc.values()):
        a[:, :L0] = a[0, :L0]
        for m in pinfo["groups"]:
            a[m, L0:P] = a[m[0], L0:P]
    cells["do"][1:, :L0] = 0.0          # prefix outputs used from sample 0 only, in both layouts
    for m in ninfo["groups"]:
        cells["do"][m[1:], :P] = 0.0
    def run(info):
        pk = {n: oracle.pack_rows(a, info) for n, a in {**cells, **kvc}.items()}
        o, _ = oracle.split_attention_forward(pk["q"], pk["k"], pk["v"], info)
        g = oracle.split_attention_backward(pk["q"], pk["k"], pk["v"], pk["do"], info)
        return o, g
    (op, gp), (on, gn) = run(pinfo), run(ninfo)
    keep = mask != 0
    flat = lambda a: a.reshape(a.shape[0], -1)
    np.testing.assert_allclose(oracle.reconstruct_sequences(flat(op), pinfo)[keep],
                               oracle.reconstruct_sequences(flat(on), ninfo)[keep], rtol=0, atol=1e-12)
    # gradients: a packed row of the prefix layout collects the rows of the other layout it stands for
    # (spread each to its source cell, then sum the cells each prefix-layout row stands for)
    for a, b in zip(gp, gn):
        want = oracle.reconstruct_backward(oracle.pack_rows_backward(flat(b), ninfo), pinfo)
        np.testing.assert_allclose(flat(a), want, rtol=0, atol=1e-11)
