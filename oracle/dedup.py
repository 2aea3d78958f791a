"""Oracle: grouping, packing and reconstruction (exact integer work).

Test infrastructure only; see the package docstring.

Readings of the pages where they leave a step open (also listed in the
design notes of the repository):

* prompt region: the first ``S - response_length`` columns of every row
  (Finding Prompt Groups only says ``response_length`` is the length of the
  response portion);
* grouping key: exact equality of those prompt token ids, pad ids included
  (``find_prompt_groups`` takes no mask);
* order: groups in order of first occurrence, members ascending -- the
  pages' example ``[[0, 1], [2, 3]]`` is consistent with it;
* the prompt copy that is packed, and whose positions and mask are used, is
  the group's first member;
* positions are gathered from ``position_ids``, not renumbered;
* unpad keeps exactly the tokens whose mask is non-zero; reconstruction
  writes 0 where no packed token maps;
* a group whose members' responses are all padding still packs its prompt,
  and a sample with an all-pad response owns no packed rows.
"""
from __future__ import annotations

import numpy as np


def find_prompt_groups(input_ids: np.ndarray, response_length: int):
    """How Prompt Deduplication Works -- Core Algorithm, Finding Prompt Groups.

    Partition the samples into lists of indices whose prompt tokens are
    identical.  Brute force: every sample is compared token by token with the
    first member of each group found so far.

    Returns ``(prompt_groups, unique_prompts)`` with ``unique_prompts`` of
    shape ``[num_unique, prompt_len]``.
    """
    ids = np.asarray(input_ids)
    B, S = ids.shape
    P = S - int(response_length)
    if not (0 <= P <= S):
        raise ValueError("response_length must be in [0, seq_len]")
    groups: list[list[int]] = []
    for b in range(B):
        for members in groups:
            if np.array_equal(ids[b, :P], ids[members[0], :P]):
                members.append(b)
                break
        else:
            groups.append([b])
    unique_prompts = np.stack([ids[m[0], :P] for m in groups]) if groups else \
        np.zeros((0, P), dtype=ids.dtype)
    return groups, unique_prompts


def find_shared_prefix(input_ids, response_length, prompt_groups):
    """Key Limitations & Future Work -- prefix caching for partially
    overlapping prompts (the pages name it as a future direction; this is
    the plainest form of it).

    The number of leading prompt columns on which the first members of all
    groups agree: the batch's shared prefix.  0 with fewer than two groups
    (a single group already shares its whole prompt).
    """
    ids = np.asarray(input_ids)
    P = ids.shape[1] - int(response_length)
    if len(prompt_groups) < 2:
        return 0
    ref = ids[prompt_groups[0][0], :P]
    L = P
    for members in prompt_groups[1:]:
        diff = np.flatnonzero(ids[members[0], :P] != ref)
        if len(diff):
            L = min(L, int(diff[0]))
    return L


def create_deduplicated_batch(input_ids, position_ids, response_length, prompt_groups,
                              unique_prompts, attention_mask=None, use_unpad=False, prefix_len=0):
    """How Prompt Deduplication Works -- Creating Deduplicated Batch; Working with
    Packed/Unpacked Sequences.

    Builds ``[Prompt_1][Response_1_1][Response_1_2]...[Prompt_2][Response_2_1]...``
    as one ``[1, T]`` sequence of ids and of positions, plus the metadata that
    maps it back.  With ``use_unpad`` tokens whose mask is 0 are dropped.

    ``info`` (the pages' reconstruction metadata, whose fields they leave
    unspecified) holds, per group ``g``: ``prompt_off[g]``, ``prompt_len[g]``,
    ``rep[g]``; per sample ``b``: ``group_of[b]``, ``resp_off[b]``,
    ``resp_len[b]``, ``prompt_cols[b]``/``resp_cols[b]`` (the original columns
    kept, in order); and ``src[T]`` (packed row -> ``b*S + t``), ``dst[B*S]``
    ((b, t) -> packed row, or -1), ``seg_start[T]`` (first packed row of the
    segment each packed row lies in).

    With ``prefix_len = L0 > 0`` (a shared prefix, see ``find_shared_prefix``)
    the first ``L0`` prompt columns are packed once, from the first sample,
    ahead of everything: ``[prefix][suffix_1][responses of 1][suffix_2]...``,
    and a group's "prompt" segment is its suffix (columns ``L0..P-1``).
    ``info`` then also holds ``L0``, ``prefix_len`` (packed rows) and
    ``prefix_cols``.
    """
    ids = np.asarray(input_ids)
    pos = np.asarray(position_ids)
    B, S = ids.shape
    P = S - int(response_length)
    if use_unpad:
        if attention_mask is None:
            raise ValueError("use_unpad needs attention_mask")
        keep = np.asarray(attention_mask) != 0
    else:
        keep = np.ones((B, S), dtype=bool)

    src: list[int] = []
    seg_start: list[int] = []
    G = len(prompt_groups)
    prompt_off = np.zeros(G, np.int64)
    prompt_len = np.zeros(G, np.int64)
    rep = np.zeros(G, np.int64)
    group_of = np.full(B, -1, np.int64)
    resp_off = np.zeros(B, np.int64)
    resp_len = np.zeros(B, np.int64)
    prompt_cols = [None] * B
    resp_cols = [None] * B
    L0 = int(prefix_len)
    if not 0 <= L0 <= P:
        raise ValueError("prefix_len must lie in [0, P]")
    r0 = prompt_groups[0][0] if len(prompt_groups) else 0
    prefix_cols = np.flatnonzero(keep[r0, :L0]) if L0 else np.zeros(0, np.int64)
    src.extend(int(r0 * S + t) for t in prefix_cols)
    seg_start.extend([0] * len(prefix_cols))
    for g, members in enumerate(prompt_groups):
        r = members[0]
        rep[g] = r
        cols = L0 + np.flatnonzero(keep[r, L0:P])
        prompt_off[g] = len(src)
        prompt_len[g] = len(cols)
        src.extend(int(r * S + t) for t in cols)
        seg_start.extend([int(prompt_off[g])] * len(cols))
        for b in members:
            group_of[b] = g
            prompt_cols[b] = cols
            rcols = P + np.flatnonzero(keep[b, P:])
            resp_off[b] = len(src)
            resp_len[b] = len(rcols)
            resp_cols[b] = rcols
            src.extend(int(b * S + t) for t in rcols)
            seg_start.extend([int(resp_off[b])] * len(rcols))
    src_a = np.asarray(src, dtype=np.int64)
    T = len(src_a)
    dst = np.full(B * S, -1, np.int64)
    for b in range(B):
        g = group_of[b]
        dst[b * S + prefix_cols] = np.arange(len(prefix_cols))
        dst[b * S + prompt_cols[b]] = prompt_off[g] + np.arange(prompt_len[g])
        dst[b * S + resp_cols[b]] = resp_off[b] + np.arange(resp_len[b])
    flat_ids = ids.reshape(-1)
    flat_pos = pos.reshape(-1)
    dedup_ids = flat_ids[src_a].reshape(1, T)
    dedup_pos = flat_pos[src_a].reshape(1, T)
    info = dict(B=B, S=S, P=P, G=G, T=T, groups=[list(m) for m in prompt_groups],
                rep=rep, group_of=group_of, prompt_off=prompt_off, prompt_len=prompt_len,
                resp_off=resp_off, resp_len=resp_len, prompt_cols=prompt_cols,
                resp_cols=resp_cols, src=src_a, dst=dst,
                seg_start=np.asarray(seg_start, dtype=np.int64),
                L0=L0, prefix_len=len(prefix_cols), prefix_cols=prefix_cols)
    return dedup_ids, dedup_pos, info


def reconstruct_sequences(dedup_hidden, info):
    """How Prompt Deduplication Works -- Reconstructing Original Batch; Phase 3.

    For each output sample copy its unique prompt, then its own response
    tokens, to the columns they came from; every other position is 0.
    Accepts ``[1, T, H]`` or ``[T, H]``; returns ``[B, S, H]``.
    """
    x = np.asarray(dedup_hidden)
    if x.ndim == 3:
        x = x[0]
    B, S = info["B"], info["S"]
    out = np.zeros((B, S) + x.shape[1:], dtype=x.dtype)
    lp = info.get("prefix_len", 0)
    for b in range(B):
        g = info["group_of"][b]
        if lp:
            out[b, info["prefix_cols"]] = x[:lp]
        po, pl = info["prompt_off"][g], info["prompt_len"][g]
        out[b, info["prompt_cols"][b]] = x[po:po + pl]
        ro, rl = info["resp_off"][b], info["resp_len"][b]
        out[b, info["resp_cols"][b]] = x[ro:ro + rl]
    return out


def pack_rows(rows, info):
    """The deduplicated layout applied to per-token rows ``[B, S, W] -> [T, W]``.

    Packed row ``j`` is the row of the token it was made from
    (Creating Deduplicated Batch: each unique prompt once, then its responses).
    """
    x = np.asarray(rows)
    B, S = info["B"], info["S"]
    flat = x.reshape((B * S,) + x.shape[2:])
    return flat[info["src"]]


def reconstruct_backward(dout, info):
    """How Prompt Deduplication Works -- Correctness & Gradients: the gradient
    flows back through the reconstruction.

    ``reconstruct_sequences`` copies packed row ``j`` to every output position
    that reads it, so the gradient of row ``j`` is the sum of the output
    gradients at those positions: a prompt row collects its column from every
    member of the group, a response row its own position; positions that read
    nothing (dropped pads) contribute nothing.  Summed in fp64, samples in
    ascending order.  ``dout [B, S, ...] -> [T, ...]`` (float64).
    """
    x = np.asarray(dout, dtype=np.float64)
    out = np.zeros((info["T"],) + x.shape[2:], dtype=np.float64)
    lp = info.get("prefix_len", 0)
    for b in range(info["B"]):
        g = info["group_of"][b]
        if lp:
            out[:lp] += x[b, info["prefix_cols"]]
        po, pl = info["prompt_off"][g], info["prompt_len"][g]
        out[po:po + pl] += x[b, info["prompt_cols"][b]]
        ro, rl = info["resp_off"][b], info["resp_len"][b]
        out[ro:ro + rl] += x[b, info["resp_cols"][b]]
    return out


def pack_rows_backward(dpacked, info):
    """Correctness & Gradients -- the gradient flows back through the
    deduplication.

    Packed row ``j`` was copied from exactly one position, ``src[j]``, so its
    gradient goes back there; every other position (the prompt columns of the
    members whose copy was not kept, dropped pads) receives 0.
    ``dpacked [T, ...] -> [B, S, ...]`` in the input's dtype.
    """
    x = np.asarray(dpacked)
    B, S = info["B"], info["S"]
    out = np.zeros((B * S,) + x.shape[1:], dtype=x.dtype)
    out[info["src"]] = x
    return out.reshape((B, S) + x.shape[1:])


def attention_mask_to_flash_attn_params(mask):
    """Flash Attention Integration: a ``[total_q, total_kv]`` block-diagonal
    attention mask -> variable-length parameters ``cu_seqlens_q``,
    ``cu_seqlens_k``, ``max_seqlen_q``, ``max_seqlen_k``.

    Readings: block ``i`` owns query rows ``[cu_q[i], cu_q[i+1])`` and key
    columns ``[cu_k[i], cu_k[i+1])``.  A row's block is named by its first
    visible key; a row that sees no key belongs to the block of the next row
    that sees one (bottom-right aligned causal blocks with more queries than
    keys start with such rows), trailing ones to the last block.  The last
    key boundary is one past the last visible key.  ``mismatched_rows``
    counts rows whose visible keys leave their block's range (0 for a
    block-diagonal mask).
    """
    m = np.asarray(mask) != 0
    Tq = m.shape[0]
    first, last = [], []
    for r in range(Tq):
        nz = np.flatnonzero(m[r])
        first.append(int(nz[0]) if len(nz) else None)
        last.append(int(nz[-1]) + 1 if len(nz) else None)
    owner = [None] * Tq          # first visible key of the row's block
    nxt = None
    for r in range(Tq - 1, -1, -1):
        if first[r] is not None:
            nxt = first[r]
        owner[r] = nxt
    cu_q, cu_k = [], []
    for r in range(Tq):
        if owner[r] is not None and (not cu_k or owner[r] != cu_k[-1]):
            cu_q.append(r)
            cu_k.append(owner[r])
    n = len(cu_q)
    if n == 0:
        return dict(cu_seqlens_q=np.zeros(1, np.int32), cu_seqlens_k=np.zeros(1, np.int32), max_seqlen_q=0,
                    max_seqlen_k=0, num_seqs=0, mismatched_rows=0)
    cu_q.append(Tq)
    cu_k.append(max(x for x in last if x is not None))
    bad = 0
    for i in range(n):
        for r in range(cu_q[i], cu_q[i + 1]):
            if first[r] is not None and (first[r] != cu_k[i] or last[r] > cu_k[i + 1]):
                bad += 1
    cu_q = np.asarray(cu_q, np.int32)
    cu_k = np.asarray(cu_k, np.int32)
    return dict(cu_seqlens_q=cu_q, cu_seqlens_k=cu_k, max_seqlen_q=int(np.diff(cu_q).max()),
                max_seqlen_k=int(np.diff(cu_k).max()), num_seqs=n, mismatched_rows=bad)


def varlen_params(info):
    """Variable-length parameters of the two attention calls of Phase 2 (Split
    Attention Optimization) for a packed batch:

    * prompt-to-prompt: ``cu_seqlens`` over the unique prompts (queries and
      keys alike), ``[G + 1]``;
    * response-to-full: queries are each sample's response rows
      (``cu_seqlens_q [B + 1]``), keys each sample's prompt followed by its
      response (``cu_seqlens_k [B + 1]``, the full batch laid out sample by
      sample).
    """
    pl = np.asarray(info["prompt_len"], np.int64)
    rl = np.asarray(info["resp_len"], np.int64)
    gof = np.asarray(info["group_of"], np.int64)
    kl = pl[gof] + rl
    cu = lambda a: np.concatenate([[0], np.cumsum(a)]).astype(np.int32)
    return dict(cu_seqlens_prompt=cu(pl), max_seqlen_prompt=int(pl.max(initial=0)),
                cu_seqlens_q=cu(rl), cu_seqlens_k=cu(kl), max_seqlen_q=int(rl.max(initial=0)),
                max_seqlen_k=int(kl.max(initial=0)))


def sample_rows(info, b):
    """Packed rows of sample ``b``'s own sequence: the shared prefix (if any), its group's
    prompt, then its response (ascending in the packed layout).

    This is the non-deduplicated ``[Prompt][Response]`` sample expressed as
    packed row indices (Phase 1 diagram: every sample is its prompt followed
    by its response).
    """
    g = info["group_of"][b]
    po, pl = info["prompt_off"][g], info["prompt_len"][g]
    ro, rl = info["resp_off"][b], info["resp_len"][b]
    lp = info.get("prefix_len", 0)
    return np.concatenate([np.arange(lp), np.arange(po, po + pl), np.arange(ro, ro + rl)]).astype(np.int64)


def redundancy_counts(info):
    """Performance Benchmarks -- Redundancy Analysis: total vs unique tokens.

    ``total`` counts every sample's prompt and response tokens (the
    non-deduplicated batch), ``unique`` counts the packed tokens, and
    ``redundancy = 1 - unique / total``.
    """
    total = int(sum(info.get("prefix_len", 0) + info["prompt_len"][info["group_of"][b]] + info["resp_len"][b]
                    for b in range(info["B"])))
    unique = int(info["T"])
    return total, unique, (1.0 - unique / total) if total else 0.0
