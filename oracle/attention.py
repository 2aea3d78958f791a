"""Oracle: split attention forward and backward, as NON-deduplicated attention.

Test infrastructure only; see the package docstring.

What it computes (How Prompt Deduplication Works -- Phase 2, Split Attention
Optimization; Correctness & Gradients): in the packed batch every unique
prompt attends causally to itself once, and each response attends to all of
its prompt's keys plus its own causal prefix.  The pages require this to equal
the ordinary, non-deduplicated computation ("Performance Benchmarks" --
Testing Correctness and Performance: outputs and gradients are validated
against a non-deduplicated reference).  So the oracle runs plain causal
softmax attention separately on every sample's own ``[prompt][response]``
sequence (gathered from the packed rows), in fp64, and maps the results
back onto the packed rows:

* forward -- each packed row takes the output of the sample it was packed
  from (response rows: their sample; prompt rows: the group's first member;
  a shared prefix: the first sample), and every other sample's output for
  that row is asserted equal to it (the deduplication invariant);
* backward -- the gradient w.r.t. the packed tensors of
  ``O_packed = assemble(attention of every sample)``: each sample's ``dO``
  is the packed ``dO`` on the rows packed from it and 0 on the shared rows
  packed from another sample (their outputs were taken from that sample
  only); per-sample textbook
  gradients are scatter-added onto the packed rows, so prompt keys and
  values collect the gradient of every response that reads them.

Readings (the pages leave these open): softmax scale ``1/sqrt(head_dim)``
unless given; query head ``h`` reads kv head ``h // (Hq // Hkv)``; a
response row ``i`` sees every prompt key and its own keys ``0..i`` (never a
sibling response); LSE is the natural log of the softmax denominator,
``[Hq, T]``.

Softmax rows are processed in blocks of query rows, each block over the keys
``[0, block_end)``: the causal extent itself, no reordering of the sums
beyond what a matrix product does.
"""
from __future__ import annotations

import math

import numpy as np

from .dedup import sample_rows

_BLOCK = 512


def _kv_head(h, Hq, Hkv):
    return h // (Hq // Hkv)


def _causal_block(Qs, Ks, Vs, i0, i1, scale, dOs=None):
    """Plain causal softmax attention for query rows ``[i0, i1)`` of one sequence.

    Query ``i`` sees keys ``0..i``.  Returns ``(p, o, lse)`` and, when
    ``dOs`` is given, also ``dS`` (the softmax-input gradient, before the
    scale), following the textbook derivation:
    ``D = rowsum(dO * O)``, ``dP = dO V^T``, ``dS = P * (dP - D)``.
    """
    s = scale * (Qs[i0:i1] @ Ks[:i1].T)
    future = np.arange(i1)[None, :] > np.arange(i0, i1)[:, None]
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
    D = (dO * o).sum(axis=1, keepdims=True)
    dP = dO @ Vs[:i1].T
    dS = p * (dP - D)
    return p, o, lse, dS


def _prep(q, k, v, scale):
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    return q, k, v, T, Hq, Hkv, d, float(scale)


def _sample_seq(info, b, valid):
    """Packed rows of sample ``b``'s sequence (ascending).

    With ``valid`` (bool per packed row; Working with Packed/Unpacked
    Sequences, padded format with an attention mask) the pads are left out of
    the sequence: they are no sample's keys or queries, so their outputs and
    gradients stay 0.
    """
    idx = sample_rows(info, b)
    if valid is None:
        return idx
    return idx[np.asarray(valid, dtype=bool)[idx]]


def _owner(info):
    """The sample each packed row was packed from: its output is that
    sample's, and only that sample carries its ``dO`` in the backward."""
    return np.asarray(info["src"], dtype=np.int64) // int(info["S"])


def _members_rep_first(info, g):
    r = int(info["rep"][g])
    return [r] + [b for b in info["groups"][g] if b != r]


def split_attention_forward(q, k, v, info, scale=None, heads=None, valid=None):
    """Split attention forward over packed ``q [T,Hq,d]``, ``k, v [T,Hkv,d]``.

    Returns ``o [T,Hq,d]`` and ``lse [Hq,T]`` (fp64).  ``heads`` restricts
    the work to some query heads (others are left 0).  ``valid`` (bool [T])
    marks pads kept in a padded-format batch: they take no part (output 0).
    """
    q, k, v, T, Hq, Hkv, d, scale = _prep(q, k, v, scale)
    heads = range(Hq) if heads is None else heads
    o = np.zeros((T, Hq, d))
    lse = np.zeros((Hq, T))
    owner = _owner(info)
    for g in range(info["G"]):
        # a group's first member first: it owns the group's prompt rows (and
        # the first group's first member owns a shared prefix)
        for b in _members_rep_first(info, g):
            idx = _sample_seq(info, b, valid)
            L = len(idx)
            mine = owner[idx] == b
            for h in heads:
                j = _kv_head(h, Hq, Hkv)
                Qs, Ks, Vs = q[idx, h], k[idx, j], v[idx, j]
                Ob = np.zeros((L, d))
                Lb = np.zeros(L)
                for i0 in range(0, L, _BLOCK):
                    i1 = min(L, i0 + _BLOCK)
                    _, Ob[i0:i1], Lb[i0:i1], _ = _causal_block(Qs, Ks, Vs, i0, i1, scale)
                o[idx[mine], h] = Ob[mine]
                lse[h, idx[mine]] = Lb[mine]
                # every copy of a shared row must produce the same output
                err = np.max(np.abs(o[idx[~mine], h] - Ob[~mine]), initial=0.0)
                assert err <= 1e-12, f"copies of a shared row disagree by {err}"
    return o, lse


def split_attention_backward(q, k, v, dout, info, scale=None, heads=None, valid=None):
    """Gradients ``(dq, dk, dv)`` of the packed split-attention output.

    Per sample: textbook causal-attention backward with that sample's
    ``dO`` (see the module docstring), then scatter-add onto packed rows;
    query heads sharing a kv head add into it.  ``heads`` restricts the work
    to some query heads (the others contribute nothing).  ``valid`` as in
    the forward: pads get zero gradients.
    """
    q, k, v, T, Hq, Hkv, d, scale = _prep(q, k, v, scale)
    dout = np.asarray(dout, dtype=np.float64)
    heads = range(Hq) if heads is None else heads
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    owner = _owner(info)
    for g in range(info["G"]):
        for b in _members_rep_first(info, g):
            idx = _sample_seq(info, b, valid)
            L = len(idx)
            for h in heads:
                j = _kv_head(h, Hq, Hkv)
                Qs, Ks, Vs = q[idx, h], k[idx, j], v[idx, j]
                dOs = dout[idx, h].copy()
                dOs[owner[idx] != b] = 0.0
                dQb = np.zeros((L, d))
                dKb = np.zeros((L, d))
                dVb = np.zeros((L, d))
                for i0 in range(0, L, _BLOCK):
                    i1 = min(L, i0 + _BLOCK)
                    p, _, _, dS = _causal_block(Qs, Ks, Vs, i0, i1, scale, dOs)
                    dVb[:i1] += p.T @ dOs[i0:i1]
                    dQb[i0:i1] = scale * (dS @ Ks[:i1])
                    dKb[:i1] += scale * (dS.T @ Qs[i0:i1])
                dq[idx, h] += dQb
                dk[idx, j] += dKb
                dv[idx, j] += dVb
    return dq, dk, dv


# ---------------------------------------------------------------------------
# Row-sampled versions for full-size checks: the same definition, evaluated
# only where asked.  A packed row is located in the sequence of the sample
# that owns it (the group's first member for prompt rows).
# ---------------------------------------------------------------------------

def _locate(info, j):
    """(owning sample, position of packed row ``j`` in that sample's sequence)."""
    b = int(info["src"][j]) // int(info["S"])
    idx = sample_rows(info, b)
    return b, int(np.searchsorted(idx, j))


def forward_rows(q, k, v, info, rows, heads, scale=None):
    """Forward output and LSE for the listed packed rows and query heads.

    Returns ``o [len(rows), len(heads), d]``, ``lse [len(rows), len(heads)]``.
    """
    q, k, v, T, Hq, Hkv, d, scale = _prep(q, k, v, scale)
    o = np.zeros((len(rows), len(heads), d))
    lse = np.zeros((len(rows), len(heads)))
    for a, j in enumerate(rows):
        b, i = _locate(info, int(j))
        idx = sample_rows(info, b)
        for c, h in enumerate(heads):
            kv = _kv_head(h, Hq, Hkv)
            _, ob, lb, _ = _causal_block(q[idx, h], k[idx, kv], v[idx, kv], i, i + 1, scale)
            o[a, c] = ob[0]
            lse[a, c] = lb[0]
    return o, lse


def dq_rows(q, k, v, dout, info, rows, heads, scale=None):
    """``dq`` for the listed packed rows and query heads (``[len(rows), len(heads), d]``).

    Only the owning sample has a non-zero ``dO`` on a row (shared rows: the
    sample they were packed from), so the row's gradient is that sample's.
    """
    q, k, v, T, Hq, Hkv, d, scale = _prep(q, k, v, scale)
    dout = np.asarray(dout, dtype=np.float64)
    out = np.zeros((len(rows), len(heads), d))
    for a, j in enumerate(rows):
        b, i = _locate(info, int(j))
        idx = sample_rows(info, b)
        owner = _owner(info)[idx]
        for c, h in enumerate(heads):
            kv = _kv_head(h, Hq, Hkv)
            Ks = k[idx, kv]
            _, _, _, dS = _causal_block(q[idx, h], Ks, v[idx, kv], i, i + 1, scale,
                                        np.where((owner == b)[:, None], dout[idx, h], 0.0))
            out[a, c] = scale * (dS @ Ks[:i + 1])[0]
    return out


def dkdv_rows(q, k, v, dout, info, keys, kv_heads, scale=None):
    """``dk, dv`` for the listed packed key rows and kv heads.

    Sums, over every sample whose sequence contains the key and every query
    position at or after it with a non-zero ``dO``, over the query heads of
    the kv head: ``dv += P dO`` and ``dk += scale * dS q``.  The keys a
    sample contains share one pass over its query rows from the earliest of
    them: a row before a key has ``P = 0`` and ``dS = 0`` there (the key is in
    its future), and a row without ``dO`` has ``dO = 0`` and ``dS = 0``, so
    such rows add exact zeros.
    """
    q, k, v, T, Hq, Hkv, d, scale = _prep(q, k, v, scale)
    dout = np.asarray(dout, dtype=np.float64)
    ratio = Hq // Hkv
    keys = np.asarray([int(x) for x in keys], dtype=np.int64)
    dk = np.zeros((len(keys), len(kv_heads), d))
    dv = np.zeros((len(keys), len(kv_heads), d))
    owner_all = _owner(info)
    for b in range(info["B"]):
        idx = sample_rows(info, b)
        L = len(idx)
        if L == 0:
            continue
        pos = np.searchsorted(idx, keys)
        present = (pos < L) & (idx[np.minimum(pos, L - 1)] == keys)
        if not present.any():
            continue                           # no listed key is in this sample's sequence
        sel = np.flatnonzero(present)
        kpos = pos[sel]
        own = owner_all[idx] == b
        later = np.flatnonzero(own[kpos.min():])
        if not len(later):
            continue                           # no query of this sample that sees a key carries dO
        first = int(kpos.min()) + int(later[0])
        for c, j in enumerate(kv_heads):
            for h in range(j * ratio, (j + 1) * ratio):
                Qs, Ks, Vs = q[idx, h], k[idx, j], v[idx, j]
                dOs = np.where(own[:, None], dout[idx, h], 0.0)
                for i0 in range(first, L, _BLOCK):
                    i1 = min(L, i0 + _BLOCK)
                    p, _, _, dS = _causal_block(Qs, Ks, Vs, i0, i1, scale, dOs)
                    seen = kpos < i1               # keys at or after i1 are in every row's future here
                    ks, kp = sel[seen], kpos[seen]
                    dv[ks, c] += p[:, kp].T @ dOs[i0:i1]
                    dk[ks, c] += scale * (dS[:, kp].T @ Qs[i0:i1])
    return dk, dv


def attended_pairs(info):
    """Number of (query, key) pairs split attention evaluates on the packed batch.

    Prompt ``g``: ``Pl (Pl + 1) / 2`` causal pairs once; response ``b``:
    ``Rl * Pl`` prompt keys plus ``Rl (Rl + 1) / 2`` causal own pairs.  With
    a shared prefix of ``Lp`` rows: ``Lp (Lp + 1) / 2`` once, and every
    prompt and response row also sees the ``Lp`` prefix keys.
    Also returns the non-deduplicated count, ``sum_b L_b (L_b + 1) / 2``.
    """
    lp = int(info.get("prefix_len", 0))
    dedup = lp * (lp + 1) // 2
    plain = 0
    for g in range(info["G"]):
        pl = int(info["prompt_len"][g])
        dedup += pl * lp + pl * (pl + 1) // 2
        for b in info["groups"][g]:
            rl = int(info["resp_len"][b])
            dedup += rl * (lp + pl) + rl * (rl + 1) // 2
            L = lp + pl + rl
            plain += L * (L + 1) // 2
    return dedup, plain
