"""Python binding of libspd: argument marshalling over the C ABI, nothing else.

Every step of the path runs in the HIP library; this module only allocates
device buffers with PyTorch, passes pointers and the current HIP stream, and
reads back the two sizes the pages' API returns on the host (the number of
groups and the packed length).

Names follow the C ABI (``group``, ``pack``, ``pack_rows``, ``split_attn_fwd``,
``split_attn_bwd``, ``reconstruct``) and, as aliases, the pages' calls
("How Prompt Deduplication Works" -- Core Algorithm: ZoRRoTrain Class):
``find_prompt_groups``, ``create_deduplicated_batch``, ``reconstruct_sequences``.
"""
from __future__ import annotations

import ctypes
import math
from typing import Optional

import torch

from ._lib import SPD_BF16, SPD_F32, SpdAttnDesc, SpdPlan, check, lib

_PLAN_FIELDS = ("group_of", "grp_off", "grp_idx", "rep", "prompt_off", "prompt_len", "resp_off", "resp_len",
                "src", "dst", "seg_start", "counts")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need_cuda(t: torch.Tensor, name: str):
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


class Plan:
    """Device arrays of a deduplication plan (``spd_plan``), owned here.

    Capacities depend only on ``B`` and ``S``.  ``G`` and ``T`` are host copies
    read back after grouping / packing.
    """

    def __init__(self, B: int, S: int, P: int, device):
        self.B, self.S, self.P = int(B), int(S), int(P)
        self.device = torch.device(device)
        i32 = dict(dtype=torch.int32, device=self.device)
        n = self.B * self.S
        self.group_of = torch.empty(self.B, **i32)
        self.grp_off = torch.empty(self.B + 1, **i32)
        self.grp_idx = torch.empty(self.B, **i32)
        self.rep = torch.empty(self.B, **i32)
        self.prompt_off = torch.empty(self.B, **i32)
        self.prompt_len = torch.empty(self.B, **i32)
        self.resp_off = torch.empty(self.B, **i32)
        self.resp_len = torch.empty(self.B, **i32)
        self.src = torch.empty(n, **i32)
        self.dst = torch.empty(n, **i32)
        self.seg_start = torch.empty(n, **i32)
        self.counts = torch.empty(8, **i32)      # every entry the calls read is written by an earlier call
        self.G: Optional[int] = None
        self.T: Optional[int] = None
        self.use_unpad = False
        self.kept_pads = 0
        self.L0 = 0
        self.prefix_len = 0
        self._c = SpdPlan(self.B, self.S, self.P, *[t.data_ptr() for t in
                                                    (getattr(self, f) for f in _PLAN_FIELDS)])

    @property
    def c(self) -> SpdPlan:
        return self._c

    def read_counts(self):
        c = self.counts.cpu().tolist()
        self.G, self.T = int(c[0]), int(c[1])
        self.kept_pads = int(c[3])
        self.L0, self.prefix_len = int(c[4]), int(c[5])
        return self.G, self.T


class PromptGroups(list):
    """``prompt_groups`` as the pages return it (a list of lists of sample
    indices), carrying the device plan it was read from."""

    def __init__(self, groups, plan: Plan):
        super().__init__(groups)
        self.plan = plan


class ReconstructionInfo(dict):
    """Reconstruction metadata: the plan's device arrays by name, plus sizes."""

    def __init__(self, plan: Plan):
        super().__init__({f: getattr(plan, f) for f in _PLAN_FIELDS})
        self.update(B=plan.B, S=plan.S, P=plan.P, G=plan.G, T=plan.T, use_unpad=plan.use_unpad,
                    kept_pads=plan.kept_pads, L0=plan.L0, prefix_len=plan.prefix_len)
        self.plan = plan
        # Padded format with pads in the packed sequence: the same batch packed without them (same groups).
        # Attention runs there, pads taking no part (Working with Packed/Unpacked Sequences).
        self.unpadded: Optional["ReconstructionInfo"] = None


# ---------------------------------------------------------------------------- group / pack


def group(input_ids: torch.Tensor, response_length: int, return_lists: bool = True):
    """spd_group: samples with identical prompt ids (``input_ids [B, S]`` int64).

    Returns ``(prompt_groups, unique_prompts [G, P])``.  With
    ``return_lists=False`` nothing is read back to the host (no
    synchronisation): ``prompt_groups`` is an empty ``PromptGroups`` carrying
    the plan, and ``unique_prompts`` is the ``[B, P]`` buffer whose first G
    rows hold the unique prompts (G is ``info["G"]`` once packed).
    """
    _need_cuda(input_ids, "input_ids")
    if input_ids.dtype != torch.int64 or input_ids.dim() != 2:
        raise ValueError("input_ids must be int64 [batch, seq_len]")
    B, S = input_ids.shape
    P = S - int(response_length)
    plan = Plan(B, S, P, input_ids.device)
    ws = torch.empty(lib.spd_group_workspace_bytes(B, S), dtype=torch.uint8, device=input_ids.device)
    uniq = torch.empty((B, P), dtype=torch.int64, device=input_ids.device)
    check("spd_group", lib.spd_group(_ptr(input_ids), B, S, int(response_length), ctypes.byref(plan.c),
                                     _ptr(uniq) if P > 0 else None, _ptr(ws), ws.numel(), _stream(input_ids.device)))
    if not return_lists:
        return PromptGroups([], plan), uniq
    plan.G = int(plan.counts[0].item())
    off = plan.grp_off[:plan.G + 1].cpu().tolist()
    idx = plan.grp_idx.cpu().tolist()
    groups = [idx[off[g]:off[g + 1]] for g in range(plan.G)]
    return PromptGroups(groups, plan), uniq[:plan.G]


def pack(input_ids: torch.Tensor, position_ids: torch.Tensor, response_length: int, prompt_groups: PromptGroups,
         unique_prompts: Optional[torch.Tensor] = None, attention_mask: Optional[torch.Tensor] = None,
         use_unpad: bool = False, share_prefix: bool = False):
    """spd_pack: the deduplicated ``[1, T]`` ids and positions plus reconstruction info.

    ``share_prefix`` (spd_share_prefix) also packs the batch's shared prompt prefix once, ahead of all groups."""
    if not isinstance(prompt_groups, PromptGroups):
        raise TypeError("prompt_groups must come from group()/find_prompt_groups() (it carries the device plan)")
    plan = prompt_groups.plan
    _need_cuda(input_ids, "input_ids")
    _need_cuda(position_ids, "position_ids")
    if tuple(input_ids.shape) != (plan.B, plan.S) or tuple(position_ids.shape) != (plan.B, plan.S):
        raise ValueError("input_ids / position_ids shape does not match the grouping")
    if plan.S - int(response_length) != plan.P:
        raise ValueError("response_length differs from the one used for grouping")
    if position_ids.dtype != torch.int64:
        raise ValueError("position_ids must be int64")
    mask_ptr, esz = None, 1
    if attention_mask is not None:
        _need_cuda(attention_mask, "attention_mask")
        if tuple(attention_mask.shape) != (plan.B, plan.S):
            raise ValueError("attention_mask shape must be [batch, seq_len]")
        esz = attention_mask.element_size()
        if attention_mask.dtype not in (torch.bool, torch.int8, torch.uint8, torch.int32, torch.int64):
            raise ValueError("attention_mask must be bool or an integer type")
        mask_ptr = _ptr(attention_mask)
    if use_unpad and attention_mask is None:
        raise ValueError("use_unpad=True needs attention_mask")
    dev = input_ids.device
    n = plan.B * plan.S
    if share_prefix:
        check("spd_share_prefix", lib.spd_share_prefix(_ptr(input_ids), plan.B, plan.S, int(response_length),
                                                       ctypes.byref(plan.c), _stream(dev)))
    dids = torch.empty(n, dtype=torch.int64, device=dev)
    dpos = torch.empty(n, dtype=torch.int64, device=dev)
    ws = torch.empty(lib.spd_pack_workspace_bytes(plan.B, plan.S), dtype=torch.uint8, device=dev)
    check("spd_pack", lib.spd_pack(_ptr(input_ids), _ptr(position_ids), mask_ptr, esz, int(bool(use_unpad)),
                                   ctypes.byref(plan.c), _ptr(dids), _ptr(dpos), _ptr(ws), ws.numel(), _stream(dev)))
    plan.use_unpad = bool(use_unpad)
    plan.read_counts()
    T = plan.T
    if plan.kept_pads == 0:
        plan.c.padded_with_mask = 0     # a mask in padded mode, but no pad among the packed rows
    info = ReconstructionInfo(plan)
    if not use_unpad and plan.kept_pads > 0:
        twin = Plan(plan.B, plan.S, plan.P, dev)
        for f in ("group_of", "grp_off", "grp_idx", "rep"):
            getattr(twin, f).copy_(getattr(plan, f))
        twin.counts[:1].copy_(plan.counts[:1])
        twin.counts[4:5].copy_(plan.counts[4:5])       # the same shared prefix, if any
        tids = torch.empty(n, dtype=torch.int64, device=dev)
        tpos = torch.empty(n, dtype=torch.int64, device=dev)
        check("spd_pack", lib.spd_pack(_ptr(input_ids), _ptr(position_ids), mask_ptr, esz, 1, ctypes.byref(twin.c),
                                       _ptr(tids), _ptr(tpos), _ptr(ws), ws.numel(), _stream(dev)))
        twin.use_unpad = True
        twin.read_counts()
        info.unpadded = ReconstructionInfo(twin)
    return dids[:T].view(1, T), dpos[:T].view(1, T), info


def _row_bytes(t: torch.Tensor, lead: int) -> int:
    """Bytes of one row of ``t`` after its first ``lead`` dimensions (from the shape, so empty tensors work)."""
    return math.prod(t.shape[lead:]) * t.element_size()


def _pack_rows(rows: torch.Tensor, info: ReconstructionInfo) -> torch.Tensor:
    plan = info.plan
    _need_cuda(rows, "rows")
    if tuple(rows.shape[:2]) != (plan.B, plan.S):
        raise ValueError("rows must be [batch, seq_len, ...]")
    tail = tuple(rows.shape[2:])
    row_bytes = _row_bytes(rows, 2)
    out = torch.empty((plan.T,) + tail, dtype=rows.dtype, device=rows.device)
    check("spd_pack_rows", lib.spd_pack_rows(ctypes.byref(plan.c), plan.T, _ptr(rows), row_bytes, _ptr(out),
                                             _stream(rows.device)))
    return out


def pack_rows_bwd(dpacked: torch.Tensor, info: ReconstructionInfo) -> torch.Tensor:
    """spd_pack_rows_bwd: ``[T, ...] -> [B, S, ...]``, each packed row's gradient back at its source cell,
    zeros elsewhere."""
    plan = info.plan
    _need_cuda(dpacked, "dpacked")
    if dpacked.shape[0] != plan.T:
        raise ValueError(f"dpacked has {dpacked.shape[0]} rows, the plan has T = {plan.T}")
    tail = tuple(dpacked.shape[1:])
    row_bytes = _row_bytes(dpacked, 1)
    out = torch.empty((plan.B, plan.S) + tail, dtype=dpacked.dtype, device=dpacked.device)
    check("spd_pack_rows_bwd", lib.spd_pack_rows_bwd(ctypes.byref(plan.c), plan.T, _ptr(dpacked), row_bytes,
                                                     _ptr(out), _stream(dpacked.device)))
    return out


class PackRows(torch.autograd.Function):
    """pack_rows with its backward (``spd_pack_rows_bwd``)."""

    @staticmethod
    def forward(ctx, rows, info):
        ctx.info = info
        return _pack_rows(rows, info)

    @staticmethod
    def backward(ctx, g):
        return pack_rows_bwd(g.contiguous(), ctx.info), None


def pack_rows(rows: torch.Tensor, info: ReconstructionInfo) -> torch.Tensor:
    """spd_pack_rows: ``rows [B, S, ...] -> [T, ...]`` with the plan's packing (differentiable)."""
    return PackRows.apply(rows, info)


def _reconstruct(x: torch.Tensor, info: ReconstructionInfo) -> torch.Tensor:
    plan = info.plan
    _need_cuda(x, "dedup_hidden")
    if x.shape[0] != plan.T:
        raise ValueError(f"dedup_hidden has {x.shape[0]} rows, the plan has T = {plan.T}")
    tail = tuple(x.shape[1:])
    row_bytes = _row_bytes(x, 1)
    out = torch.empty((plan.B, plan.S) + tail, dtype=x.dtype, device=x.device)
    check("spd_reconstruct", lib.spd_reconstruct(ctypes.byref(plan.c), plan.T, _ptr(x), row_bytes, _ptr(out),
                                                 _stream(x.device)))
    return out


def reconstruct_bwd(dout: torch.Tensor, info: ReconstructionInfo) -> torch.Tensor:
    """spd_reconstruct_bwd: ``dout [B, S, ...] -> [T, ...]``; a packed prompt row receives the sum of its
    group members' gradients (fp32 accumulation, one rounding).  bf16 or fp32."""
    plan = info.plan
    _need_cuda(dout, "dout")
    if tuple(dout.shape[:2]) != (plan.B, plan.S):
        raise ValueError("dout must be [batch, seq_len, ...]")
    if dout.dtype == torch.bfloat16:
        dt = SPD_BF16
    elif dout.dtype == torch.float32:
        dt = SPD_F32
    else:
        raise TypeError("reconstruct_bwd supports bfloat16 and float32 gradients")
    tail = tuple(dout.shape[2:])
    row_bytes = _row_bytes(dout, 2)
    out = torch.empty((plan.T,) + tail, dtype=dout.dtype, device=dout.device)
    check("spd_reconstruct_bwd", lib.spd_reconstruct_bwd(ctypes.byref(plan.c), plan.T, _ptr(dout), row_bytes, dt,
                                                         _ptr(out), _stream(dout.device)))
    return out


class Reconstruct(torch.autograd.Function):
    """reconstruct with its backward (``spd_reconstruct_bwd``)."""

    @staticmethod
    def forward(ctx, x, info):
        ctx.info = info
        return _reconstruct(x, info)

    @staticmethod
    def backward(ctx, g):
        return reconstruct_bwd(g.contiguous(), ctx.info), None


def reconstruct(dedup_hidden: torch.Tensor, info: ReconstructionInfo) -> torch.Tensor:
    """spd_reconstruct: ``[1, T, ...]`` or ``[T, ...]`` -> ``[B, S, ...]`` (differentiable)."""
    plan = info.plan
    x = dedup_hidden
    if x.dim() >= 3 and x.shape[0] == 1 and x.shape[1] == plan.T:
        x = x[0]
    return Reconstruct.apply(x, info)


def singleton_groups(input_ids: torch.Tensor, response_length: int):
    """spd_group_singletons: every sample its own group (the non-deduplicated batch).

    Returns ``(prompt_groups, prompts [B, P])`` like ``group``."""
    _need_cuda(input_ids, "input_ids")
    if input_ids.dtype != torch.int64 or input_ids.dim() != 2:
        raise ValueError("input_ids must be int64 [batch, seq_len]")
    B, S = input_ids.shape
    P = S - int(response_length)
    plan = Plan(B, S, P, input_ids.device)
    check("spd_group_singletons", lib.spd_group_singletons(B, S, int(response_length), ctypes.byref(plan.c),
                                                           _stream(input_ids.device)))
    plan.G = B
    return PromptGroups([[b] for b in range(B)], plan), input_ids[:, :P]


def create_full_batch(input_ids, position_ids, response_length, attention_mask=None, use_unpad=False):
    """The full (non-deduplicated) batch in packed variable-length form -- every sample's prompt, then its
    response: ``(ids [1, T_full], positions [1, T_full], info)``.  Attention on ``info`` is standard per-sample
    causal attention (Phase 2, Standard QKV Optimization)."""
    groups, prompts = singleton_groups(input_ids, response_length)
    return pack(input_ids, position_ids, response_length, groups, prompts, attention_mask, use_unpad)


def repack_rows(x: torch.Tensor, to_info: ReconstructionInfo, from_info: ReconstructionInfo) -> torch.Tensor:
    """spd_repack_rows: rows of ``from_info``'s packed layout ``[T_from, ...]`` -> ``to_info``'s ``[T_to, ...]``."""
    to, fr = to_info.plan, from_info.plan
    _need_cuda(x, "x")
    if x.shape[0] != fr.T:
        raise ValueError(f"x has {x.shape[0]} rows, the source layout has T = {fr.T}")
    out = torch.empty((to.T,) + tuple(x.shape[1:]), dtype=x.dtype, device=x.device)
    check("spd_repack_rows", lib.spd_repack_rows(ctypes.byref(to.c), to.T, ctypes.byref(fr.c), fr.T, _ptr(x),
                                                 _row_bytes(x, 1), _ptr(out), _stream(x.device)))
    return out


def repack_rows_bwd(dout: torch.Tensor, to_info: ReconstructionInfo, from_info: ReconstructionInfo) -> torch.Tensor:
    """spd_repack_rows_bwd: the transpose of ``repack_rows(., to_info, from_info)``: ``[T_to, ...] -> [T_from, ...]``
    (fp32 accumulation, one rounding; bf16 or fp32)."""
    to, fr = to_info.plan, from_info.plan
    _need_cuda(dout, "dout")
    if dout.shape[0] != to.T:
        raise ValueError(f"dout has {dout.shape[0]} rows, the layout has T = {to.T}")
    if dout.dtype == torch.bfloat16:
        dt = SPD_BF16
    elif dout.dtype == torch.float32:
        dt = SPD_F32
    else:
        raise TypeError("repack_rows_bwd supports bfloat16 and float32 gradients")
    out = torch.empty((fr.T,) + tuple(dout.shape[1:]), dtype=dout.dtype, device=dout.device)
    check("spd_repack_rows_bwd", lib.spd_repack_rows_bwd(ctypes.byref(to.c), to.T, ctypes.byref(fr.c), fr.T,
                                                         _ptr(dout), _row_bytes(dout, 1), dt, _ptr(out),
                                                         _stream(dout.device)))
    return out


# ---------------------------------------------------------------------------- varlen parameters


def attention_mask_to_flash_attn_params(attention_mask: torch.Tensor) -> dict:
    """Flash Attention Integration: block-diagonal ``[total_q, total_kv]`` mask -> ``cu_seqlens_q``,
    ``cu_seqlens_k`` (device int32), ``max_seqlen_q``, ``max_seqlen_k``, plus ``num_seqs`` and
    ``mismatched_rows`` (rows whose visible keys leave their block; 0 for a block-diagonal mask)."""
    _need_cuda(attention_mask, "attention_mask")
    if attention_mask.dim() != 2:
        raise ValueError("attention_mask must be [total_q, total_kv]")
    m = attention_mask.contiguous()
    Tq, Tk = m.shape
    dev = m.device
    cu_q = torch.empty(Tq + 1, dtype=torch.int32, device=dev)
    cu_k = torch.empty(Tq + 1, dtype=torch.int32, device=dev)
    stats = torch.empty(4, dtype=torch.int32, device=dev)
    ws = torch.empty(max(1, lib.spd_mask_varlen_workspace_bytes(Tq)), dtype=torch.uint8, device=dev)
    check("spd_mask_to_varlen", lib.spd_mask_to_varlen(_ptr(m), m.element_size(), Tq, Tk, _ptr(cu_q), _ptr(cu_k),
                                                       _ptr(stats), _ptr(ws), ws.numel(), _stream(dev)))
    n, mq, mk, bad = stats.cpu().tolist()
    return dict(cu_seqlens_q=cu_q[:n + 1], cu_seqlens_k=cu_k[:n + 1], max_seqlen_q=mq, max_seqlen_k=mk,
                num_seqs=n, mismatched_rows=bad)


def flash_attn_params(info: ReconstructionInfo) -> dict:
    """spd_varlen_params: cu_seqlens of the two Phase 2 attention calls for a packed batch --
    ``cu_seqlens_prompt`` (prompt-to-prompt), ``cu_seqlens_q`` / ``cu_seqlens_k`` (response-to-full: each sample's
    response rows against its prompt + response) and the three maxima."""
    plan = info.plan
    dev = plan.device
    cp = torch.empty(plan.B + 1, dtype=torch.int32, device=dev)
    cq = torch.empty(plan.B + 1, dtype=torch.int32, device=dev)
    ck = torch.empty(plan.B + 1, dtype=torch.int32, device=dev)
    mx = torch.empty(3, dtype=torch.int32, device=dev)
    check("spd_varlen_params", lib.spd_varlen_params(ctypes.byref(plan.c), _ptr(cp), _ptr(cq), _ptr(ck), _ptr(mx),
                                                     _stream(dev)))
    m = mx.cpu().tolist()
    return dict(cu_seqlens_prompt=cp[:plan.G + 1], max_seqlen_prompt=m[0], cu_seqlens_q=cq, cu_seqlens_k=ck,
                max_seqlen_q=m[1], max_seqlen_k=m[2])


# ---------------------------------------------------------------------------- attention


def _desc(q: torch.Tensor, k: torch.Tensor, softmax_scale: Optional[float]) -> SpdAttnDesc:
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("q must be [T, Hq, d] and k, v [T, Hkv, d]")
    T, Hq, d = q.shape
    if k.shape[0] != T or k.shape[2] != d:
        raise ValueError("q and k disagree on T or head_dim")
    if q.dtype == torch.bfloat16:
        dt = SPD_BF16
    elif q.dtype == torch.float32:
        dt = SPD_F32
    else:
        raise ValueError("attention tensors must be bfloat16 or float32")
    scale = (1.0 / math.sqrt(d)) if softmax_scale is None else float(softmax_scale)
    return SpdAttnDesc(Hq, k.shape[1], d, dt, scale)


def _attn_ws(desc: SpdAttnDesc, plan: Plan, T: int, device, forward: bool):
    query = lib.spd_attn_fwd_workspace_bytes if forward else lib.spd_attn_workspace_bytes
    n = query(ctypes.byref(desc), plan.B, T)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


def split_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, info: ReconstructionInfo,
                   softmax_scale: Optional[float] = None):
    """spd_split_attn_fwd: packed ``q [T,Hq,d]``, ``k, v [T,Hkv,d]`` -> ``(o, lse [Hq,T])``.

    For a padded-format plan that kept pads (``info.unpadded`` set), the rows move to the unpadded layout, the
    attention runs there and ``o`` comes back with zeros on the pads; ``lse`` is then in the unpadded layout
    (``[Hq, info.unpadded["T"]]``), as ``split_attn_bwd`` expects it."""
    u = info.unpadded
    if u is not None:
        ou, lse = _attn_fwd(*(repack_rows(t, u, info) for t in (q, k, v)), u, softmax_scale)
        return repack_rows(ou, info, u), lse
    return _attn_fwd(q, k, v, info, softmax_scale)


def _attn_fwd(q, k, v, info, softmax_scale):
    plan = info.plan
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need_cuda(t, name)
        if t.dtype != q.dtype:
            raise ValueError("q, k, v must share a dtype")
    desc = _desc(q, k, softmax_scale)
    T = q.shape[0]
    if T != plan.T:
        raise ValueError(f"q has {T} rows, the plan has T = {plan.T}")
    o = torch.empty_like(q)
    lse = torch.empty((q.shape[1], T), dtype=torch.float32, device=q.device)
    ws = _attn_ws(desc, plan, T, q.device, forward=True)
    check("spd_split_attn_fwd", lib.spd_split_attn_fwd(ctypes.byref(desc), ctypes.byref(plan.c), T, _ptr(q), _ptr(k),
                                                       _ptr(v), _ptr(o), _ptr(lse), _ptr(ws), ws.numel(),
                                                       _stream(q.device)))
    return o, lse


def split_attn_fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, info: ReconstructionInfo,
                           softmax_scale: Optional[float] = None):
    """spd_split_attn_fwd_noalloc: as ``split_attn_fwd`` (same results), with the library's fixed device scratch
    instead of a workspace, so only ``o`` and ``lse`` are allocated here.  Not for padded-format plans that kept
    pads (the C call refuses them)."""
    plan = info.plan
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need_cuda(t, name)
        if t.dtype != q.dtype:
            raise ValueError("q, k, v must share a dtype")
    desc = _desc(q, k, softmax_scale)
    T = q.shape[0]
    if T != plan.T:
        raise ValueError(f"q has {T} rows, the plan has T = {plan.T}")
    o = torch.empty_like(q)
    lse = torch.empty((q.shape[1], T), dtype=torch.float32, device=q.device)
    check("spd_split_attn_fwd_noalloc", lib.spd_split_attn_fwd_noalloc(ctypes.byref(desc), ctypes.byref(plan.c), T,
                                                                       _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                                                       _stream(q.device)))
    return o, lse


def split_attn_bwd(q, k, v, o, lse, dout, info: ReconstructionInfo, softmax_scale: Optional[float] = None):
    """spd_split_attn_bwd: ``(dq, dk, dv)`` from the forward's ``o``, ``lse`` and ``dout`` (for a padded-format
    plan that kept pads, computed in the unpadded layout; the pads' gradients are 0)."""
    u = info.unpadded
    if u is not None:
        grads = _attn_bwd(*(repack_rows(t, u, info) for t in (q, k, v, o)), lse, repack_rows(dout, u, info), u,
                          softmax_scale)
        return tuple(repack_rows(g, info, u) for g in grads)
    return _attn_bwd(q, k, v, o, lse, dout, info, softmax_scale)


def _attn_bwd(q, k, v, o, lse, dout, info, softmax_scale):
    plan = info.plan
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("lse", lse), ("dout", dout)):
        _need_cuda(t, name)
    if not (k.dtype == v.dtype == o.dtype == dout.dtype == q.dtype) or lse.dtype != torch.float32:
        raise ValueError("q, k, v, o, dout share a dtype; lse is float32")
    desc = _desc(q, k, softmax_scale)
    T = q.shape[0]
    if T != plan.T:
        raise ValueError(f"q has {T} rows, the plan has T = {plan.T}")
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    ws = _attn_ws(desc, plan, T, q.device, forward=False)
    check("spd_split_attn_bwd", lib.spd_split_attn_bwd(ctypes.byref(desc), ctypes.byref(plan.c), T, _ptr(q), _ptr(k),
                                                       _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
                                                       _ptr(dv), _ptr(ws), ws.numel(), _stream(q.device)))
    return dq, dk, dv


class SplitAttention(torch.autograd.Function):
    """Autograd wrapper: forward/backward are the library's two calls."""

    @staticmethod
    def forward(ctx, q, k, v, info, softmax_scale=None):
        o, lse = split_attn_fwd(q, k, v, info, softmax_scale)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.info, ctx.scale = info, softmax_scale
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv = split_attn_bwd(q, k, v, o, lse, do.contiguous(), ctx.info, ctx.scale)
        return dq, dk, dv, None, None


def split_attention(q, k, v, info, softmax_scale=None):
    return SplitAttention.apply(q, k, v, info, softmax_scale)


class StandardAttention(torch.autograd.Function):
    """Phase 2, Standard QKV Optimization: Q, K, V of the deduplicated batch are reconstructed to the full batch
    (``full_info`` from ``create_full_batch``), standard per-sample causal attention runs there, and the output
    comes back in the deduplicated layout (each prompt row from the member it was packed from).  The result equals
    split attention's; the prompt's self-attention is computed once per member instead of once per group."""

    @staticmethod
    def forward(ctx, q, k, v, info, full_info, softmax_scale=None):
        qf, kf, vf = (repack_rows(t, full_info, info) for t in (q, k, v))
        of, lsef = split_attn_fwd(qf, kf, vf, full_info, softmax_scale)
        ctx.save_for_backward(qf, kf, vf, of, lsef)
        ctx.info, ctx.full_info, ctx.scale = info, full_info, softmax_scale
        return repack_rows(of, info, full_info)

    @staticmethod
    def backward(ctx, do):
        qf, kf, vf, of, lsef = ctx.saved_tensors
        info, full = ctx.info, ctx.full_info
        dof = repack_rows_bwd(do.contiguous(), info, full)
        dqf, dkf, dvf = split_attn_bwd(qf, kf, vf, of, lsef, dof, full, ctx.scale)
        return (repack_rows_bwd(dqf, full, info), repack_rows_bwd(dkf, full, info), repack_rows_bwd(dvf, full, info),
                None, None, None)


def standard_attention(q, k, v, info, full_info, softmax_scale=None):
    return StandardAttention.apply(q, k, v, info, full_info, softmax_scale)


# ---------------------------------------------------------------------------- the pages' names


def find_prompt_groups(input_ids: torch.Tensor, response_length: int):
    """Finding Prompt Groups: ``(prompt_groups, unique_prompts [G, P])``."""
    return group(input_ids, response_length)


def create_deduplicated_batch(input_ids, position_ids, response_length, prompt_groups, unique_prompts,
                              attention_mask=None, use_unpad=False, share_prefix=False):
    """Creating Deduplicated Batch: ``(dedup_input_ids [1,T], dedup_position_ids [1,T], reconstruction_info)``;
    ``share_prefix`` also packs the prompts' common prefix once (prefix caching)."""
    return pack(input_ids, position_ids, response_length, prompt_groups, unique_prompts, attention_mask, use_unpad,
                share_prefix)


def reconstruct_sequences(dedup_hidden: torch.Tensor, reconstruction_info: ReconstructionInfo) -> torch.Tensor:
    """Reconstructing Original Batch: ``[1, T, H] -> [B, S, H]``."""
    return reconstruct(dedup_hidden, reconstruction_info)


# ---------------------------------------------------------------------------- kernel timing


def profile_begin() -> None:
    """Start recording HIP events around the library's main kernels (this thread)."""
    check("spd_profile_begin", lib.spd_profile_begin())


def profile_end() -> dict:
    """Stop recording; ``{kernel: (launches, total_ms)}`` measured on the launch streams."""
    from ._lib import SPD_K_NAMES
    n = len(SPD_K_NAMES)
    launches = (ctypes.c_int64 * n)()
    total = (ctypes.c_double * n)()
    check("spd_profile_end", lib.spd_profile_end(launches, total))
    return {SPD_K_NAMES[i]: (int(launches[i]), float(total[i])) for i in range(n)}
