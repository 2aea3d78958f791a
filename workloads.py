"""Seeded synthetic inputs for prompt-deduplicated split attention.

This module only draws random numbers and lays them out as an RL training
batch: ``[prompt][response]`` token rows, position ids, an attention mask,
and attention tensors in packed layout.  It holds none of the method's
arithmetic (no grouping, packing, reconstruction or attention); both the CPU
oracle's tests and the GPU path's tests and bench import it, and neither of
those imports the other.

The batch shapes follow the workloads the pages describe ("Performance
Benchmarks", Usage Tips: a 16-sample batch with 2 unique prompts of 8192
tokens and 512-token responses; "Redundancy Analysis": a 10K prompt with ten
1K responses; "How Prompt Deduplication Works", Debugging & Analysis: a long
prompt with response lengths between 0.4Ki and 1.0Ki padded to 1.0Ki).
No dataset is used anywhere; every value is drawn here from a fixed seed.

Draw order for a workload with seed ``s`` (numpy PCG64):
  batch stream ``default_rng(s)``: prompt ids ``[G, P]``, response ids
  ``[B, R]``, then (variable-length workloads only) response lengths ``[B]``;
  attention stream ``default_rng([s, 1])``: Q ``[T, Hq, d]``, K, V
  ``[T, Hkv, d]``, dO ``[T, Hq, d]``, each ``standard_normal(float32) * sigma``
  and, for bf16 workloads, rounded to bf16 with round-to-nearest-even.
Sample ``b`` carries prompt ``b // n`` (rollout order) unless a seeded
permutation of the rows is requested.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    num_prompts: int          # G: unique prompts
    rollout_n: int            # n: responses per prompt
    prompt_len: int           # P
    response_len: int         # R (padded response length)
    num_q_heads: int          # Hq
    num_kv_heads: int         # Hkv
    head_dim: int             # d
    dtype: str                # "f32" or "bf16"
    vocab: int
    sigma: float              # scale of the N(0,1) attention tensors
    seed: int
    # (lo, hi) inclusive response-length range for right-padded variable
    # responses (packed with use_unpad=True); None = every response is full.
    resp_len_range: Optional[tuple] = None
    shared_prefix: int = 0      # leading prompt tokens common to every prompt (0: prompts independent)

    @property
    def batch(self) -> int:
        return self.num_prompts * self.rollout_n

    @property
    def seq_len(self) -> int:
        return self.prompt_len + self.response_len

    @property
    def use_unpad(self) -> bool:
        return self.resp_len_range is not None

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


QWEN_VOCAB = 151936

WORKLOADS = {
    # 8 samples = 2 prompts x 4 responses, prompt 64, response 32, MQA 2/1/64, fp32.
    "tiny_fp32": Workload("tiny_fp32", 2, 4, 64, 32, 2, 1, 64, "f32", 1000, 1.0, 1000),
    # Qwen3-0.6B-like attention layer: 16 = 2 x 8, prompt 8192, response 512, GQA 16/8/128.
    "qwen3_0p6b_2x8_p8192_r512": Workload(
        "qwen3_0p6b_2x8_p8192_r512", 2, 8, 8192, 512, 16, 8, 128, "bf16", QWEN_VOCAB, 0.5, 1001),
    # The redundancy example: one 10K prompt, ten 1K responses.
    "redundancy_1x10_p10240_r1024": Workload(
        "redundancy_1x10_p10240_r1024", 1, 10, 10240, 1024, 16, 8, 128, "bf16", QWEN_VOCAB, 0.5, 1002),
    # Long context, right-padded responses of U[256,1024] tokens, unpadded packing.
    "long_2x8_p32768_r256to1024_unpad": Workload(
        "long_2x8_p32768_r256to1024_unpad", 2, 8, 32768, 1024, 16, 8, 128, "bf16", QWEN_VOCAB, 0.5,
        1003, (256, 1024)),
    # Backward-heavy batch: 32 = 4 x 8, prompt 4096, response 1024.
    "bwd_4x8_p4096_r1024": Workload(
        "bwd_4x8_p4096_r1024", 4, 8, 4096, 1024, 16, 8, 128, "bf16", QWEN_VOCAB, 0.5, 1004),
    # Partially overlapping prompts: 32 = 4 x 8, four 5120-token prompts that share their first 4096 tokens
    # (a common system prompt), response 512.  Exercises prefix sharing.
    "prefix_4x8_s4096_p5120_r512": Workload(
        "prefix_4x8_s4096_p5120_r512", 4, 8, 5120, 512, 16, 8, 128, "bf16", QWEN_VOCAB, 0.5, 1005,
        shared_prefix=4096),
}

# The single-GPU workload that throughput is quoted on: the largest one (32K-token prompts, about 1.4e9 attended
# pairs).  The other bf16 workloads are measured with bench.py --workload.
BENCH_WORKLOAD = "long_2x8_p32768_r256to1024_unpad"


@dataclass
class Batch:
    input_ids: np.ndarray        # [B, S] int64
    position_ids: np.ndarray     # [B, S] int64
    attention_mask: np.ndarray   # [B, S] int64, 1 = valid, 0 = pad
    response_length: int         # S - P
    row_prompt: np.ndarray       # [B] which drawn prompt each row carries
    row_resp_len: np.ndarray     # [B] number of valid response tokens


def make_batch(w: Workload, permute: bool = False, pad_id: int = 0) -> Batch:
    """Token rows ``[prompt][response]`` per sample, right-padded responses."""
    rng = np.random.default_rng(w.seed)
    B, P, R = w.batch, w.prompt_len, w.response_len
    S = P + R
    prompts = rng.integers(0, w.vocab, size=(w.num_prompts, P), dtype=np.int64)
    if w.shared_prefix:
        L = w.shared_prefix
        prompts[:, :L] = prompts[0, :L]
        if L < P:   # column L differs between prompts, so the common prefix is exactly L long
            prompts[:, L] = (prompts[0, L] + np.arange(w.num_prompts)) % w.vocab
    resps = rng.integers(0, w.vocab, size=(B, R), dtype=np.int64)
    if w.resp_len_range is not None:
        lo, hi = w.resp_len_range
        rlen = rng.integers(lo, hi + 1, size=B).astype(np.int64)
    else:
        rlen = np.full(B, R, dtype=np.int64)
    row_prompt = np.arange(B) // w.rollout_n
    if permute:
        perm = np.random.default_rng([w.seed, 2]).permutation(B)
        row_prompt = row_prompt[perm]
    ids = np.empty((B, S), dtype=np.int64)
    ids[:, :P] = prompts[row_prompt]
    ids[:, P:] = resps
    t = np.arange(S)[None, :]
    mask = (t < (P + rlen)[:, None]).astype(np.int64)
    ids[mask == 0] = pad_id
    pos = np.broadcast_to(np.arange(S, dtype=np.int64), (B, S)).copy()
    return Batch(ids, pos, mask, R, row_prompt, rlen)


def round_to_bf16(x: np.ndarray):
    """Round float32 to bf16 (nearest, ties to even).

    Returns ``(bits, values)``: the uint16 bf16 bit patterns and the same
    numbers as float32.  Inputs here are finite draws, so no NaN handling.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bits = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    vals = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return bits, vals


@dataclass
class AttnInputs:
    q: np.ndarray     # [T, Hq, d] float32 values (bf16-exact for bf16 workloads)
    k: np.ndarray     # [T, Hkv, d]
    v: np.ndarray     # [T, Hkv, d]
    do: np.ndarray    # [T, Hq, d]
    q_bits: Optional[np.ndarray] = None   # uint16 bf16 patterns (bf16 workloads)
    k_bits: Optional[np.ndarray] = None
    v_bits: Optional[np.ndarray] = None
    do_bits: Optional[np.ndarray] = None


def make_attn_inputs(w: Workload, T: int, with_grad: bool = True) -> AttnInputs:
    """Packed-layout Q/K/V (and dO) for ``T`` packed rows.

    ``T`` is a caller-supplied row count; drawing directly in packed layout
    makes every prompt's rows exist once, so copies agree by construction.
    """
    rng = np.random.default_rng([w.seed, 1])
    shapes = [(T, w.num_q_heads, w.head_dim), (T, w.num_kv_heads, w.head_dim),
              (T, w.num_kv_heads, w.head_dim)]
    if with_grad:
        shapes.append((T, w.num_q_heads, w.head_dim))
    arrs = []
    for shp in shapes:
        a = rng.standard_normal(size=shp, dtype=np.float32)
        a *= np.float32(w.sigma)
        arrs.append(a)
    if w.dtype == "bf16":
        bits, vals = zip(*(round_to_bf16(a) for a in arrs))
        bits, vals = list(bits), list(vals)
        if not with_grad:
            bits.append(None)
            vals.append(None)
        return AttnInputs(vals[0], vals[1], vals[2], vals[3], bits[0], bits[1], bits[2], bits[3])
    if not with_grad:
        arrs.append(None)
    return AttnInputs(arrs[0], arrs[1], arrs[2], arrs[3])
