#!/usr/bin/env python3
"""Throughput of prompt-deduplicated split attention on one MI355X.

One step is one pass of the whole hot path over one synthetic batch already
resident in HBM, forward and backward:
  group (spd_group) -> pack ids/positions (spd_pack) -> pack the per-token
  rows entering the layer (spd_pack_rows) -> split-attention forward
  (spd_split_attn_fwd) -> reconstruct the attention output to
  [batch, seq, Hq*d] (spd_reconstruct);
  then the gradient of that output back to the packed rows
  (spd_reconstruct_bwd, which gives the attention's dO) -> split-attention
  backward (spd_split_attn_bwd) -> the packed rows' gradient (dQ standing in
  for it) back to [batch, seq, Hq*d] (spd_pack_rows_bwd).

`value` is the useful split-attention forward+backward work per step
(4*d*Hq FLOP per attended (query, key) pair forward, 10*d*Hq backward,
pairs counted from the plan) divided by the measured time of the whole step.
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from workloads import BENCH_WORKLOAD  # noqa: E402  (numpy only)

METRIC = "split-attn fwd+bwd TFLOP/s & % bf16 MFMA peak; pack/reconstruct GB/s"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E

# HBM traffic per launch from two rocprofv3 --pmc passes (FETCH_SIZE, then
# WRITE_SIZE, KiB per dispatch) over `bench.py --steps 1 --warmup 1
# --cpu-baseline off --profile-steps 1 [--workload W]`.  The same counters
# read for the 1 GiB device-to-device copy in that run give the scale factors
# (FETCH_SIZE counts half of what is read on this chip, WRITE_SIZE counts
# exactly).  Valid only for the kernel sources hashed in TRAFFIC_SOURCES:
# after any change there the figure is reported as null.
TRAFFIC_FETCH_SCALE = 2.0
TRAFFIC_WRITE_SCALE = 1.0
TRAFFIC_SOURCES = ("spd_attn.h", "spd_attn_dev.h", "spd_attn_api.hip", "spd_attn_fwd.hip", "spd_attn_bwd.hip",
                   "spd_internal.h", "spd_dedup.hip")
TRAFFIC_SOURCES_SHA256 = "bb06d9c9f236dc2d0c97683468fbcaee33bb538e13262d0e92214e6828262a7b"
TRAFFIC_KIB = {   # workload -> kernel -> (FETCH_SIZE KiB, WRITE_SIZE KiB) per dispatch, uncalibrated
    "long_2x8_p32768_r256to1024_unpad": {
        "fwd": (1271923, 318043), "bwd_pre": (305777, 9784), "bwd_dq": (1804535, 303184),
        "bwd_dkdv": (5037939, 303206), "reconstruct": (163459, 2162688), "pack_rows": (152799, 303190),
        "reconstruct_bwd": (1070312, 303180), "pack_rows_bwd": (163248, 2162688),
    },
}


def sources_sha256():
    h = hashlib.sha256()
    for name in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, "shared_prompt_dedup_amd", "csrc", name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def measured_traffic(kernel, workload):
    """Calibrated HBM bytes per launch, or None when not measured for these sources and this workload."""
    table = TRAFFIC_KIB.get(workload, {})
    if kernel not in table or TRAFFIC_SOURCES_SHA256 != sources_sha256():
        return None
    fetch, write = table[kernel]
    return round((fetch * TRAFFIC_FETCH_SCALE + write * TRAFFIC_WRITE_SCALE) * 1024)


def attended_pairs(info):
    """(query, key) pairs split attention evaluates, from the plan's segment lengths (a shared prefix of Lp rows:
    Lp (Lp + 1) / 2 once, and every later row also sees its Lp keys)."""
    G = info["G"]
    lp = int(info.get("prefix_len", 0))
    pl = info["prompt_len"][:G].cpu().tolist()
    rl = info["resp_len"].cpu().tolist()
    gof = info["group_of"].cpu().tolist()
    pairs = lp * (lp + 1) // 2 + sum(p * lp + p * (p + 1) // 2 for p in pl)
    for b, r in enumerate(rl):
        pairs += r * (lp + pl[gof[b]]) + r * (r + 1) // 2
    return pairs


def attention_split(kern_ms, fwd_flops, bwd_flops):
    """Forward, backward and forward + backward kernel time and useful TFLOP/s (backward = preprocessing, dq and
    dk/dv, FlashAttention's 10 d FLOPs per pair and head)."""
    fwd = kern_ms.get("fwd")
    bwd = sum(kern_ms.get(k) or 0.0 for k in ("bwd_pre", "bwd_dq", "bwd_dkdv")) or None
    out = {}
    for key, ms, flops in (("fwd", fwd, fwd_flops), ("bwd", bwd, bwd_flops),
                           ("fwd_bwd", (fwd or 0.0) + (bwd or 0.0) or None, fwd_flops + bwd_flops)):
        if ms:
            out[key] = {"ms": round(ms, 4), "tflops": round(flops / (ms * 1e-3) / 1e12, 2)}
    return out


def cpu_baseline(w, bt, pairs, min_seconds=10.0, max_tokens=16384):
    """The oracle, as it stands, forward + backward (fp64), timed on a bounded slice of the same workload and
    scaled to the whole batch.

    The slice is the batch's first sample alone, cut to its first `max_tokens` tokens (a causal sequence in its
    own right), one query head at a time until at least `min_seconds` of CPU work.  The oracle runs
    non-deduplicated attention, so on the whole batch it does sum_b L_b (L_b + 1) / 2 (query, key) pairs per
    head; its time there is the slice's time scaled by that count over the slice's, and `value` is the batch's
    useful (deduplicated) FLOPs over that time, counted as on the GPU (14 d FLOP per pair and head)."""
    import oracle
    from workloads import Batch, make_attn_inputs
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"],
                           default=1)
    except Exception:  # pragma: no cover
        blas_threads = 1
    S = bt.input_ids.shape[1]
    n = min(S, max_tokens)
    resp = max(0, bt.response_length - (S - n))       # response columns left in the first n
    one = Batch(bt.input_ids[:1, :n], bt.position_ids[:1, :n], bt.attention_mask[:1, :n], resp, None, None)
    groups, uniq = oracle.find_prompt_groups(one.input_ids, one.response_length)
    _, _, info = oracle.create_deduplicated_batch(one.input_ids, one.position_ids, one.response_length, groups, uniq,
                                                  attention_mask=one.attention_mask, use_unpad=w.use_unpad)
    x = make_attn_inputs(w, info["T"])
    _, slice_plain = oracle.attended_pairs(info)
    heads = 0
    dt = 0.0
    while heads < w.num_q_heads and dt < min_seconds:
        t0 = time.perf_counter()
        oracle.split_attention_forward(x.q, x.k, x.v, info, heads=[heads])
        oracle.split_attention_backward(x.q, x.k, x.v, x.do, info, heads=[heads])
        dt += time.perf_counter() - t0
        heads += 1
    # non-deduplicated pairs of the whole batch (one causal sequence per sample), counted by the oracle's plan
    g_all, u_all = oracle.find_prompt_groups(bt.input_ids, bt.response_length)
    _, _, info_all = oracle.create_deduplicated_batch(bt.input_ids, bt.position_ids, bt.response_length, g_all,
                                                      u_all, attention_mask=bt.attention_mask, use_unpad=w.use_unpad)
    _, plain = oracle.attended_pairs(info_all)
    t_full = dt * (plain * w.num_q_heads) / (slice_plain * heads)
    useful = 14 * w.head_dim * w.num_q_heads * pairs
    return {"value": round(useful / t_full / 1e12, 6), "unit": "TFLOP/s", "cores": int(blas_threads),
            "kind": "oracle",
            "sample": f"fp64 numpy oracle (non-deduplicated per-sample attention), forward+backward of the batch's "
                      f"first sample alone, its first {info['T']} tokens, {heads} of {w.num_q_heads} query heads, "
                      f"{dt:.1f} s; scaled to the whole batch by non-deduplicated pairs ({plain} per head vs "
                      f"{slice_plain} in the slice: {t_full:.0f} s estimated); value = the batch's deduplicated "
                      f"useful FLOPs (14 d per pair and head) over that time; host cores available "
                      f"{len(os.sched_getaffinity(0))}, {platform.processor() or platform.machine()}"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=None, help="workload name in workloads.WORKLOADS")
    ap.add_argument("--cpu-baseline", choices=("on", "off"), default="on")
    ap.add_argument("--profile-steps", type=int, default=20, help="steps timed per kernel with HIP events")
    ap.add_argument("--share-prefix", action="store_true",
                    help="also pack the prompts' common prefix once (prefix caching); try it with --workload "
                         "prefix_4x8_s4096_p5120_r512")
    ap.add_argument("--mode", choices=("split", "standard", "padded_mask"), default="split",
                    help="split attention on the deduplicated batch (default); the standard QKV mode: the same "
                         "layer with attention run per sample on the full batch; or padded_mask: a batch with "
                         "padding packed in the padded format with its attention mask (pads kept, no part in "
                         "attention; default workload long_2x8_p32768_r256to1024_unpad)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this build measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "groups shard across GPUs without exchange, so the per-GPU figure is the one reported.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import shared_prompt_dedup_amd as spd
    from workloads import WORKLOADS, make_attn_inputs, make_batch

    name = args.workload or BENCH_WORKLOAD
    w = WORKLOADS[name]
    use_unpad = w.use_unpad and args.mode != "padded_mask"
    assert w.dtype == "bf16"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    bt = make_batch(w)
    ids = torch.from_numpy(bt.input_ids).to(dev)
    pos = torch.from_numpy(bt.position_ids).to(dev)
    mask = torch.from_numpy(bt.attention_mask).to(dev)
    R = bt.response_length
    B, S = ids.shape
    Hq, Hkv, d = w.num_q_heads, w.num_kv_heads, w.head_dim
    W = Hq * d

    groups, uniq = spd.group(ids, R, return_lists=False)
    _, _, info = spd.pack(ids, pos, R, groups, uniq, attention_mask=mask, use_unpad=use_unpad,
                          share_prefix=args.share_prefix)
    T = info["T"]
    pairs = attended_pairs(info.unpadded if info.unpadded is not None else info)
    x = make_attn_inputs(w, T)
    conv = lambda bits: torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)
    q, k, v = conv(x.q_bits), conv(x.k_bits), conv(x.v_bits)
    del x
    gen = torch.Generator(device=dev).manual_seed(w.seed)
    hidden = torch.randn((B, S, W), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    dout_full = torch.randn((B, S, W), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)

    def step_split():
        g, u = spd.group(ids, R, return_lists=False)
        _, _, inf = spd.pack(ids, pos, R, g, u, attention_mask=mask, use_unpad=use_unpad,
                             share_prefix=args.share_prefix)
        packed = spd.pack_rows(hidden, inf)
        o, lse = spd.split_attn_fwd(q, k, v, inf)
        out = spd.reconstruct(o.view(T, W), inf)
        dout = spd.reconstruct_bwd(dout_full, inf).view(T, Hq, d)
        dq, dk, dv = spd.split_attn_bwd(q, k, v, o, lse, dout, inf)
        dhidden = spd.pack_rows_bwd(dq.view(T, W), inf)
        return packed, out, dhidden, dk, dv

    def step_standard():
        # Standard QKV: Q, K, V reconstructed to the full batch (every sample its own prompt copy), attention
        # per sample there, output and gradients moved back to the deduplicated layout.
        g, u = spd.group(ids, R, return_lists=False)
        _, _, inf = spd.pack(ids, pos, R, g, u, attention_mask=mask, use_unpad=use_unpad,
                             share_prefix=args.share_prefix)
        _, _, full = spd.create_full_batch(ids, pos, R, attention_mask=mask, use_unpad=use_unpad)
        packed = spd.pack_rows(hidden, inf)
        qf, kf, vf = (spd.repack_rows(t, full, inf) for t in (q, k, v))
        of, lsef = spd.split_attn_fwd(qf, kf, vf, full)
        o = spd.repack_rows(of, inf, full)
        out = spd.reconstruct(o.view(T, W), inf)
        dout = spd.reconstruct_bwd(dout_full, inf)
        dof = spd.repack_rows_bwd(dout, inf, full).view(-1, Hq, d)
        dqf, dkf, dvf = spd.split_attn_bwd(qf, kf, vf, of, lsef, dof, full)
        dq, dk, dv = (spd.repack_rows_bwd(t, full, inf) for t in (dqf, dkf, dvf))
        dhidden = spd.pack_rows_bwd(dq.view(T, W), inf)
        return packed, out, dhidden, dk, dv

    step = step_standard if args.mode == "standard" else step_split
    kernel_pairs = pairs
    if args.mode == "standard":
        _, _, full0 = spd.create_full_batch(ids, pos, R, attention_mask=mask, use_unpad=use_unpad)
        kernel_pairs = attended_pairs(full0)      # what the full-batch attention evaluates
        T_full = full0["T"]
        del full0

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps

    fwd_flops = 4 * d * Hq * pairs
    bwd_flops = 10 * d * Hq * pairs
    value = (fwd_flops + bwd_flops) / (ms_per_step * 1e-3) / 1e12

    # Per-kernel HIP events (recorded by the library on the launch stream), one
    # window per step so that the spread across steps is seen too.
    per_step = {}
    for _ in range(args.profile_steps):
        spd.profile_begin()
        step()
        torch.cuda.synchronize()
        for kname, (n, tot) in spd.profile_end().items():
            if n:
                per_step.setdefault(kname, []).append(tot / n)
    kern_ms = {kname: float(np.mean(v)) for kname, v in per_step.items()}
    kern_spread = {kname: [round(float(x), 4) for x in np.percentile(v, [10, 50, 90])]
                   for kname, v in per_step.items()}
    row_bytes = W * 2
    Ta = {"split": T, "standard": None, "padded_mask": None}[args.mode]     # rows the attention kernels run on
    if args.mode == "standard":
        Ta = T_full
    elif args.mode == "padded_mask":
        Ta = info.unpadded["T"] if info.unpadded is not None else T
    kernel_work = {
        "fwd": ("mfma", 4 * d * Hq * kernel_pairs),
        "bwd_dkdv": ("mfma", 8 * d * Hq * kernel_pairs),      # S, dP recomputed; dV, dK
        "bwd_dq": ("mfma", 6 * d * Hq * kernel_pairs),        # S, dP recomputed; dQ
        "bwd_pre": ("hbm", 2 * Ta * W * 2 + Ta * Hq * 4),
        "reconstruct": ("hbm", T * row_bytes + B * S * row_bytes),
        "pack_rows": ("hbm", 2 * T * row_bytes),
        "reconstruct_bwd": ("hbm", B * S * row_bytes + T * row_bytes),
        "pack_rows_bwd": ("hbm", T * row_bytes + B * S * row_bytes),
    }
    kernels = {}
    for kname, (bound, work) in kernel_work.items():
        ms = kern_ms.get(kname)
        if not ms:
            continue
        if bound == "mfma":
            ach = work / (ms * 1e-3) / 1e12
            kernels[kname] = {"ms": round(ms, 4), "bound": "mfma", "achieved": round(ach, 2),
                              "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4)}
        else:
            ach = work / (ms * 1e-3) / 1e9
            kernels[kname] = {"ms": round(ms, 4), "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                              "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4)}
        kernels[kname]["ms_p10_p50_p90"] = kern_spread[kname]
        if args.mode == "split":
            kernels[kname]["traffic"] = measured_traffic(kname, name)
    # The gathers again, alone, with the 256 MB Infinity Cache flushed before each
    # call by reading a 512 MB buffer (a read leaves clean lines behind, so the
    # flush adds no write-back to the timed call; outside the timed windows).
    if args.mode == "split":
        flush = torch.ones((512 << 20) // 4, dtype=torch.float32, device=dev)
        o_rows = torch.empty(T, W, dtype=torch.bfloat16, device=dev)
        for kname, call in (("reconstruct", lambda: spd.reconstruct(o_rows, info)),
                            ("pack_rows", lambda: spd.pack_rows(hidden, info))):
            times = []
            for _ in range(max(5, args.profile_steps)):
                flush.sum()
                torch.cuda.synchronize()
                spd.profile_begin()
                call()
                torch.cuda.synchronize()
                n, tot = spd.profile_end()[kname]
                times.append(tot / n)
            ms = float(np.median(times))
            ach = kernel_work[kname][1] / (ms * 1e-3) / 1e9
            kernels[kname + "_cache_flushed"] = {"ms": round(ms, 4), "bound": "hbm", "achieved": round(ach, 1),
                                                 "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                                 "frac": round(ach / PEAK_HBM_GBS, 4)}
        del flush, o_rows
    # Flash Attention Integration: the block-diagonal prompt-to-prompt mask of this batch -> cu_seqlens.
    if args.mode == "split":
        G = info["G"]
        pl = info["prompt_len"][:G].to(torch.int64)
        ptot = int(pl.sum().item())
        if ptot > 0:
            blk = torch.repeat_interleave(torch.arange(G, device=dev), pl)
            ar = torch.arange(ptot, device=dev)
            pmask = (blk[:, None] == blk[None, :]) & (ar[None, :] <= ar[:, None])
            spd.attention_mask_to_flash_attn_params(pmask)
            torch.cuda.synchronize()
            spd.profile_begin()
            for _ in range(5):
                spd.attention_mask_to_flash_attn_params(pmask)
            torch.cuda.synchronize()
            n_mv, tot_mv = spd.profile_end()["mask_to_varlen"]
            ms = tot_mv / n_mv
            ach = ptot * ptot / (ms * 1e-3) / 1e9
            kernels["mask_to_varlen"] = {"ms": round(ms, 4), "bound": "hbm", "achieved": round(ach, 1),
                                         "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4)}
            del pmask, blk, ar
    # Practical HBM reference: a plain device-to-device copy of 1 GiB (read + write).
    src_buf = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst_buf = torch.empty_like(src_buf)
    dst_buf.copy_(src_buf)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(5):
        dst_buf.copy_(src_buf)
    ev1.record()
    torch.cuda.synchronize()
    copy_gbs = 5 * 2 * (1 << 30) / (ev0.elapsed_time(ev1) * 1e-3) / 1e9
    del src_buf, dst_buf
    dom = max(kernels, key=lambda kk: kernels[kk]["ms"])
    roof = dict(kernels[dom])
    roof.pop("ms")
    roof = {"kernel": dom, **roof, "traffic": measured_traffic(dom, name) if args.mode == "split" else None}

    attn_ms = sum(kern_ms[kk] for kk in ("fwd", "bwd_pre", "bwd_dq", "bwd_dkdv") if kern_ms.get(kk))
    result = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": name, "batch": B, "unique_prompts": w.num_prompts, "prompt_len": w.prompt_len,
                   "response_len": w.response_len, "q_heads": Hq, "kv_heads": Hkv, "head_dim": d,
                   "packed_tokens": T, "attended_pairs": pairs, "parallelism": "single GPU",
                   "attention": args.mode, "shared_prefix_rows": int(info.get("prefix_len", 0))},
        "frac_of_bf16_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "attention_kernels_tflops": round((fwd_flops + bwd_flops) / (attn_ms * 1e-3) / 1e12, 2),
        "attention_split": attention_split(kern_ms, fwd_flops, bwd_flops),
        "roofline": roof,
        "kernels": kernels,
        "hbm_copy_gbs": round(copy_gbs, 1),
    }
    if args.cpu_baseline == "on":
        result["cpu_baseline"] = cpu_baseline(w, bt, pairs)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
