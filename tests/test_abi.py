"""The C ABI: the library loads, exports every symbol include/spd.h declares,
and rejects bad arguments on the host before anything is launched.

CPU only.  Every call here fails validation (or returns for an empty input)
before it would touch a device pointer, so no pointer is ever dereferenced.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spd.h")

spd_lib = pytest.importorskip("shared_prompt_dedup_amd._lib", reason="libspd.so not built")
lib = spd_lib.lib
SpdPlan, SpdAttnDesc = spd_lib.SpdPlan, spd_lib.SpdAttnDesc

OK, INVALID, UNSUPPORTED, ALIGN, WS = 0, -1, -2, -3, -4


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(spd_[a-z_0-9]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert {"spd_group", "spd_pack", "spd_pack_rows", "spd_split_attn_fwd", "spd_split_attn_bwd",
            "spd_reconstruct"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in spd.h but not exported"
    assert set(names) == set(spd_lib.EXPORTED)


def test_status_strings_and_version():
    for s in (OK, INVALID, UNSUPPORTED, ALIGN, WS, -5):
        assert lib.spd_status_string(s)
    assert lib.spd_version() >= 100


# Fake non-null, 16-byte aligned addresses.  Each call below must fail a host
# check before any of them could be used.
A = [0x10000 * (i + 1) for i in range(16)]


def _plan(B=4, S=8, P=6, **over):
    p = SpdPlan(B, S, P, *A[:12])
    for k, v in over.items():
        setattr(p, k, v)
    return p


def test_group_rejects_bad_arguments():
    ws = lib.spd_group_workspace_bytes(4, 8)
    assert ws > 0
    p = _plan()
    # B mismatch, response_length out of range, P inconsistent
    assert lib.spd_group(A[12], 3, 8, 2, ctypes.byref(p), None, A[13], ws, None) == INVALID
    assert lib.spd_group(A[12], 4, 8, 9, ctypes.byref(p), None, A[13], ws, None) == INVALID
    assert lib.spd_group(A[12], 4, 8, 3, ctypes.byref(p), None, A[13], ws, None) == INVALID
    # null input, null plan field
    assert lib.spd_group(None, 4, 8, 2, ctypes.byref(p), None, A[13], ws, None) == INVALID
    assert lib.spd_group(A[12], 4, 8, 2, ctypes.byref(_plan(src=None)), None, A[13], ws, None) == INVALID
    # misaligned ids, workspace too small / missing
    assert lib.spd_group(A[12] + 8, 4, 8, 2, ctypes.byref(p), None, A[13], ws, None) == ALIGN
    assert lib.spd_group(A[12], 4, 8, 2, ctypes.byref(p), None, A[13], ws - 1, None) == WS
    assert lib.spd_group(A[12], 4, 8, 2, ctypes.byref(p), None, None, ws, None) == WS
    # B out of range, B*S too large for int32 indices
    assert lib.spd_group(A[12], 0, 8, 2, ctypes.byref(_plan(B=0)), None, A[13], ws, None) == INVALID
    big = _plan(B=65536, S=40000, P=39000)
    assert lib.spd_group(A[12], 65536, 40000, 1000, ctypes.byref(big), None, A[13], 1 << 40, None) == UNSUPPORTED


def test_pack_workspace_size():
    r = lambda x: (x + 255) // 256 * 256
    assert lib.spd_pack_workspace_bytes(0, 8) == 0 and lib.spd_pack_workspace_bytes(4, 0) == 0
    for B, S in ((4, 8), (16, 33792), (1, 1024), (1, 1025), (65536, 32)):
        chunks = (S + 1023) // 1024
        assert lib.spd_pack_workspace_bytes(B, S) == r(2 * B * 4) + r(B * chunks * 3 * 4), (B, S)


def test_pack_rejects_bad_arguments():
    ws = lib.spd_pack_workspace_bytes(4, 8)
    p = _plan()
    call = lambda **kw: lib.spd_pack(kw.get("ids", A[12]), kw.get("pos", A[13]), kw.get("mask", None),
                                     kw.get("esz", 8), kw.get("unpad", 0), ctypes.byref(kw.get("plan", p)),
                                     kw.get("dids", A[14]), kw.get("dpos", A[15]), kw.get("ws", A[11]),
                                     kw.get("wsb", ws), None)
    assert call(unpad=1) == INVALID             # unpad without a mask
    assert call(mask=A[10], esz=2) == INVALID    # unsupported mask element size
    assert call(unpad=2, mask=A[10]) == INVALID
    assert call(pos=None) == INVALID
    assert call(dids=A[14] + 4) == ALIGN
    assert call(wsb=ws - 1) == WS


def test_rows_calls_reject_bad_arguments():
    p = _plan()
    assert lib.spd_pack_rows(ctypes.byref(p), 5, A[12], 24, A[13], None) == ALIGN   # row bytes % 16
    assert lib.spd_pack_rows(ctypes.byref(p), 33, A[12], 32, A[13], None) == INVALID  # T > B*S
    assert lib.spd_pack_rows(ctypes.byref(p), 5, A[12] + 2, 32, A[13], None) == ALIGN
    assert lib.spd_pack_rows(ctypes.byref(p), 0, A[12], 32, A[13], None) == OK       # empty: nothing to do
    assert lib.spd_pack_rows(ctypes.byref(p), 0, A[12], 32, None, None) == OK        # zero rows may be NULL
    assert lib.spd_pack_rows(ctypes.byref(p), 5, A[12], 32, None, None) == INVALID   # ... but only zero rows
    assert lib.spd_reconstruct(ctypes.byref(p), 5, None, 48, A[13], None) == INVALID
    assert lib.spd_reconstruct(ctypes.byref(p), 5, A[12], 0, A[13], None) == INVALID
    assert lib.spd_reconstruct(ctypes.byref(p), 5, A[12], 48, A[13] + 8, None) == ALIGN
    assert lib.spd_reconstruct(ctypes.byref(p), -1, A[12], 48, A[13], None) == INVALID
    # backward calls (the zero-fill of pack_rows_bwd launches even for T = 0, so no valid call here)
    UNSUP = -2
    assert lib.spd_reconstruct_bwd(ctypes.byref(p), 5, A[12], 24, 1, A[13], None) == ALIGN
    assert lib.spd_reconstruct_bwd(ctypes.byref(p), 5, A[12], 32, 7, A[13], None) == UNSUP     # dtype
    assert lib.spd_reconstruct_bwd(ctypes.byref(p), 33, A[12], 32, 1, A[13], None) == INVALID  # T > B*S
    assert lib.spd_reconstruct_bwd(ctypes.byref(p), 5, None, 32, 1, A[13], None) == INVALID
    assert lib.spd_reconstruct_bwd(ctypes.byref(p), 5, A[12], 32, 0, A[13] + 4, None) == ALIGN
    assert lib.spd_reconstruct_bwd(ctypes.byref(p), 0, A[12], 32, 1, A[13], None) == OK       # empty
    assert lib.spd_reconstruct_bwd(ctypes.byref(p), 0, A[12], 32, 1, None, None) == OK        # zero rows: NULL
    assert lib.spd_reconstruct_bwd(ctypes.byref(p), 5, A[12], 32, 1, None, None) == INVALID
    assert lib.spd_pack_rows_bwd(ctypes.byref(p), 5, None, 32, A[13], None) == INVALID
    assert lib.spd_pack_rows_bwd(ctypes.byref(p), 5, A[12], 0, A[13], None) == INVALID
    assert lib.spd_pack_rows_bwd(ctypes.byref(p), 5, A[12] + 8, 32, A[13], None) == ALIGN
    assert lib.spd_pack_rows_bwd(ctypes.byref(p), -1, A[12], 32, A[13], None) == INVALID
    assert lib.spd_pack_rows_bwd(ctypes.byref(p), 5, A[12], 32, None, None) == INVALID


def test_share_prefix_rejects_bad_arguments():
    p = _plan()
    assert lib.spd_share_prefix(A[12], 3, 8, 2, ctypes.byref(p), None) == INVALID   # B mismatch
    assert lib.spd_share_prefix(A[12], 4, 8, 3, ctypes.byref(p), None) == INVALID   # P = S - response_length
    assert lib.spd_share_prefix(None, 4, 8, 2, ctypes.byref(p), None) == INVALID


def test_standard_mode_calls_reject_bad_arguments():
    p, q = _plan(), _plan()
    other = _plan(B=3)
    assert lib.spd_group_singletons(3, 8, 2, ctypes.byref(p), None) == INVALID     # B mismatch
    assert lib.spd_group_singletons(4, 8, 3, ctypes.byref(p), None) == INVALID     # P = S - response_length
    assert lib.spd_repack_rows(ctypes.byref(p), 5, ctypes.byref(other), 5, A[12], 32, A[13], None) == INVALID
    assert lib.spd_repack_rows(ctypes.byref(p), 33, ctypes.byref(q), 5, A[12], 32, A[13], None) == INVALID
    assert lib.spd_repack_rows(ctypes.byref(p), 5, ctypes.byref(q), 5, A[12], 24, A[13], None) == ALIGN
    assert lib.spd_repack_rows(ctypes.byref(p), 5, ctypes.byref(q), 5, None, 32, A[13], None) == INVALID
    assert lib.spd_repack_rows(ctypes.byref(p), 0, ctypes.byref(q), 5, A[12], 32, A[13], None) == OK   # empty
    assert lib.spd_repack_rows_bwd(ctypes.byref(p), 5, ctypes.byref(q), 5, A[12], 32, 9, A[13], None) == UNSUPPORTED
    assert lib.spd_repack_rows_bwd(ctypes.byref(p), 5, ctypes.byref(other), 5, A[12], 32, 1, A[13], None) == INVALID
    assert lib.spd_repack_rows_bwd(ctypes.byref(p), 5, ctypes.byref(q), 5, A[12], 32, 1, A[13] + 2, None) == ALIGN
    assert lib.spd_repack_rows_bwd(ctypes.byref(p), 5, ctypes.byref(q), 0, A[12], 32, 1, A[13], None) == OK


def test_varlen_calls_reject_bad_arguments():
    ws = lib.spd_mask_varlen_workspace_bytes(10)
    assert ws > 0 and lib.spd_mask_varlen_workspace_bytes(0) == 0
    assert lib.spd_mask_to_varlen(A[10], 3, 10, 10, A[11], A[12], A[13], A[14], ws, None) == INVALID   # elem size
    assert lib.spd_mask_to_varlen(A[10], 1, 0, 10, A[11], A[12], A[13], A[14], ws, None) == INVALID    # no rows
    assert lib.spd_mask_to_varlen(None, 1, 10, 10, A[11], A[12], A[13], A[14], ws, None) == INVALID
    assert lib.spd_mask_to_varlen(A[10], 1, 10, 10, A[11], A[12], A[13], A[14], ws - 1, None) == WS
    assert lib.spd_mask_to_varlen(A[10], 8, 10, 2**28, A[11], A[12], A[13], A[14], ws, None) == UNSUPPORTED
    assert lib.spd_mask_to_varlen(A[10], 1, 10, 10, A[11], A[12], A[13], A[14] + 4, ws, None) == ALIGN
    p = _plan()
    assert lib.spd_varlen_params(ctypes.byref(p), None, A[13], A[14], A[15], None) == INVALID


def _desc(**kw):
    d = dict(num_q_heads=16, num_kv_heads=8, head_dim=128, dtype=1, softmax_scale=0.088)
    d.update(kw)
    return SpdAttnDesc(**d)


def test_attention_rejects_bad_descriptors():
    p = _plan()
    for bad, code in ((dict(num_q_heads=12, num_kv_heads=8), INVALID), (dict(num_kv_heads=0), INVALID),
                      (dict(head_dim=96), UNSUPPORTED), (dict(dtype=7), UNSUPPORTED),
                      (dict(softmax_scale=0.0), INVALID), (dict(softmax_scale=float("nan")), INVALID)):
        d = _desc(**bad)
        assert lib.spd_attn_workspace_bytes(ctypes.byref(d), 4, 20) == 0
        assert lib.spd_split_attn_fwd(ctypes.byref(d), ctypes.byref(p), 20, *A[:5], A[5], 1 << 30, None) == code


def test_attention_validation_order():
    p = _plan()
    d = _desc()
    ws = lib.spd_attn_workspace_bytes(ctypes.byref(d), 4, 20)
    fws = lib.spd_attn_fwd_workspace_bytes(ctypes.byref(d), 4, 20)
    assert 0 < fws < ws
    fwd = lambda T, ptrs, wsb=fws: lib.spd_split_attn_fwd(ctypes.byref(d), ctypes.byref(p), T, *ptrs, A[5], wsb,
                                                          None)
    assert fwd(20, A[:5], fws - 1) == WS
    assert fwd(33, A[:5]) == INVALID     # T > B*S
    assert fwd(20, [A[0], None, A[2], A[3], A[4]]) == INVALID
    assert fwd(20, [A[0], A[1] + 2, A[2], A[3], A[4]]) == ALIGN
    assert fwd(0, A[:5], lib.spd_attn_fwd_workspace_bytes(ctypes.byref(d), 4, 0)) == OK   # empty batch
    assert fwd(0, [None] * 5, lib.spd_attn_fwd_workspace_bytes(ctypes.byref(d), 4, 0)) == OK   # zero rows: NULL
    assert lib.spd_split_attn_bwd(ctypes.byref(d), ctypes.byref(p), 20, *A[:9], A[9], ws - 1, None) == WS
    assert lib.spd_split_attn_bwd(ctypes.byref(d), ctypes.byref(p), 0, *([None] * 9), A[9],
                                  lib.spd_attn_workspace_bytes(ctypes.byref(d), 4, 0), None) == OK
    bwd = lambda ptrs: lib.spd_split_attn_bwd(ctypes.byref(d), ctypes.byref(p), 20, *ptrs, A[9], ws, None)
    assert bwd([*A[:8], None]) == INVALID
    assert bwd([*A[:8], A[8] + 8]) == ALIGN


def test_attention_rejects_kv_beyond_4gib():
    """K / V row offsets in the kernels are 32-bit: T * Hkv * d * element bytes must stay below 2^32.  The limit
    is checked before the workspace, so a missing workspace tells which side of it a size falls on."""
    p = _plan(B=64, S=65536, P=65000)
    for dt, elt in ((1, 2), (0, 4)):
        d = _desc(dtype=dt)
        limit = (1 << 32) // (8 * 128 * elt)           # first T that reaches 4 GiB of K (Hkv 8, d 128)
        for T, code in ((limit, UNSUPPORTED), (limit - 1, WS)):
            assert lib.spd_split_attn_fwd(ctypes.byref(d), ctypes.byref(p), T, *A[:5], None, 0, None) == code
            assert lib.spd_split_attn_bwd(ctypes.byref(d), ctypes.byref(p), T, *A[:9], None, 0, None) == code


def test_attention_rejects_padded_plan_with_mask():
    """A plan packed in the padded format with an attention mask may hold pads among its rows; the attention
    calls refuse it (the caller runs attention on the unpadded plan of the same groups)."""
    d = _desc()
    p = _plan(padded_with_mask=1)
    fws = lib.spd_attn_fwd_workspace_bytes(ctypes.byref(d), 4, 20)
    ws = lib.spd_attn_workspace_bytes(ctypes.byref(d), 4, 20)
    assert lib.spd_split_attn_fwd(ctypes.byref(d), ctypes.byref(p), 20, *A[:5], A[5], fws, None) == UNSUPPORTED
    assert lib.spd_split_attn_bwd(ctypes.byref(d), ctypes.byref(p), 20, *A[:9], A[9], ws, None) == UNSUPPORTED
    assert lib.spd_split_attn_fwd(ctypes.byref(d), ctypes.byref(p), 0, *([None] * 5), A[5], fws, None) == UNSUPPORTED


def test_noalloc_forward_rejects_before_touching_the_device():
    """The workspace-free forward validates like the forward and refuses sizes whose workspace exceeds its fixed
    4 MiB scratch -- all before any HIP call."""
    d = _desc()
    call = lambda plan, T, ptrs: lib.spd_split_attn_fwd_noalloc(ctypes.byref(d), ctypes.byref(plan), T, *ptrs, None)
    p = _plan()
    assert call(p, 33, A[:5]) == INVALID                          # T > B*S
    assert call(p, 20, [A[0], None, A[2], A[3], A[4]]) == INVALID
    assert call(p, 20, [A[0], A[1] + 2, A[2], A[3], A[4]]) == ALIGN
    assert call(_plan(padded_with_mask=1), 20, A[:5]) == UNSUPPORTED
    assert call(p, 0, [None] * 5) == OK                           # empty batch: nothing to do
    mqa = _desc(num_q_heads=1, num_kv_heads=1)
    big = _plan(B=65536, S=32, P=16)                               # 8 bytes of planner scratch per sample
    need = lib.spd_attn_fwd_workspace_bytes(ctypes.byref(mqa), 65536, 1000)
    assert need > 4 << 20
    assert lib.spd_split_attn_fwd_noalloc(ctypes.byref(mqa), ctypes.byref(big), 1000, *A[:5], None) == WS


def test_workspace_grows_with_sizes():
    d = _desc()
    small = lib.spd_attn_workspace_bytes(ctypes.byref(d), 4, 1000)
    big = lib.spd_attn_workspace_bytes(ctypes.byref(d), 4, 100000)
    assert 0 < small < big
    # holds at least the per-row softmax statistic of every query head
    assert big >= 16 * 100000 * 4


def test_single_hip_runtime_in_process():
    """The binding must share PyTorch's HIP runtime, never map a second one."""
    import subprocess
    import sys
    code = ("import shared_prompt_dedup_amd._lib as L, re\n"
            "maps = open('/proc/self/maps').read()\n"
            "paths = sorted(set(re.findall(r'(\\S*libamdhip64\\S*)', maps)))\n"
            "print(len(paths), paths)\n"
            "assert len(paths) == 1, paths\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(spd_lib, "LIB_PATH", "/nonexistent/libspd.so")
    with pytest.raises(ImportError, match="not built"):
        spd_lib._load()
