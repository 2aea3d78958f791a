"""Prompt-deduplicated split attention for AMD Instinct MI355X (gfx950).

The compute path is the HIP library ``libspd.so`` (C ABI in ``include/spd.h``);
this package is its thin Python binding.  Using any of its functions requires
the built library (``python -m shared_prompt_dedup_amd.build``): the first
access raises ImportError when it is missing -- there is no CPU or PyTorch
fallback.  (The package itself imports without it so that the build step,
``shared_prompt_dedup_amd.build``, can run.)
"""
import importlib

_API = ("Plan", "PromptGroups", "ReconstructionInfo", "SplitAttention", "PackRows", "Reconstruct",
        "create_deduplicated_batch", "find_prompt_groups", "group", "pack", "pack_rows", "pack_rows_bwd",
        "reconstruct", "reconstruct_bwd", "reconstruct_sequences", "split_attention", "split_attn_bwd",
        "split_attn_fwd", "profile_begin", "profile_end", "singleton_groups", "create_full_batch", "repack_rows",
        "repack_rows_bwd", "StandardAttention", "standard_attention", "attention_mask_to_flash_attn_params",
        "flash_attn_params")
_LIB = ("EXPORTED", "LIB_PATH", "SpdError")

__all__ = list(_API + _LIB)


def __getattr__(name):
    if name in _API:
        return getattr(importlib.import_module(".api", __name__), name)
    if name in _LIB:
        return getattr(importlib.import_module("._lib", __name__), name)
    raise AttributeError(name)
