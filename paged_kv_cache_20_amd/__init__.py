"""Paged grouped-query attention for AMD MI355X (gfx950).

The work happens in ``libpagedattn.so`` (hand-written HIP kernels behind the
C ABI of ``include/pagedattn.h``); this package is its ctypes binding
(``_lib``), the in-tree build script (``build``) and the seeded synthetic
input generators (``synth``).  The binding loads on first use of any of its
names and raises ImportError if the library has not been built; the build
script itself imports without it.
"""
import importlib

_API = {
    "ATTN_E_ARG", "ATTN_E_DEVICE", "ATTN_E_RANGE", "ATTN_E_SHAPE", "ATTN_E_UNSUPPORTED",
    "ATTN_E_WORKSPACE", "ATTN_OK", "ATTN_PREFILL_FP8_PV", "ATTN_PREFILL_FP8_QK", "EXPORTS", "KV_BF16", "KV_FP8_E4M3", "LIB_PATH", "PAGE_SIZE",
    "VERIFY_ROWS", "AttnError", "attn_block_table_build", "attn_caps",
    "attn_check_block_table_host", "attn_check_device", "attn_check_lengths_host",
    "attn_kv_append",
    "attn_last_error", "attn_paged_decode", "attn_paged_decode_noalloc", "attn_paged_decode_window",
    "attn_paged_mixed",
    "attn_paged_prefill", "attn_paged_prefill_fp8", "attn_paged_prefill_window",
    "attn_paged_verify", "attn_paged_verify_tree", "attn_paged_verify_width",
    "attn_paged_workspace_bytes", "attn_set_kernel_timer", "attn_set_max_workgroups", "lib",
}

__all__ = sorted(_API)


def __getattr__(name):
    if name in _API:
        return getattr(importlib.import_module("._lib", __name__), name)
    raise AttributeError(name)
