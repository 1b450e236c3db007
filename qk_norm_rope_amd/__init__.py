"""qk_norm_rope_amd: paged QK-norm + RoPE + GQA attention for MI355X (gfx950).

The kernels live in libqknr.so (built from csrc/ by ``python -m
qk_norm_rope_amd.build``) behind the C ABI of include/qknr.h; this package is a
thin ctypes binding with the same names. The library is loaded on first use of
any binding name, so the build module imports without it; a missing library
raises ImportError there.
"""
_NAMES = (
    "EXPORTED", "LIB_PATH", "QKR_EDATA", "check_indices", "QKR_BF16", "QKR_F32", "QknrError", "decode_workspace_bytes", "decode_kernel_name",
    "last_error", "mfma_probe", "packed_prefill_attn", "packed_workspace_bytes", "paged_decode_attn", "paged_decode_attn_noalloc",
    "paged_prefill_attn", "pool_desc", "prefill_workspace_bytes",
    "qknorm_rope_append", "read_probe", "rope_table", "status_str", "step_paged", "step_workspace_bytes", "version",
)


def __getattr__(name):
    if name in _NAMES:
        from . import _lib
        return getattr(_lib, name)
    raise AttributeError(name)


def __dir__():
    return sorted(list(globals()) + list(_NAMES))
