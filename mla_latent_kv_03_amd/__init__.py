"""Weight-absorbed MLA decode for MI355X (gfx950): HIP kernels behind a C ABI.

The entry points mirror include/mla_decode.h and live in ``binding``:
``mla_decode_fwd``, ``mla_decode_splitkv_combine``, ``mla_paged_cache_append``,
``mla_decode_workspace_size`` and ``mla_decode_num_splits``.  They are loaded on
first use; a missing or incomplete libmla_decode.so raises ImportError.
``workloads`` holds the seeded synthetic inputs.
"""
_EXPORTS = ("mla_decode_fwd", "mla_decode_splitkv_combine", "mla_paged_cache_append",
            "mla_decode_workspace_size", "mla_decode_num_splits", "mla_decode_fwd_append", "mla_set_attention_events", "params_for", "make_params",
            "workspace_views", "MLAError")


def __getattr__(name):
    if name in _EXPORTS:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
