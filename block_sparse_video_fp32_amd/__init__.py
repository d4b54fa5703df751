"""Routed block-sparse attention (Sol-style) for AMD Instinct MI355X (gfx950).

The compute path is the C-ABI library ``libsparse_attn.so`` (HIP kernels for
gfx950); :mod:`block_sparse_video_fp32_amd.binding` marshals torch tensors
into it.  The library is loaded on first use and its absence is an error:
there is no fallback path.
"""

__all__ = ["sparse_attn", "SparseAttnPlan", "load_library"]


def __getattr__(name):
    if name in __all__:
        from . import binding

        return getattr(binding, name)
    raise AttributeError(name)
