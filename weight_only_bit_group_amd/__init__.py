"""weight_only_bit_group_amd -- group-wise INT4 (W4A16), AWQ calibration and FP4 decode on MI355X.

The compute lives in libaq.so (hand-written HIP kernels for gfx950 behind the C
ABI of include/aq.h).  ``binding`` exposes the entry points to torch under the
same names; ``layer`` builds on it the quantized linear module and the
norm-group AWQ apply step; ``synth`` holds the seeded synthetic inputs.  Importing this package
does not load the library; the first binding call does, and fails loudly if it
has not been built.
"""

__all__ = ["aq_quantize_pack", "aq_w4a16_gemv", "aq_w4a16_gemm", "aq_w4a16_gemm_workspace", "aq_act_absmean",
           "aq_act_absmean_workspace", "aq_awq_search", "aq_awq_search_workspace", "aq_fp4_gemm",
           "aq_fp4_gemm_workspace", "aq_fp4_quantize", "aq_fp4_quantize_workspace", "aq_quantize_pack8",
           "aq_w8a16_gemv", "aq_w8a16_gemm", "aq_w8a16_gemm_workspace"]


def __getattr__(name):
    if name in __all__:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
