"""augmentation_amd -- FusedNormalization on AMD Instinct MI355X (gfx950).

One pass over a batch of uint8 NHWC images produces per-channel normalized
(x/255 - mean)/std tensors in fp32 or fp16, with a per-sample random
horizontal flip and a per-sample RandomErasing rectangle applied in the
same pass (page "(11) FusedNormalization", tech-renaissance.cn/blog/?p=487).

The work runs in the hand-written HIP kernels of ``libfn.so`` (built from
``csrc/``).  ``augmentation_amd.binding`` exposes the library's C entry
points under the same names; importing one of them from this package
loads the library and raises if it has not been built.  ``synth`` (seeded
synthetic inputs) needs no GPU library.
"""
_BINDING_NAMES = (
    "fn_params", "fn_params_ex", "fn_fused_normalize", "fn_fused_normalize_ex", "fn_last_error",
    "fn_test_erase_dims", "fn_test_cr_ops", "fn_test_stream", "FnError", "PARAMS_DTYPE",
    "FN_OUT_FP32", "FN_OUT_FP16", "FN_OUT_FP16_PAD4", "fused_normalize", "sample_params",
)


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(f"module 'augmentation_amd' has no attribute {name!r}")
