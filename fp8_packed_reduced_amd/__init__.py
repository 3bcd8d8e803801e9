"""Packed FP8 QKV projection with reduced-width Q/K heads, for MI355X (gfx950).

The compute path lives in the HIP library ``libfpr.so`` (sources in
``csrc/``, C interface in ``include/fpr.h``).  ``binding`` marshals torch
device tensors into its calls (pack_quantize_weights, qkv_forward,
qkv_pack_forward, qkv_backward, and the FP8 ReLU^2 MLP's mlp_* calls);
``inputs`` draws seeded synthetic data.
Importing this package does not load the library: ``binding.load()`` does,
and raises if it has not been built.
"""
