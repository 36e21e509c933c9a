"""fake_quant_amd: fake quantization of tensors on AMD MI355X (gfx950).

The product is libfq.so (HIP kernels behind the C ABI in include/fq.h); its
Python binding is ``fake_quant_amd.fq`` (imported explicitly, it fails loudly
when the library is not built).  ``fake_quant_amd.synthetic`` draws the seeded
benchmark and test inputs.
"""
