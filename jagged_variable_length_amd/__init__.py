"""jagged_variable_length_amd: jagged (unpadded, variable-length) attention,
forward and backward, as hand-written HIP kernels for AMD MI355X (gfx950).

* ``binding``   -- ctypes binding of libjattn.so (the C ABI in include/jattn.h)
* ``attention`` -- JaggedAttention: plan + workspace + torch tensors
* ``inputs``    -- seeded synthetic jagged inputs
* ``build``     -- compiles libjattn.so in-tree with hipcc for gfx950

The library is loaded lazily on first use; if it has not been built, the
first call raises (there is no CPU fallback).
"""
