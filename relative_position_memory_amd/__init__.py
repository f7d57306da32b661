"""Transformer-XL relative-position attention over segment-level memory, on MI355X.

The compute path is libtxl.so (hand-written HIP kernels for gfx950 behind a C
ABI, declared in include/txl.h).  `relative_position_memory_amd.txl` is its thin
ctypes binding; `relative_position_memory_amd.inputs` draws seeded synthetic
inputs.  Importing this package loads nothing; importing `.txl` loads the
library and fails loudly if it has not been built.
"""
