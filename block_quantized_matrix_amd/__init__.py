"""Block-quantized (Q4_0 / Q8_0) matrix products on AMD MI355X (gfx950).

The compute path is the HIP library libbqm.so (C ABI in include/bqm.h); ``bqm`` is
its thin binding.  Build with ``__graft_entry__.build()`` or
``python -m block_quantized_matrix_amd._build``.
"""
from . import bqm  # noqa: F401
