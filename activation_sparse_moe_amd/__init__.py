"""BlockFFN layer forward on MI355X (gfx950): C-ABI library + thin binding.

The HIP kernels and the C ABI live in ``csrc/`` and ``include/blockffn.h``;
``binding`` exposes the same entry points to Python with torch tensors for
device memory and streams.  The library is loaded on first use and there is
no CPU fallback.
"""
from ._capi import (BF16, EXPORTS, F32, MODES, BlockFFNError, BlockffnLayer, BlockffnStats, load)

__all__ = ["BF16", "F32", "MODES", "EXPORTS", "BlockFFNError", "BlockffnLayer", "BlockffnStats", "load"]
