"""MI355X-native MoE expert-FFN layer with int4 experts and a sigmoid router.

The compute path is libcoli_moe.so (hand-written HIP for gfx950) behind the C
ABI in include/coli_moe.h; this package is its Python binding.
"""
from ._lib import (COLI_ACCUMULATE, COLI_EDEVICE, COLI_EINVAL, COLI_EUNSUPPORTED, COLI_EWORKSPACE,
                   COLI_GEMV_MAX_T, COLI_MAX_T, COLI_MAX_TOPK, COLI_OK, COLI_PATH_GEMV, COLI_PATH_GROUPED,
                   EXPORTS, ColiError, LIB_PATH)

__all__ = ["COLI_ACCUMULATE", "COLI_PATH_GEMV", "COLI_PATH_GROUPED", "ColiError", "LIB_PATH", "EXPORTS"]
