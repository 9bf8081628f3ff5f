"""ROCmFPX block-quantized MoE layers on MI355X (gfx950): Python binding of libqmoe.

The compute path is the HIP library ``libqmoe.so`` built from ``csrc/``; this
package only marshals arguments. See include/qmoe.h for the C ABI.
"""
from ._binding import *  # noqa: F401,F403
from ._binding import LIB, LIB_PATH, EXPORTED, QmoeError, qmoe_layer, make_layer  # noqa: F401
from . import device  # noqa: F401
