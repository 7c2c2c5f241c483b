"""SmolVLA action-expert denoising loop on AMD MI355X (gfx950).

The work is done by libsmolexp.so (hand-written HIP kernels behind a C ABI,
include/smolexp.h); this package is its ctypes binding.  Importing it fails
if the library has not been built.
"""
from ._binding import *  # noqa: F401,F403
from ._binding import (  # noqa: F401
    LIB_PATH, EXPORTED, SmolexpError, raw,
    K_QKV, K_ATTN_SELF, K_ATTN_CROSS, K_O, K_GATE_UP, K_DOWN, K_ACTION_OUT, K_WHOLE_LOOP, K_Q_CROSS, K_TIME_IN,
    K_TIME_OUT,
)
