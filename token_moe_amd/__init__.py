"""MI355X-native TokenMixer-Large block-stack forward.

The compute lives in ``libtmx.so`` (hand-written HIP for gfx950, C ABI in
``include/tmx.h``); this package is a thin ctypes binding over it. There is
no CPU fallback: importing :mod:`token_moe_amd.tmx` fails loudly if the
library has not been built (``python -m token_moe_amd.build``).
"""

__all__ = ["tmx"]
