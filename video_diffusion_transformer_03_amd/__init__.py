"""h3k: the W8A8 DiT block forward of the MiniMax-H3 denoiser on MI355X (gfx950).

The compute runs in hand-written HIP kernels behind the C ABI of libh3k.so
(include/h3k.h); `h3k` is its thin Python binding.
"""
from . import h3k  # noqa: F401
