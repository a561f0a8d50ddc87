"""MI355X-native canvas denoise step of block text diffusion (DiffusionGemma
style): libcd (HIP kernels for gfx950 behind a C ABI, include/cd.h) and its
thin Python binding."""
from . import binding  # noqa: F401
