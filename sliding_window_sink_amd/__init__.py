"""MI355X (gfx950) sink attention: HIP kernels behind a C ABI, bound with ctypes."""
