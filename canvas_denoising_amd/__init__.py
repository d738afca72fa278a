"""canvas_denoising_amd: MI355X-native canvas-denoising step (libdg + a thin Python layer).

The compute path is the HIP library libdg.so (include/dg.h). This package
holds its ctypes binding (`_lib`), device-buffer plumbing on top of torch
(`runtime`), the benchmark configurations (`configs`) and the build script
(`build`). Importing `_lib` (and everything that uses it) fails when
libdg.so is not built; there is no fallback path.
"""
__all__ = ["build", "configs"]
