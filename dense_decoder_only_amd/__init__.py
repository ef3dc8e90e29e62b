"""Llama-3/3.1 dense decoder block on MI355X (gfx950): HIP kernels behind a C ABI.

The library (include/llb.h, built by dense_decoder_only_amd.build into
dense_decoder_only_amd/_lib/libllb.so) does all compute; `llb` is its ctypes
binding.  Importing the package does not load the library; the first call does.
"""
from . import llb  # noqa: F401
