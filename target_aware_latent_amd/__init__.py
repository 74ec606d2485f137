"""MI355X (gfx950) implementation of the LLaTTE target-aware MLA sequence
transformer forward pass: a C-ABI HIP library (libllatte.so, declared in
include/llatte.h) and this thin Python binding."""
from . import llatte  # noqa: F401

__all__ = ["llatte"]
