"""GenRank ranking hot path on MI355X (gfx950): HIP kernels behind a C ABI.

``binding`` mirrors the C entry points one to one; ``device`` uploads host arrays;
``model.GenRank`` chains the entry points into embed -> blocks -> head (forward) and the
matching backward.  Nothing here computes on the CPU: if ``libgenrank.so`` is missing the
calls raise.
"""
from . import binding  # noqa: F401
from .slopes import alibi_slopes  # noqa: F401

__all__ = ["binding", "alibi_slopes"]
