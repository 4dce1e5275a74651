"""MI355X (gfx950) routed-expert MoE layer: C-ABI library libmoe.so and its Python binding.

Importing the package loads nothing; ``moe.lib()`` loads the built library and
raises if it is missing.
"""
from . import moe  # noqa: F401
