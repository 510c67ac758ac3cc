"""Prefill-only decision library for AMD MI355X (gfx950).

The compute path lives in the HIP library libs1.so (C ABI in include/s1.h);
`binding` is its ctypes marshalling layer and `build` compiles it in-tree.
"""
from . import binding  # noqa: F401
from .binding import (Model, Plan, S1Error, load_library, make_batch, make_config,  # noqa: F401
                      validate, DECISION_DTYPE)
