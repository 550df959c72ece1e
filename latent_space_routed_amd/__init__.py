"""Stable LatentMoE layer forward on MI355X (gfx950): C-ABI library liblmoe.so + thin binding."""
from . import _lib  # noqa: F401
from ._lib import LmoeError, make_shape  # noqa: F401
from .layer import LatentMoE, to_device, upload_weights  # noqa: F401
