"""Persistent decode megakernel for AMD Instinct MI355X (gfx950).

The product is libpmk.so (hand-written HIP behind the C ABI of include/pmk.h);
this package only builds it (``build``) and binds it (``_abi``, ``model``).
"""
from ._abi import EXPORTS, PmkError, load  # noqa: F401
from .model import DecodeModel  # noqa: F401
