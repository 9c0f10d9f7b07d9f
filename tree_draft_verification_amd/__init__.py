"""EAGLE-3 draft-tree verification on AMD Instinct MI355X (gfx950).

The compute lives in libeagle3.so (HIP kernels behind the C ABI declared in
include/eagle3.h); ``binding`` wraps each entry point with the same name and
``verify`` strings the calls of one verify step together on one stream and
``draft`` those of the EAGLE-3 draft head and its tree growth, ``target``
those of the target model's own decoder layers over the trees, ``loop`` the
device-resident speculative decoding step built from both.
"""
from . import binding  # noqa: F401  (raises ImportError when the library is missing)
from .binding import *  # noqa: F401,F403
from .verify import VerifyStep  # noqa: F401
from .draft import DraftHead  # noqa: F401
from .target import TargetModel  # noqa: F401
from .loop import SpecLoop  # noqa: F401
