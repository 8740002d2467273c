"""libringattn: the Ring Attention hot path on one AMD Instinct MI355X (gfx950).

The compute runs in hand-written HIP kernels behind a C ABI
(``include/ringattn.h``); this package holds those sources (``csrc/``), the
in-tree build (``build.py``) and a thin ctypes binding with the ABI's names
(``api.py``).  Importing the package does not load the library; the first
call does, and raises if ``libringattn.so`` has not been built.
"""
from .api import *  # noqa: F401,F403
from .api import Dims, RingCfg, RingAttnError  # noqa: F401
from . import overlap  # noqa: F401
