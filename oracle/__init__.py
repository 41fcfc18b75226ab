"""CPU oracle (test infrastructure only; see ``svdq_oracle`` and ``mxfp4_oracle``)."""
from .svdq_oracle import *  # noqa: F401,F403
from . import mxfp4_oracle as mx  # noqa: F401
