"""CPU oracle (test infrastructure only; see ``svdq_oracle``, ``mxfp4_oracle`` and ``awq_oracle``)."""
from .svdq_oracle import *  # noqa: F401,F403
from . import mxfp4_oracle as mx  # noqa: F401
from . import awq_oracle as awq  # noqa: F401
