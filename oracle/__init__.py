"""CPU oracle (test infrastructure only; see ``svdq_oracle``)."""
from .svdq_oracle import *  # noqa: F401,F403
