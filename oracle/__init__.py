"""CPU oracle package (test infrastructure only; see ``lrq_oracle``)."""
from .lrq_oracle import *  # noqa: F401,F403
from .lrq_oracle import Spec, forward, backward, rel_frobenius  # noqa: F401
