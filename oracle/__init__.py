"""CPU oracle (test infrastructure only; see ``tp_oracle``)."""
from .tp_oracle import *  # noqa: F401,F403
