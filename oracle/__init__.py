"""CPU oracle for SOCKET decode (test infrastructure only; see socket_oracle)."""

from .socket_oracle import *  # noqa: F401,F403
from .socket_oracle import __all__  # noqa: F401
