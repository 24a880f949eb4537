"""CPU oracle (test infrastructure only; see sage_oracle.py's header)."""
from .sage_oracle import *  # noqa: F401,F403
from . import sage_oracle  # noqa: F401
from .sage_bwd_oracle import *  # noqa: F401,F403
from . import sage_bwd_oracle  # noqa: F401
