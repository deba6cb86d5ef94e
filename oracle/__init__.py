"""CPU oracle for SQuad-Attention (test infrastructure only; see squad_oracle)."""
from .squad_oracle import *  # noqa: F401,F403
from .squad_oracle import __all__  # noqa: F401
