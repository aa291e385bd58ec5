"""CPU oracle (test infrastructure only; never imported by the product path)."""
from .reference import *  # noqa: F401,F403
from .reference import __all__  # noqa: F401
