"""fp64 CPU oracle (test infrastructure only; never on the product path)."""
from .gist_oracle import *  # noqa: F401,F403
