"""CPU oracle for the QSA decode path (test infrastructure only; see qsa_oracle)."""
from .qsa_oracle import *  # noqa: F401,F403
