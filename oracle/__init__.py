"""CPU oracle (test infrastructure only): see msa_oracle.py."""
from .msa_oracle import *  # noqa: F401,F403
