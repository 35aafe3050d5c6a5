"""CPU oracle (test infrastructure only): see qlora_oracle.py."""
from .qlora_oracle import *  # noqa: F401,F403
