"""CPU oracle for the GPT-2 training step (test infrastructure only; see gpt2_oracle)."""
from .gpt2_oracle import *  # noqa: F401,F403
from . import gpt2_oracle  # noqa: F401
