"""CPU oracle (test infrastructure only; the product path never imports it)."""
from .emb_oracle import *  # noqa: F401,F403
