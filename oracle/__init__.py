"""CPU oracle (test infrastructure only; never imported by the product path)."""
from .spa_oracle import *  # noqa: F401,F403
from .spa_oracle import INT32_MIN  # noqa: F401
