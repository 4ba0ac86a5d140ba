"""CPU oracle of the LSA hot path: test infrastructure only (see lsa_oracle)."""
from .lsa_oracle import *  # noqa: F401,F403
from .lsa_oracle import INT32_MIN  # noqa: F401
