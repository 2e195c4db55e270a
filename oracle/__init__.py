"""CPU oracle of the Token Sparse Attention prefill layer (test infrastructure only; see
``tsa_oracle``).  Nothing on the product path may import this package."""

from .tsa_oracle import *  # noqa: F401,F403
