"""fp64 CPU oracle (test infrastructure only; never imported by the product path)."""
from . import brute, twinkv_oracle

__all__ = ["brute", "twinkv_oracle"]
