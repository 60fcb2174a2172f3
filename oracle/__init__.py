"""fp64 CPU oracle (test infrastructure only; never used by the product path)."""
