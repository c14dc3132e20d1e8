"""fp64 CPU oracle for KDA (test infrastructure only; never used by the product path)."""
