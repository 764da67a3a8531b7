"""fp64 CPU oracle of the verification step (test infrastructure only)."""
