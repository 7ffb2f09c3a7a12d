"""fp64 CPU oracle of the TriAttention pruning pass (test infrastructure only)."""
