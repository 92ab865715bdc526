"""CPU oracle of the sparse MoE block forward (test infrastructure only)."""
