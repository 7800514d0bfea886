"""CPU oracle for the sparse MoE FFN block (test infrastructure only)."""
