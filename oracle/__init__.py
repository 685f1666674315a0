"""CPU reference for the attention forward path (test infrastructure only)."""
