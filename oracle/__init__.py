"""fp64 CPU oracle for the routed LoRA delta (test infrastructure only)."""
