"""CPU oracle for the SharQ linear layer (test infrastructure only)."""
