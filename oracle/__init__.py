"""CPU oracle for the MoE layer forward: test infrastructure, not part of the product path."""
