"""CPU oracle for the MoE dispatch/combine path: test infrastructure only."""
