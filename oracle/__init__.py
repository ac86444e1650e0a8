"""CPU oracle of the routed WNA16 MoE layer (test infrastructure only)."""
