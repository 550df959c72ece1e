"""CPU oracle of the Stable LatentMoE forward pass (test infrastructure only; see lmoe_oracle)."""
