"""CPU oracle of the MoE expert-FFN layer. Test infrastructure only."""
