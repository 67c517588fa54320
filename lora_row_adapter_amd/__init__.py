"""Multi-adapter LoRA linear layer for AMD MI355X (gfx950)."""
