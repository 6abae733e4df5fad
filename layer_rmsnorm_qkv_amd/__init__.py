"""Fused RMSNorm -> QKV projection (+ LoRA) -> RoPE for AMD MI355X (gfx950)."""
