"""MI355X-native causal sliding-window attention with a fused RoPE + RMS QK-norm prologue."""
