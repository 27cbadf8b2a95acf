"""MI355X-native causal grouped-query attention with RoPE (placeholder)."""
