"""MI355X-native batched paged-attention decode step (placeholder until the binding lands)."""
