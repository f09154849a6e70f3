"""MI355X-native tiled-matmul hot path: dense Y = X W^T and causal attention scores."""
