"""MI355X-native chunkwise forward of key-only gated linear attention (GTR)."""
