"""MI355X-native Looped Latent Attention (LLA) latent-cache kernels."""
