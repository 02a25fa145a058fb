"""MI355X-native blocked local self-attention with haloing (HaloNet forward)."""
