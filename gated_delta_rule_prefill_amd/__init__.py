"""MI355X-native Kimi Delta Attention (KDA) prefill and decode."""
