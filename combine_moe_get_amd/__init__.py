"""MI355X-native MoE expert-parallel dispatch and combine (placeholder, binding follows)."""
