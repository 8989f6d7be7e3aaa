"""MI355X-native routed-expert epilogue (clamped SwiGLU x probs, fp32 router-weight multiply)."""
