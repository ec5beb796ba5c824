"""MI355X-native MoE route / INT8 dispatch / INT8 SwiGLU experts / combine."""
