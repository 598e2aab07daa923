"""MI355X-native prefill sparse-MoE layer with in-GEMM 4-bit dequant."""
