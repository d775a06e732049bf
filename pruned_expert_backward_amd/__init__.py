"""MI355X-native pruned MoE expert backward (LRMoE score, select, compact,
varlen grouped GEMM) behind a C-ABI library; see ``lrmoe`` for the binding."""
