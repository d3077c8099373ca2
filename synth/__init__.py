"""Seeded synthetic inputs shared by the oracle tests and the HIP path.

This package only draws random numbers and lays them out; it contains none of
the attention method's arithmetic (no permutation, masking, pooling, routing,
quantisation or softmax).
"""
from .workloads import CONFIGS, Workload, make_grad, make_qkv, round_to_bf16, bf16_bits

__all__ = ["CONFIGS", "Workload", "make_grad", "make_qkv", "round_to_bf16", "bf16_bits"]
