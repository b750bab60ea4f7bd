"""fp64 CPU oracle for causal GQA with QK-RMSNorm + RoPE.

TEST INFRASTRUCTURE: importable only by the tests, the graft entry smoke check and the CPU
baseline leg of the benchmark. The HIP library and its binding never import it.
"""
from . import brute, gqa_oracle  # noqa: F401
