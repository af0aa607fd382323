"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This package only draws inputs (lengths, page tables, bf16/fp8 tensors, the
angle tables a rotary-embedding caller supplies). It
holds none of the attention method's arithmetic: no append, no de-paging, no
softmax. Both the CPU oracle and the GPU path consume what it produces.
"""
from .workloads import WORKLOADS, Workload, make_workload, make_custom, rope_tables, subset  # noqa: F401
