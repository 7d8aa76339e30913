"""Seeded synthetic inputs for sink attention.

This module is the only code shared by the oracle side and the HIP side.
It draws random numbers and lays them out; it holds none of the attention
arithmetic.  Every workload is a stand-in for GPT-OSS-20B attention shapes
(the model named in "GPT-OSS Agentic RL Training: A Practical
Retrospective", section "Agentic RL and GPT-OSS").
"""
from .workloads import WORKLOADS, Workload, make_inputs, workload  # noqa: F401
