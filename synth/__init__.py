"""Seeded synthetic inputs for the MoE layer workloads.

This package only draws random numbers and lays them out; it holds none of the
layer's arithmetic (no routing, quantisation, matrix products or activations).
Both the CPU oracle and the GPU library consume what it produces.
"""
from .workloads import *  # noqa: F401,F403
