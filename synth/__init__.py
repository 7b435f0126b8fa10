"""Seeded synthetic inputs for the routed-expert MoE FFN (shared by the tests, the
benchmark and the smoke check).

This package draws random numbers and lays them out as the inputs the MoE layer
takes: bf16 activations and router weights, packed expert weight bytes, fp16 and
UE8M0 block-scale bytes, per-expert logit biases and logits.  It holds none of the
layer's arithmetic (no decoding, routing, matrix products or quantisation rules):
both the CPU oracle and the GPU path consume what it returns, each with its own
code.
"""
from .gen import *  # noqa: F401,F403
