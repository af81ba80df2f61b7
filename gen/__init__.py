"""Seeded synthetic inputs for the block-quantized matrix products.

This module is shared by the tests, the benchmark and the oracle's checks.  It
only *produces inputs*: Gaussian weights and activations, the Q4_0 / Q8_0 block
encoders that turn Gaussian weights into quantized blocks (the input recipe of
the workloads), hand-chosen blocks for exact probes, and router expert ids.  It
holds none of the product's own arithmetic: no block decoding, no dot products,
no activation quantization.
"""
from .inputs import *  # noqa: F401,F403
