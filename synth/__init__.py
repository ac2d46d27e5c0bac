"""Seeded synthetic inputs for the VGG-T^3 test-time-training layer.

This package only draws random numbers and lays them out in the token order the
layer expects; it holds none of the layer's arithmetic. Both the CPU oracle
(through the tests) and the HIP path are fed from it.
"""
from .gen import LayerConfig, CONFIGS, LayerInputs, make_inputs, view_token_count  # noqa: F401
