"""Seeded synthetic inputs for one MoE layer forward.

This package is shared by the HIP path's tests/bench and by the oracle's
tests.  It only *draws* inputs (tokens, router weights, quantised expert
weights); it holds none of the layer's arithmetic (routing, permutation,
activation quantisation, FFN, combine).  Weight quantisation to FP8 happens
here because the layer consumes already-quantised weights, the way the
DSV2-236B-MegaKernel README ("Layout": the block-FP8 quantiser) quantises a
checkpoint offline before any forward pass.
"""
from .configs import CONFIGS, LayerConfig, get_config, with_norm  # noqa: F401
from .generate import LayerInputs, ExpertWeights, make_inputs, make_experts, redraw_tokens, draw_tokens  # noqa: F401
