"""Seeded synthetic inputs for the DFlash draft step.

This package draws weights, verifier hidden states, anchors, target tokens and
the logit rows of the sampling stage from fixed seeds, and converts them to the
storage dtype.  It holds none of the method's arithmetic: both the CPU oracle
(tests only) and the HIP path receive exactly the arrays produced here.
"""
from .configs import CONFIGS, Dims, Workload, get_config  # noqa: F401
from .gen import (  # noqa: F401
    as_f32,
    bf16_bits_to_f32,
    conv_weights_as_f32,
    f32_to_bf16_bits,
    draw_accepted,
    make_anchors,
    make_conv_weights,
    make_hidden,
    make_relay_weights,
    make_sampling_logits,
    make_selector_weights,
    make_suffix_hidden,
    make_targets,
    make_weights,
    draw_first_mismatch,
    weights_as_f32,
)
