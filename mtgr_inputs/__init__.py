"""Seeded synthetic inputs for the MTGR HSTU layer.

This package only draws random numbers and lays them out (jagged offsets,
token-group ids, timestamps, activations, weights).  It holds none of the
layer's arithmetic, so that both the CPU oracle and the HIP path can take
their inputs from it without sharing any part of the computation.
"""

from .synth import (  # noqa: F401
    CONFIGS,
    GROUP_U,
    GROUP_S,
    GROUP_R,
    GROUP_C,
    Batch,
    LayerParams,
    make_batch,
    make_batch_from_lengths,
    make_layer_params,
    make_activations,
    make_probe_head,
    config_inputs,
    make_user_pool,
    make_uniform_draws,
    HeadParams,
    make_head_params,
    make_labels,
    NUM_GROUPS,
)
