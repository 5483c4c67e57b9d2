"""Seeded synthetic inputs for the Whisper hot path.

This package holds model shapes and seeded random draws only: no step of
the log-mel, encoder or decoder arithmetic lives here. Both the oracle
tests and the GPU tests/bench read their inputs from here, so the two sides
see the same numbers.
"""
from .configs import Dims, CONFIGS, get_config  # noqa: F401
from .gen import (  # noqa: F401
    rng_for, round_to_bf16, weight_specs, gen_weight, gen_weights,
    gen_audio_tones, gen_audio_longform, gen_tokens, gen_prefill_lengths,
    gen_prefill_kv, gen_normal,
)
