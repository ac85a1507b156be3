"""Seeded synthetic inputs for draft-tree rounds.

This module holds workload shapes and random-number plumbing only: it draws
weights, hidden states and root tokens from fixed seeds and never computes
any step of the tree-construction method.  Both the CPU oracle's tests and
the GPU path's tests and benchmark take their inputs from here, so the two
sides always see identical values.
"""
from .configs import CONFIGS, Config, config_by_name  # noqa: F401
from .inputs import make_inputs, custom_config  # noqa: F401
from .attn import ATTN_CONFIGS, AttnConfig, make_attn_inputs, random_parents  # noqa: F401
