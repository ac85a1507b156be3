"""The five workloads at full size: GPU path vs oracle on every request,
seed 0 of each and three more seeds of each large workload.

Every request is compared with the oracle to its last node (checker.py).
Where the GPU kept a different set at a selection, that set must be an
admissible alternative of the oracle's own decision (its values within
1e-4 of the cutoff), and the oracle then builds the rest of the tree along
it; at most two such tolerated ties per request are accepted.
"""
import pytest

import synth
from gpu_util import check_config

pytestmark = pytest.mark.gpu

_NAMES = ("tiny", "qwen3_4b", "wide", "qwen3_8b_x8", "stress_b0", "stress_b01")
# seed 0 of every workload, plus three more seeds of each large one
_CASES = [(n, 0) for n in _NAMES] + [(n, sd) for n in _NAMES if n != "tiny" for sd in (1, 2, 3)]


@pytest.mark.parametrize("name,seed", _CASES)
def test_config_full_size(gpu_lib, name, seed):
    cfg = synth.CONFIGS[name]
    check_config(synth.make_inputs(cfg, seed), cfg, f"{name} seed {seed}",
                 max_ties_per_request=0 if name == "tiny" else 2, seed=seed)
