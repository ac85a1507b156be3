"""The five workloads at full size: GPU path vs oracle on every request,
seed 0 of each and three more seeds of each large workload.

Near-ties (values within 1e-4 of a selection cutoff) are tolerated on a few
requests of the large workloads (the single request of the Qwen3-4B and
wide-tree rounds included); see checker.py.
"""
import pytest

import synth
from gpu_util import check_config

pytestmark = pytest.mark.gpu


_TIES = {"tiny": 0.0, "qwen3_4b": 1.0, "wide": 1.0, "qwen3_8b_x8": 0.25, "stress_b0": 0.25,
         "stress_b01": 0.25}
# seed 0 of every workload, plus three more seeds of each large one
_CASES = [(n, 0) for n in _TIES] + [(n, sd) for n in _TIES if n != "tiny" for sd in (1, 2, 3)]


@pytest.mark.parametrize("name,seed", _CASES)
def test_config_full_size(gpu_lib, name, seed):
    cfg = synth.CONFIGS[name]
    check_config(synth.make_inputs(cfg, seed), cfg, f"{name} seed {seed}",
                 max_tie_frac=_TIES[name])
