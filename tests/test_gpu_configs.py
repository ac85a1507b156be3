"""The five workloads at full size: GPU path vs oracle on every request.

Near-ties (values within 1e-4 of a selection cutoff) are tolerated on a few
requests of the large batched workloads; see checker.py.
"""
import pytest

import synth
from gpu_util import check_config

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,max_tie", [("tiny", 0.0), ("qwen3_4b", 0.0), ("wide", 1.0),
                                          ("qwen3_8b_x8", 0.25), ("stress_b0", 0.25),
                                          ("stress_b01", 0.25)])
def test_config_full_size(gpu_lib, name, max_tie):
    cfg = synth.CONFIGS[name]
    check_config(synth.make_inputs(cfg, 0), cfg, name, max_tie_frac=max_tie)
