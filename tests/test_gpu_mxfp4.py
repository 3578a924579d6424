"""MXFP4 matrices on the GPU (E2M1 codes + an E8M0 scale per block of 32, MK_WEIGHTS_MXFP4) against the
oracle over the same packed rows (``oracle.mxfp4``: the step over the dequantized weights), with the gates of
the bf16 parity tests:

* the small model: 16 free-running greedy steps at batch 1; three ragged sequences for 8 steps; both
  with the K/V replay of ``run_steps`` (this model's greedy run repeats one token from its third
  step on, and a value of that token's V row lies on a bf16 rounding boundary: the oracle's own
  fp32 and fp64 runs differ by 1.2e-5 in the router logits at step 5 and 3.8e-5 at step 15 through
  the cache, against 1e-7 for the bf16 and FP8 models);
* the 48-layer model at batch 1 (two steps checked) and at batch 8 (first step), in the launch
  configuration bench.py times.
The prefill of the MXFP4 model (the chunked kernel instance) is in test_gpu_prefill.py.
"""

import sys

import pytest
import torch

from decode_megakernel_03_amd import synth
from tests import harness

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900),
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def test_tiny_mxfp4_free_running_16_steps():
    from tests.test_gpu_parity import run_steps
    say("test_tiny_mxfp4_free_running_16_steps")
    stats = run_steps(synth.workload("tiny_mxfp4"), 16, gains="uniform", kv_replay=True)
    say(f"  max |dlogit| per step: {[round(s[0], 7) for s in stats]}")


def test_tiny_mxfp4_batch3_ragged():
    from tests.test_gpu_parity import run_steps
    say("test_tiny_mxfp4_batch3_ragged")
    run_steps(synth.workload("tiny_mxfp4", batch=3), 8, gains="uniform", ctx=[5, 60, 17], kv_replay=True)


def test_full_mxfp4_batch1_8k():
    from tests.test_gpu_full import Model
    say("test_full_mxfp4_batch1_8k")
    m = Model(synth.workload("full_mxfp4"), steps=2)
    try:
        for s in range(2):
            m.step_and_check()
    finally:
        m.close()


def test_full_mxfp4_batch8_8k():
    from tests.test_gpu_full import Model
    say("test_full_mxfp4_batch8_8k")
    m = Model(synth.workload("full_b8_mxfp4"), steps=1)
    try:
        m.step_and_check()
    finally:
        m.close()
