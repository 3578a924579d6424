"""FP8 matrices on the GPU (E4M3 codes + a float32 scale per row, MK_WEIGHTS_FP8) against the oracle
over the same packed rows (``oracle.fp8``: the step over the dequantized weights), with the gates of
the bf16 parity tests:

* the small model: 16 free-running greedy steps at batch 1; three ragged sequences for 8 steps;
* the 48-layer model at batch 1 (two steps checked) and at batch 8 (first step), in the launch
  configuration bench.py times.
The prefill of the FP8 model (the chunked kernel instance) is in test_gpu_prefill.py.
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


def test_tiny_fp8_free_running_16_steps():
    from tests.test_gpu_parity import run_steps
    say("test_tiny_fp8_free_running_16_steps")
    stats = run_steps(synth.workload("tiny_fp8"), 16, gains="uniform")
    say(f"  max |dlogit| per step: {[round(s[0], 7) for s in stats]}")


def test_tiny_fp8_batch3_ragged():
    from tests.test_gpu_parity import run_steps
    say("test_tiny_fp8_batch3_ragged")
    run_steps(synth.workload("tiny_fp8", batch=3), 8, gains="uniform", ctx=[5, 60, 17])


def test_full_fp8_batch1_8k():
    from tests.test_gpu_full import Model
    say("test_full_fp8_batch1_8k")
    m = Model(synth.workload("full_fp8"), steps=2)
    try:
        for s in range(2):
            m.step_and_check()
    finally:
        m.close()


def test_full_fp8_batch8_8k():
    from tests.test_gpu_full import Model
    say("test_full_fp8_batch8_8k")
    m = Model(synth.workload("full_b8_fp8"), steps=1)
    try:
        m.step_and_check()
    finally:
        m.close()
