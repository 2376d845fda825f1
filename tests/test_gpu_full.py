"""The two full 28-layer workloads at their benchmark sizes: batch 1 with a
2048-token context, and batch 16 with contexts uniform over [1024, 4096].

The oracle checks the launch configuration the benchmark times, operation by
operation: the embedding gather bit-exactly, every operation of a sample of
layers against its oracle stage (the GPU's inputs fed in), and the final
RMSNorm + fp16 lm_head on a sample of vocabulary rows. Layers between the
sampled ones run on the GPU only. The full step through decode_step must
reproduce the op-by-op result bit for bit (same kernels, same order)."""
import pytest

import workloads as wl
from tests.staged import full_check

pytestmark = pytest.mark.gpu


def test_step_b1_full_size():
    full_check(wl.step_b1(), check_layers={0, 13, 27})


def test_step_b16_full_size():
    full_check(wl.step_b16(), check_layers={0, 27}, n_rows=1024)
