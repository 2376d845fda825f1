"""The two full 28-layer workloads at their benchmark sizes: batch 1 with a
2048-token context, and batch 16 with contexts uniform over [1024, 4096].

The oracle checks the launch configuration the benchmark times:
  * operation by operation (tests/staged.py): the embedding gather
    bit-exactly, every operation of the checked layers against its oracle
    stage fed the GPU's inputs, the final RMSNorm and every lm_head row;
    decode_step (graph) must reproduce the op-by-op logits bit for bit;
  * end to end: decode_step's logits for every vocabulary row against the
    oracle's own chain from the embedding, held to the envelope of the
    oracle's two fp16 placements (canonical and mirror).
At batch 16 the synthetic weights overflow fp16 for 9 of the 16 sequences
(on both sides, at the same elements); at layers 13 and 27 and before the
lm_head those sequences get finite stand-in rows, so every sequence's
attention over its real context and its logits are still compared.
"""
import pytest

import workloads as wl
from tests.staged import full_check

pytestmark = pytest.mark.gpu


@pytest.mark.timeout(1200)
def test_step_b1_full_size_every_layer_and_end_to_end():
    full_check(wl.step_b1(), check_layers=set(range(wl.QWEN7B.n_layers)), chains=True)


@pytest.mark.timeout(1200)
def test_step_b16_full_size_forced_rows_and_end_to_end():
    full_check(wl.step_b16(), check_layers={0, 13, 27}, force_layers={13, 27}, chains=True)
