"""Host checks of bench.py's reporting helpers (no GPU): the token coverage it reports for the
granularity ablation is the oracle's coverage, and the scored-candidate count is the closed form of
sum_i floor(i/B)."""
import numpy as np
import pytest
import torch

import bench
import datagen
from tests.gpu_common import bits


def test_scored_candidates_closed_form():
    for n, b, g in [(1, 8, 1), (7, 8, 2), (8, 8, 1), (9, 8, 3), (2048, 8, 1), (1000, 1, 2), (1003, 16, 4)]:
        assert bench.scored_candidates(n, b, g) == g * sum(i // b for i in range(n))


@pytest.mark.parametrize("i_min", [0, 40, 255])
def test_bench_coverage_equals_oracle(orc, i_min):
    wl = datagen.PREFILL.replace(n_tokens=256, n_q_heads=16, n_kv_heads=2)
    x = datagen.prefill_inputs(wl)
    qi, ki, w = bits(x["qi"]), bits(x["ki"]), x["w"].numpy()
    s1 = orc.index_topk(qi, w, orc.compress(ki, 1), 1, 24)
    s8 = orc.index_topk(qi, w, orc.compress(ki, 8), 8, 6)
    got = bench.token_coverage(torch, torch.from_numpy(s1), torch.from_numpy(s8), 8, i_min=i_min, rows_per_chunk=50)
    assert got == pytest.approx(orc.coverage(s1, s8, 8, i_min=i_min), abs=1e-12)
