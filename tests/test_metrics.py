"""Host-side work/traffic counts against the memory table the course page
prints (tests/golden/table_t1_memory.txt)."""
import os

import pytest

from evoformer_attention_amd import metrics as M

GOLDEN = os.path.join(os.path.dirname(__file__), "golden",
                      "table_t1_memory.txt")


def _rows():
    with open(GOLDEN) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                n, pair, logits, ratio = line.split()
                yield int(n), float(pair), float(logits), float(ratio)


@pytest.mark.parametrize("row", list(_rows()))
def test_memory_table(row):
    n, pair_mb, logits_mb, ratio = row
    assert round(M.pair_rep_bytes(n, 128, 2) / 1e6, 1) == pair_mb
    assert round(M.triangle_logit_bytes(n, 4, 2) / 1e6, 1) == logits_mb
    assert M.triangle_logit_bytes(n, 4, 2) / M.pair_rep_bytes(n, 128, 2) == ratio


def test_flop_counts():
    # 4 * B*R*H*N^2 * C forward, 2.5x backward
    assert M.fwd_flops(1, 768, 768, 4, 32) == 4 * 768 * 4 * 768 ** 2 * 32
    assert M.bwd_flops(1, 1, 2, 1, 1) == 2.5 * 16
    # ending-node workload at N = 768: logits avoided 3.62 GB (bf16)
    assert abs(M.triangle_logit_bytes(768, 4, 2) / 1e9 - 3.62) < 0.01
