"""The benchmark workloads' seeded operands are the recorded bytes:
tests/golden/workload_sha256.txt (written by make_workload_sha256.py next to
it, from the input generator alone) holds the SHA-256 of each workload's A and
B as binary16, so a change of generator, seed or rounding shows up here."""
import os

import numpy as np
import pytest

from dense_tiled_gemm_tgemm_amd import inputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "workload_sha256.txt")


def _recorded():
    rows = {}
    with open(GOLDEN) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            name, ha, hb = line.split()
            rows[name] = (ha, hb)
    return rows


def test_every_workload_is_recorded():
    assert set(_recorded()) == set(inputs.WORKLOADS)


@pytest.mark.parametrize("name", sorted(inputs.WORKLOADS))
def test_workload_operands_match_recorded_bytes(name):
    A, B = inputs.make_inputs(inputs.WORKLOADS[name])
    assert A.dtype == np.float16 and B.dtype == np.float16
    assert (inputs.sha256(A), inputs.sha256(B)) == _recorded()[name], f"numpy {np.__version__}"
