"""The OpenMP CSR baseline the benchmark times beside the oracle: it must
compute the same y as the oracle (both sum each row in fp64 in row order), so
the reported CPU throughput is for a correct SpMV."""
import numpy as np
import pytest

import oracle
from spmv_storage_formats_amd import synth


@pytest.mark.parametrize("name", ["fig14_1", "c1s", "c2s", "c4s", "c5s"])
def test_openmp_csr_equals_oracle(name):
    w = synth.workload(name)
    y_omp = oracle.spmv_csr_omp(w.row_ptrs, w.col_idx, w.values, w.x, w.y)
    y_ref, _ = oracle.spmv_csr(w.row_ptrs, w.col_idx, w.values, w.x, w.y)
    assert np.array_equal(y_omp.view(np.uint32), y_ref.astype(np.float32).view(np.uint32))


def test_openmp_thread_count_positive():
    assert oracle.omp_threads() >= 1
