"""The full-size comparison helper (row blocks of the oracle on threads, over
a compact one-request pool) gives exactly what one plain oracle call over the
workload's own shuffled pool gives."""
import numpy as np
import pytest

import workloads as wl
from pkv_testlib import compact_request, oracle_out, oracle_pools, oracle_rows_parallel


@pytest.mark.parametrize("window", [0, 37])
def test_parallel_rows_equal_one_oracle_call(window):
    P = np.array([40, 0, 300], np.int32)
    L = np.array([70, 5, 33], np.int32)
    pt = wl.shuffled_page_table(71, 64, P + L, 16)
    w = wl.Workload("par", 71, "bf16", 8, 2, 64, 16, 64, window, P, L, pt)
    ref = oracle_out(w, oracle_pools(w))
    qo = np.concatenate([[0], np.cumsum(L)])
    for b in range(w.batch):
        got = oracle_rows_parallel(w, b, block=7)
        assert np.array_equal(got, ref[qo[b]:qo[b + 1]])
        rows = [0, int(L[b]) - 1]
        assert np.array_equal(oracle_rows_parallel(w, b, rows), ref[qo[b] + np.array(rows)])


def test_compact_pool_holds_the_sequence_in_order():
    P, L = np.array([21], np.int32), np.array([6], np.int32)
    w = wl.Workload("c", 72, "bf16", 4, 2, 64, 8, 16, 0, P, L, wl.shuffled_page_table(72, 16, P + L, 8))
    one, (kp, vp) = compact_request(w, 0)
    k, v = w.kv_seq(0, storage=True)
    assert np.array_equal(kp.reshape(-1, 2, 64)[:27], k) and np.array_equal(vp.reshape(-1, 2, 64)[:27], v)
    assert (kp.reshape(-1, 2, 64)[27:] == wl.nan_fill("bf16")).all()
    assert one.page_table.tolist() == [[0, 1, 2, 3]]
