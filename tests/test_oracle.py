"""The fp64 oracle against what the pages and mathematics fix (CPU only)."""

import pytest

import oracle
import pins


@pytest.fixture(scope="module")
def lib():
    oracle.build()
    return oracle.load()


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(lib, pin):
    pin(lib)


def test_rejects_malformed_arguments(lib):
    import numpy as np
    q, k, v, lv, w, cu = pins.tiny_inputs(0, (4, 4), 4, 2, 2)
    with pytest.raises(ValueError):     # cu[nseq] != T
        oracle.fwd(q, k, v, *lv, 0.2, w, 1e-5, True, np.array([0, 4, 7], np.int32), lib=lib)
    with pytest.raises(ValueError):     # decreasing boundaries
        oracle.fwd(q, k, v, *lv, 0.2, w, 1e-5, True, np.array([0, 5, 4, 8], np.int32), lib=lib)
    with pytest.raises(ValueError):     # token out of range
        oracle.rows(q, k, v, *lv, 0.2, [8], [0], w, 1e-5, True, cu, lib=lib)


def test_kv_rejects_malformed_arguments(lib):
    q, k, v, lv, w, cq, ck = pins.kv_inputs(0, (3, 1), (2, 4), 2, 1, 2)
    with pytest.raises(ValueError):     # causal: 3 queries, 2 keys
        pins.run_kv(lib, q, k, v, lv, 0.2, w, 1e-5, True, cq, ck)
    q, k, v, lv, w, cq, ck = pins.kv_inputs(0, (1, 1), (0, 4), 2, 1, 2)
    with pytest.raises(ValueError):     # a query with no keys at all
        pins.run_kv(lib, q, k, v, lv, 0.2, w, 1e-5, False, cq, ck)
