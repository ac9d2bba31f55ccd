"""The fp64 oracle against what the pages and mathematics fix (CPU only)."""
import pytest

import oracle as O
from tests import _pins


@pytest.fixture(scope="module")
def lib():
    return O.load()


@pytest.mark.parametrize("check", _pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_pin(check, lib):
    check(lib)


def test_oracle_threads_do_not_change_results(lib):
    from paged_kv_cache_161_amd import workloads as W
    w = W.build(_pins.small_specs()[1])
    kp, vp = _pins.appended(w, lib)
    a, _ = O.decode_paged(w.q, kp, vp, w.dtype, w.block_tables, w.context_lens, w.scale,
                          threads=1, lib=lib)
    b, _ = O.decode_paged(w.q, kp, vp, w.dtype, w.block_tables, w.context_lens, w.scale,
                          threads=5, lib=lib)
    assert a.tobytes() == b.tobytes()


def test_oracle_rejects_out_of_range_table(lib):
    import numpy as np
    from paged_kv_cache_161_amd import workloads as W
    w = W.build(_pins.small_specs()[1])
    kp, vp = w.host_pools()
    bt = w.block_tables.copy()
    bt[2, 0] = w.num_blocks
    with pytest.raises(ValueError):
        O.decode_paged(w.q, kp, vp, w.dtype, bt, w.context_lens, w.scale, lib=lib)
