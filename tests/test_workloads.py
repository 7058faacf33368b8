"""Seeded generators: reproducible and shaped like the pages' workloads (CPU)."""
import numpy as np

import workloads
from tests.checks import as_f64


def test_same_seed_same_digest():
    for num in (1, 2, 3, 4, 5):
        shape = {1: {}, 2: {"batch": 3}, 3: {"batch": 3}, 4: {"batch": 64, "n_cols": 4096},
                 5: {"batch": 1, "n_cols": 1 << 16}}[num]
        w = workloads.workload(num, **shape)
        a = workloads.make_input(w)
        b = workloads.make_input(w)
        assert workloads.digest(*a) == workloads.digest(*b)
        c = workloads.make_input(w, seed=1234)
        assert workloads.digest(*c) != workloads.digest(*a)


def test_shapes_and_strides_are_16_byte_aligned():
    for w in workloads.WORKLOADS.values():
        assert (w.row_stride * w.elem_bytes) % 16 == 0
        assert w.row_stride >= w.n_cols
    w = workloads.workload(2, batch=2, n_cols=1001)
    x, _ = workloads.make_input(w)
    assert x.shape == (2, 1004)
    assert np.isnan(x[:, 1001:]).all()


def test_sampler_spikes():
    w = workloads.workload(2, batch=4)
    x, _ = workloads.make_input(w)
    assert ((x > 8).sum(axis=1) >= 32).all()
    assert abs(float(x[:, :1000].std()) - 3.0) < 0.3


def test_indexer_prefill_zeros_and_ramp():
    w = workloads.workload(4, batch=128, n_cols=4096)
    x, end = workloads.make_input(w, poison_tail=True)
    assert end[0] == 512 and end[1] == 528 and end[-1] == min(4096, 512 + 16 * 127)
    v = as_f64(x[100, :end[100]], 1)
    assert not np.isnan(v).any()
    assert 0.4 < (v == 0).mean() < 0.6
    tail = x[0, end[0]:]
    assert (tail == 0x7FC0).all()


def test_indexer_decode_has_heavy_ties():
    w = workloads.workload(3, batch=2)
    x, _ = workloads.make_input(w)
    v = as_f64(x[0], 1)
    kth = np.sort(v)[::-1][w.k - 1]
    assert (v == kth).sum() >= 10


def test_ascending_rows():
    w = workloads.workload(5, batch=2, n_cols=1 << 16)
    x, _ = workloads.make_input(w)
    means = x[0].reshape(-1, 4096).mean(axis=1)
    assert (np.diff(means) > 0).all()
    assert float(x[0, -1]) < 0.0052


def test_full_sizes_bytes():
    assert workloads.algorithmic_bytes(workloads.WORKLOADS[2]) == 33_095_680
    assert workloads.algorithmic_bytes(workloads.WORKLOADS[3]) == 33_554_432
    w4 = workloads.WORKLOADS[4]
    assert workloads.algorithmic_bytes(w4, workloads.end_ramp(w4.batch, w4.n_cols)) == 272_548_352
    assert workloads.algorithmic_bytes(workloads.WORKLOADS[5]) == 536_870_912
