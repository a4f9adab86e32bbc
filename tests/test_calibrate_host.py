"""Host-side choice of the dominant FCs (fasa_select_dominant, no GPU call)
against the oracle's, on random agreement values and the pins' hand example."""

import numpy as np
import pytest

import oracle


@pytest.fixture(scope="module")
def fasa():
    import sparse_kv_cache_rope_amd as m
    return m


@pytest.mark.parametrize("shape,n_dom", [((1, 2, 32), 4), ((5, 32, 64), 16), ((3, 8, 64), 64)])
def test_select_dominant_matches_oracle(fasa, shape, n_dom):
    r = np.random.default_rng(sum(shape))
    # Multiples of 1/8 force many equal means (ties go to the lower FC).
    ca = (r.integers(0, 9, size=shape) / 8.0).astype(np.float32)
    got = fasa.select_dominant(ca, n_dom)
    want = oracle.calibrate.dominant_from_ca(ca.astype(np.float64), n_dom)
    assert np.array_equal(got, want)


def test_select_dominant_hand_example(fasa):
    ca = np.array([[[0.5, 0.5, 0.9, 0.1], [0.2, 0.2, 0.2, 0.2]],
                   [[0.5, 0.3, 0.7, 0.1], [0.0, 0.4, 0.2, 0.4]]], dtype=np.float32)
    assert fasa.select_dominant(ca, 2).tolist() == [[0, 2], [1, 3]]
    assert fasa.select_dominant(ca, 1).tolist() == [[2], [1]]


def test_select_dominant_rejects_bad_sizes(fasa):
    ca = np.zeros((1, 2, 4), dtype=np.float32)
    for n_dom in (0, 5):
        with pytest.raises(fasa.FasaError):
            fasa.select_dominant(ca, n_dom)
