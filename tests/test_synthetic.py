"""CPU checks of the seeded input helpers (no arithmetic of the method lives there)."""
import numpy as np

from synthetic import sample_rows, stratified_rows


def test_stratified_rows_cover_every_tile_and_band():
    for m in (1, 5, 31, 32, 33, 255, 256, 257, 1000, 2048, 4096, 16384):
        r = stratified_rows(m, seed=m)
        assert np.all(np.diff(r) > 0) and r[0] == 0 and r[-1] == m - 1
        assert set((r // 256).tolist()) == set(range((m + 255) // 256))
        assert set((r // 32).tolist()) == set(range((m + 31) // 32))
        for t0 in range(0, m, 256):  # first and last row of every 256-row tile
            assert t0 in r and min(t0 + 256, m) - 1 in r


def test_stratified_rows_are_seeded():
    assert np.array_equal(stratified_rows(4096, seed=7), stratified_rows(4096, seed=7))
    assert not np.array_equal(stratified_rows(4096, seed=7), stratified_rows(4096, seed=8))


def test_sample_rows_holds_ends():
    r = sample_rows(1000, 50, seed=1)
    assert len(r) == 50 and r[0] == 0 and r[-1] == 999 and len(np.unique(r)) == 50
