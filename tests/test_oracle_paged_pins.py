"""Pins for the paged-cache reference (oracle.paged): a hand-worked table and an append sequence that crosses page
boundaries, each checked against arrays written out directly (no pool arithmetic), and a planted mistake that
both must catch."""
import numpy as np
import pytest

from oracle import paged


def _pools(n_pages, P, d_h, H, r):
    """Pool row g holds k = (g, 100 + g), v = -k, latents 1000 + 10 g + h (K) and -(1000 + 10 g + h) (V)."""
    g = np.arange(n_pages * P, dtype=np.float64)
    k = np.stack([g, 100 + g], axis=1).reshape(n_pages, P, d_h)
    zk = (1000 + 10 * g[:, None, None] + np.arange(H)[None, :, None] + np.zeros((1, 1, r))).reshape(n_pages, P, H, r)
    return k, -k, zk, -zk


def pin_hand_table(plant=0):
    # page_rows 2, max_pages 3, pool of 5 pages; sequence 0 -> pages 3, 0, 4 (5 rows), sequence 1 -> pages 1, 2 (3 rows)
    k, v, zk, zv = _pools(5, 2, 2, 1, 1)
    table = np.array([[3, 0, 4], [1, 2, 0]], dtype=np.int32)
    got = paged.gather(k, v, zk, zv, table, [5, 3], 2, 3, plant=plant)
    # by hand: sequence 0 reads pool rows 6, 7, 0, 1, 8; sequence 1 reads 2, 3, 4; unused rows stay zero
    want_k = np.array([[[6, 106], [7, 107], [0, 100], [1, 101], [8, 108], [0, 0]],
                       [[2, 102], [3, 103], [4, 104], [0, 0], [0, 0], [0, 0]]], dtype=np.float64)
    want_zk = np.array([[1060, 1070, 1000, 1010, 1080, 0], [1020, 1030, 1040, 0, 0, 0]], dtype=np.float64)
    assert np.array_equal(got["k_shared"], want_k), got["k_shared"]
    assert np.array_equal(got["v_shared"], -want_k)
    assert np.array_equal(got["z_k"][:, 0, :, 0], want_zk)
    assert np.array_equal(got["z_v"][:, 0, :, 0], -want_zk)


def pin_append_across_pages(plant=0):
    """Ten rows appended one at a time with 4-row pages (two boundaries crossed) read back in order."""
    P, maxp, npg, d_h, H, r = 4, 3, 7, 3, 2, 2
    k = np.full((npg, P, d_h), np.nan)
    v, zk, zv = k.copy(), np.full((npg, P, H, r), np.nan), np.full((npg, P, H, r), np.nan)
    table = np.array([[5, 2, 6], [0, 3, 1]], dtype=np.int32)
    lens = np.array([0, 2], dtype=np.int32)
    rows = []
    rng = np.arange(1, 1 + 2 * d_h * 12, dtype=np.float64).reshape(12, 2, d_h)
    for step in range(12):  # sequence 1 starts at 2 and fills up after 10 appends; the last 2 are dropped
        kn = rng[step]
        zn = np.stack([kn[:, :r] * (h + 1) for h in range(H)], axis=1)
        paged.append(k, v, zk, zv, table, lens, P, maxp, kn, -kn, zn, -zn)
        rows.append((kn, zn))
    assert lens.tolist() == [12, 12]
    got = paged.gather(k, v, zk, zv, table, lens, P, maxp, plant=plant)
    # sequence 0 holds steps 0..11 from row 0; sequence 1 started at 2 and held steps 0..9 when it filled up
    for b, lo, n in ((0, 0, 12), (1, 2, 10)):
        want = np.stack([rows[s][0][b] for s in range(n)])
        wz = np.stack([rows[s][1][b] for s in range(n)]).transpose(1, 0, 2)  # [H][n][r]
        assert np.array_equal(got["k_shared"][b, lo:lo + n], want), f"sequence {b} rows out of order"
        assert np.array_equal(got["v_shared"][b, lo:lo + n], -want)
        assert np.array_equal(got["z_k"][b, :, lo:lo + n], wz)
        assert np.array_equal(got["z_v"][b, :, lo:lo + n], -wz)


PAGED_PINS = [pin_hand_table, pin_append_across_pages]


@pytest.mark.parametrize("pin", PAGED_PINS, ids=lambda p: p.__name__)
def test_paged_pin(pin):
    pin()


def test_paged_planted_mistake_is_caught():
    failed = []
    for pin in PAGED_PINS:
        try:
            pin(plant=1)
        except AssertionError:
            failed.append(pin.__name__)
    assert len(failed) == len(PAGED_PINS), f"only {failed} caught the reversed in-page row"
