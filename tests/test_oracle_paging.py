"""Pins for the oracle's paged-row gather (CPU only): scattering contiguous
rows into randomly placed pages and gathering them back gives the rows
unchanged, sequence by sequence, for page sizes that do and do not divide
the sequence lengths; a hand-built two-page table reads its rows in order."""
import numpy as np
import pytest

from oracle import paging as opg
from synth.paging import to_paged


@pytest.mark.parametrize("page_size", [64, 128, 256])
def test_scatter_then_gather_is_the_identity(page_size):
    rng = np.random.default_rng(page_size)
    lens, T, Hkv, D = [37, 300, 0, 129], 11, 2, 8
    indptr = np.zeros(len(lens) + 1, dtype=np.int64)
    indptr[1:] = np.cumsum(np.asarray(lens) + T)
    k = rng.standard_normal((int(indptr[-1]), Hkv, D)).astype(np.float32)
    v = rng.standard_normal((int(indptr[-1]), Hkv, D)).astype(np.float32)
    kp, vp, table = to_paged(k, v, indptr, lens, T, page_size, rng)
    for b, L in enumerate(lens):
        n = L + T
        assert np.array_equal(opg.gather(kp, table, b, n, page_size), k[indptr[b]: indptr[b] + n])
        assert np.array_equal(opg.gather(vp, table, b, n, page_size), v[indptr[b]: indptr[b] + n])
    used = np.concatenate([table[b, :(L + T + page_size - 1) // page_size] for b, L in enumerate(lens)])
    assert len(set(used.tolist())) == len(used)          # no page is shared


def test_hand_built_table():
    P = 64
    pool = np.arange(4 * P).reshape(4 * P, 1, 1)          # each row holds its physical index
    table = np.array([[2, 0]], dtype=np.int32)            # logical rows 0..63 in page 2, 64.. in page 0
    rows = opg.gather(pool, table, 0, 70, P)[:, 0, 0]
    assert rows[:64].tolist() == list(range(128, 192)) and rows[64:].tolist() == list(range(0, 6))
