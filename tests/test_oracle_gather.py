"""Pins of the oracle's gathered A (the first result of a = all_gather(a_shared), out = a @ b
in the Helion thread's Kraken-optimization comment; shard r holds global rows
[r*M_per_rank, (r+1)*M_per_rank)).

- closed form: shard d filled with (d << 12) | (local row << 4) | (column & 15), so row m
  of the result must read (m // M_s) << 12 | (m % M_s) << 4 | (k & 15);
- a bit copy: every 16-bit pattern (NaNs and signed zeros included) passes unchanged;
- empty shards and K = 0;
- planted mistakes (shards in reverse order, rows of a shard reversed, a shard's first row
  dropped) each fail the closed form.
"""
import numpy as np
import pytest

import oracle


def _coded_shards(D, Ms, K):
    k = np.arange(K, dtype=np.uint32) & 15
    return [(((d << 12) | (np.arange(Ms, dtype=np.uint32)[:, None] << 4) | k[None, :])
             .astype(np.uint16)) for d in range(D)]


def _closed_form(D, Ms, K):
    m = np.arange(D * Ms, dtype=np.uint32)[:, None]
    k = np.arange(K, dtype=np.uint32)[None, :]
    return (((m // Ms) << 12) | ((m % Ms) << 4) | (k & 15)).astype(np.uint16) if Ms else \
        np.zeros((0, K), dtype=np.uint16)


@pytest.mark.parametrize("D,Ms,K", [(1, 5, 24), (2, 3, 16), (3, 200, 8), (8, 17, 40), (15, 1, 1)])
def test_closed_form(D, Ms, K):
    got = oracle.all_gather(_coded_shards(D, Ms, K))
    assert got.shape == (D * Ms, K) and got.dtype == np.uint16
    np.testing.assert_array_equal(got, _closed_form(D, Ms, K))


def test_bit_copy_of_every_pattern():
    allbits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).reshape(4, 128, 128)
    got = oracle.all_gather([allbits[d] for d in range(4)])
    np.testing.assert_array_equal(got, allbits.reshape(512, 128))


def test_empty():
    assert oracle.all_gather([np.zeros((0, 8), np.uint16)] * 3).shape == (0, 8)
    assert oracle.all_gather([np.zeros((4, 0), np.uint16)] * 2).shape == (8, 0)


def test_planted_mistakes_are_caught():
    D, Ms, K = 4, 6, 16
    sh = _coded_shards(D, Ms, K)
    want = _closed_form(D, Ms, K)
    assert not np.array_equal(oracle.all_gather(sh[::-1]), want)              # rank order
    assert not np.array_equal(oracle.all_gather([s[::-1] for s in sh]), want)  # row order
    dropped = [np.vstack([s[1:], s[:1]]) for s in sh]
    assert not np.array_equal(oracle.all_gather(dropped), want)               # a row lost
