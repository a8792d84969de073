"""The test-side SplitMix64 inverse (tests/splitmix_inverse.py) against the oracle.

The GPU modulo-edge tests build raw IDs from target hash values; each such ID
must hash back to its target under the oracle's SplitMix64, itself pinned to the
published test vectors."""
import numpy as np

import oracle
from splitmix_inverse import M64, edge_hashes, id_for_hash


def test_inverse_round_trips_through_the_oracle_hash():
    rng = np.random.default_rng(5)
    targets = [0, 1, 2, M64, M64 - 1, 1 << 63, (1 << 63) - 1]
    for rows in (1, 2, 1024, 1 << 20, 10_000_000, (1 << 31) - 1):
        targets += edge_hashes(rows)
    targets += [int(x) for x in rng.integers(0, 1 << 63, 2000, dtype=np.uint64)]
    targets += [M64 - int(x) for x in rng.integers(0, 1 << 20, 500, dtype=np.uint64)]
    ids = np.array([id_for_hash(h) for h in targets], dtype=np.int64)
    got = oracle.splitmix64(ids.view(np.uint64))
    assert [int(x) for x in got] == [h & M64 for h in targets]


def test_edge_hashes_cover_the_remainder_edges():
    rows = 10_000_000
    hs = set(edge_hashes(rows))
    top = (M64 // rows) * rows
    assert {0, M64, top - 1, top, top + 1, rows - 1, rows} <= hs
    # at the top multiple the remainder wraps from rows - 1 to 0
    assert (top - 1) % rows == rows - 1 and top % rows == 0 and (top + 1) % rows == 1
