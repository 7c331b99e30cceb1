"""Pins of the oracle's row-tiled weight layout (tile_rows).

The layout is a permutation of the weight values (megakernel page, the GEMV's
tiled-weights option; here tiles of four rows by 256 values).  It is pinned by
hand-derived offsets, by the byte runs one 64-lane, 16-byte-a-lane load reads,
and by the GEMV over the untiled values being unchanged.
"""
import json
import os

import numpy as np
import pytest

import oracle


def test_tile_layout_golden(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "tile_layout.json")))
    N, K = g["N"], g["K"]
    # every value names its own position: row r, column c -> code r*K + c, kept
    # as an index array (the layout is a pure permutation of bytes)
    idx = np.arange(N * K, dtype=np.int64).reshape(N, K)
    tiled_pos = np.empty(N * K, np.int64)
    # tile_rows moves bytes; run it on the low and high bytes of the index
    lo = oracle.tile_rows((idx & 0xFF).astype(np.uint8).view(np.int8)).view(np.uint8).reshape(-1)
    hi = oracle.tile_rows(((idx >> 8) & 0xFF).astype(np.uint8).view(np.int8)).view(np.uint8).reshape(-1)
    tiled_pos[:] = lo.astype(np.int64) | (hi.astype(np.int64) << 8)
    for c in g["cases"]:
        assert divmod(int(tiled_pos[c["offset"]]), K) == (c["row"], c["col"]), c


def test_tile_is_a_permutation_and_one_wave_load_is_four_row_pieces():
    rng = np.random.default_rng(7)
    N, K = 12, 768
    wq = rng.integers(-127, 128, size=(N, K), dtype=np.int8)
    t = oracle.tile_rows(wq).reshape(-1)
    assert t.shape == (N * K,)
    assert np.array_equal(np.sort(t), np.sort(wq.reshape(-1)))
    # a wave's 1 KiB at 1024*(t*K/256 + s) holds rows 4t..4t+3, columns 256s..256s+255, row after row
    for tt in range(N // 4):
        for s in range(K // 256):
            piece = t[1024 * (tt * (K // 256) + s):][:1024].reshape(4, 256)
            assert np.array_equal(piece, wq[4 * tt:4 * tt + 4, 256 * s:256 * s + 256])


def test_tile_rejects_ragged_shapes():
    with pytest.raises(ValueError):
        oracle.tile_rows(np.zeros((6, 512), np.int8))
    with pytest.raises(ValueError):
        oracle.tile_rows(np.zeros((8, 288), np.int8))
