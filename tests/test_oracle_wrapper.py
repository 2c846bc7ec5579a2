"""The oracle's Python wrapper: running the layer chain on a subset of query
rows (as the full-size GPU tests do) gives those rows' results of the full run."""
import numpy as np

import oracle
import synth


def test_row_subset_chain_equals_full_chain():
    wl = synth.config("chain_c2", n_seq=3, n=20000, Hm=4)
    full = oracle.layer_chain(wl)
    pick = np.array([2, 0])
    sub = oracle.layer_chain(wl, rows=pick)
    for f, s in zip(full, sub):
        assert np.array_equal(f["idx"][pick], s["idx"]), f["layer"]
        assert np.array_equal(f["out"][pick], s["out"]), f["layer"]
        if "pool_pos" in f:
            assert np.array_equal(f["pool_pos"][pick], s["pool_pos"])
