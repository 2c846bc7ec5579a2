"""The allocation-free Top-K (csa2_topk_noalloc) against csa2_topk with a
caller workspace, through the C ABI: two calls in a row on the same GPU, the
second with fewer rows and shorter rows than the first, so the second reads a
scratch the first left dirty.  Rows are longer than 16,384 slots, so the
selection runs through the workspace (histogram, row state, candidates)."""
import numpy as np
import pytest
import torch

import oracle
from compressed_sparse_attention_amd import csa2 as C

pytestmark = pytest.mark.gpu


def _scores(rng, nq, n, ties):
    s = rng.random((nq, n), dtype=np.float32)
    if ties:  # few distinct values: long runs of equal keys at the thresholds
        s = np.floor(s * 50.0).astype(np.float32) / 50.0
    return s


@pytest.mark.parametrize("ties", [False, True])
def test_topk_noalloc_matches_topk(ties):
    rng = np.random.default_rng(4242 + ties)
    for nq, n in ((200, 60000), (37, 20001)):
        lens = [n] * nq
        qp = [np.array([n - 1 - (r % 3)]) for r in range(nq)]
        b = C.Batch(lens, qp)
        sc_h = _scores(rng, nq, n, ties)
        sc = torch.from_numpy(sc_h).cuda()
        want = C.csa2_topk(b, sc, 512)
        got = torch.full((nq, 512), -7, dtype=torch.int32, device="cuda")
        C.csa2_topk_noalloc(b, sc, 512, got)
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"{nq} rows of {n}"
        vis = np.array([min(n, int(p[0]) + 1) for p in qp], np.int64)
        assert np.array_equal(got.cpu().numpy(), oracle.topk(sc_h, vis, 512))


def test_topk_noalloc_rejects_too_many_rows():
    b = C.Batch([30000] * 257, [np.array([29999])] * 257)
    sc = torch.zeros((257, 30000), dtype=torch.float32, device="cuda")
    idx = torch.empty((257, 512), dtype=torch.int32, device="cuda")
    with pytest.raises(C.CSA2Error):
        C.csa2_topk_noalloc(b, sc, 512, idx)
