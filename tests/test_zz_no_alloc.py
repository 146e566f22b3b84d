"""GPU check of uep_load_matrix_noalloc, the load matrix for callers that cannot
allocate: on two calls in a row (the second smaller, so the scratch array still holds
the first call's larger histograms) and in counts-only mode, its counts and bucket
positions equal those of uep_load_matrix with a caller workspace, bit for bit, and the
oracle's; a geometry beyond the scratch array is refused before any launch."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import oracle as O                                       # noqa: E402
from moe_expert_load_amd import uep as U                 # noqa: E402
from moe_expert_load_amd import workload as W            # noqa: E402
from tests.gpu_helpers import to_dev, host, err_word, say  # noqa: E402

pytestmark = pytest.mark.gpu


def test_load_matrix_noalloc_matches_the_workspace_call():
    cases = [W.LPLB_LAYER, W.scaled(W.QWEN_LAYER, T=3000), W.TINY]
    for w in cases:
        assert U.load_matrix_workspace_size(w.R, w.T, w.K, w.E) <= 8 << 20
        say(f"case: load_matrix_noalloc R={w.R} T={w.T} K={w.K} E={w.E}")
        ids = W.routing(w)
        ids[0, :5, 0] = -1                                  # a few empty slots
        ids_d = to_dev(ids)
        e1, e2 = err_word(), err_word()
        c_ws, bp_ws = U.load_matrix(ids_d, w.E, err=e1)
        counts = torch.full((w.R, w.E), -5, dtype=torch.int32, device="cuda")
        bp = torch.full((w.R, w.T, w.K), -5, dtype=torch.int32, device="cuda")
        c_na, bp_na = U.load_matrix_noalloc(ids_d, w.E, counts, bp, err=e2)
        assert host(e1)[0] == 0 and host(e2)[0] == 0
        assert torch.equal(c_na, c_ws) and torch.equal(bp_na, bp_ws)
        c_o, bp_o = O.load_matrix(ids, w.E)
        assert np.array_equal(host(c_na), c_o) and np.array_equal(host(bp_na), bp_o)
        c_only, none = U.load_matrix_noalloc(ids_d, w.E, counts_only=True)
        assert none is None and np.array_equal(host(c_only), c_o)
    # beyond the 8 MiB array: refused on the host, nothing launched
    big = torch.zeros(64, 65536, 8, dtype=torch.int32, device="cuda")
    assert U.load_matrix_workspace_size(64, 65536, 8, 1024) > 8 << 20
    with pytest.raises(U.UEPError, match="workspace"):
        U.load_matrix_noalloc(big, 1024)
