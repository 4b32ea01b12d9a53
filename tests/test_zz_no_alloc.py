"""rrs_linear_noalloc (no workspace argument, the library's fixed scratch)
against rrs_linear with a caller's workspace: the same kernels, so the same
bits, on two calls in a row, the second with fewer tokens; requests beyond
the scratch are rejected before any launch."""
import numpy as np
import pytest
import torch

import oracle
import rotated_runtime_activation_amd as rra
import workloads
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _run_both(M, K, N, G, seed):
    x, xc, w = workloads.random_case(seed, M, K, N)
    perm = oracle.calibrate_perm(xc)
    X, P = gu.to_dev(x), gu.to_dev(perm)
    wq = gu.prepare_weights(w, perm)
    ws = torch.zeros(rra.rrs_workspace_bytes(M, K, G), dtype=torch.uint8, device=gu.DEV)
    rra.rrs_workspace_init(ws)
    Y_ref = torch.empty(M, N, dtype=torch.float32, device=gu.DEV)
    rra.rrs_linear(X, G, P, wq, Y_ref, ws)
    Y = torch.full((M, N), float("nan"), dtype=torch.float32, device=gu.DEV)
    st = rra.lib().rrs_linear_noalloc(X.data_ptr(), M, K, N, G, P.data_ptr(), wq.data_ptr(), Y.data_ptr(),
                                     torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == rra.RRS_OK, rra.rrs_status_string(st)
    return x, w, perm, Y, Y_ref


@pytest.mark.parametrize("shapes", [
    [(700, 4096, 300, 128), (64, 4096, 300, 128)],     # one row per wave, then one row per workgroup
    [(2048, 4096, 512, 128), (5, 2048, 130, 32)],      # o_proj tokens, then a few tokens at another K, G
    [(3000, 8192, 64, 256), (300, 1792, 40, 64)],      # three launches at K = 8192, then a Kronecker K
])
def test_noalloc_matches_rrs_linear(shapes):
    for i, (M, K, N, G) in enumerate(shapes):
        gu.log(f"[noalloc] call {i}: M={M} K={K} N={N} G={G}")
        x, w, perm, Y, Y_ref = _run_both(M, K, N, G, 100 + i + M)
        assert torch.equal(Y, Y_ref), f"{int((Y != Y_ref).sum())} outputs differ from rrs_linear"
        if i == 0:   # and the first call against the oracle itself
            ref = oracle.rrs_linear(x, w, perm, G)
            err = gu.y_error(Y.cpu().numpy(), {"Y": ref["Y"], "C": ref["C"]})
            gu.log(f"  err/C vs oracle {err:.3e}")
            assert err < 0.05  # the code flips' movement; the kernels are checked tightly elsewhere


def test_noalloc_rejects_beyond_scratch():
    K, N, G = 4096, 64, 128
    M = 12167   # one token more than fits 24 MiB at K = 4096, G = 128
    X = torch.zeros(16, dtype=torch.float16, device=gu.DEV)   # never read: rejected before any launch
    st = rra.lib().rrs_linear_noalloc(X.data_ptr(), M, K, N, G, X.data_ptr(), X.data_ptr(), X.data_ptr(), None)
    assert st == rra.RRS_ETOOBIG
    assert rra.lib().rrs_linear_noalloc(X.data_ptr(), 1, 100, N, G, X.data_ptr(), X.data_ptr(), X.data_ptr(),
                                        None) == rra.RRS_EINVAL
