"""GPU parity at the workload sizes, in the launch configuration the
benchmark times (rrs_linear on a workspace initialised once). The oracle
computes every code and scale at full size; outputs of the two widest
configurations are compared on sampled rows and columns."""
import numpy as np
import pytest
import torch

import oracle
import rotated_runtime_activation_amd as rra
import workloads
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

# name -> (output rows sampled, output columns sampled); None = all
SAMPLING = {"tiny": None, "o_proj": None, "decode": None, "gate_up": (96, 384), "g_sweep": (96, 384),
            "down_proj": (96, 384)}
# group sizes run beyond the workload's own: G = 64 takes its own GEMM
# schedule (one group per 32x32x64 MFMA K step), G = 256 the generic one
EXTRA_G = {"g_sweep": (64, 256)}


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_workload(name):
    wl = workloads.WORKLOADS[name]
    M, K, N = wl.M, wl.K, wl.N
    gu.log(f"[workload {name}] M={M} K={K} N={N} G={wl.G}: generating inputs")
    x = workloads.runtime_x(wl)
    w = workloads.weights(wl)
    xc = workloads.calib_x(wl)
    perm_ref = oracle.calibrate_perm(xc)

    # the calibration reorder on the GPU (what the benchmark uses)
    gu.log(f"[workload {name}] calibrate_perm")
    perm_gpu = torch.empty(K, dtype=torch.int32, device=gu.DEV)
    cws = torch.empty(rra.rrs_calibrate_workspace_bytes(K), dtype=torch.uint8, device=gu.DEV)
    rra.rrs_calibrate_perm(gu.to_dev(xc), perm_gpu, cws)
    torch.cuda.synchronize()
    pg = perm_gpu.cpu().numpy()
    c = np.abs(oracle.rotate_rows(xc)).max(axis=0)
    diff = pg != perm_ref
    assert np.all(np.abs(c[pg[diff]] - c[perm_ref[diff]]) <= 1e-5 * c[perm_ref[diff]])
    gu.log(f"  perm: {int(diff.sum())} near-tie positions differ")

    sample = SAMPLING[name]
    rng = np.random.default_rng(wl.index)
    if sample is None:
        rows, cols = np.arange(M), np.arange(N)
    else:
        rows = np.sort(rng.choice(M, size=sample[0], replace=False))
        cols = np.sort(rng.choice(N, size=sample[1], replace=False))
        cols[-1] = N - 1     # include the ragged end of the last tile
        rows[-1] = M - 1

    gu.log(f"[workload {name}] prepare_weights")
    wq = gu.prepare_weights(w, perm_ref)
    torch.cuda.synchronize()
    codes, dw = rra.weight_views(wq, K, N)
    wp = oracle.prepare_weights(w[:, cols], perm_ref)
    qw_gpu = oracle.unpack_codes(codes[torch.from_numpy(cols).to(gu.DEV)].cpu().numpy())
    gu.compare_codes(qw_gpu, wp["qw"], wp["uw"], "weight codes")
    gu.rel_close(dw.cpu().numpy()[cols], wp["dw"], gu.SCALE_TOL, "dw")

    X = gu.to_dev(x)
    P = gu.to_dev(perm_ref)
    for G in tuple(wl.G) + EXTRA_G.get(name, ()):
        gu.log(f"[workload {name}] rrs_linear G={G}")
        ws = torch.zeros(rra.rrs_workspace_bytes(M, K, G), dtype=torch.uint8, device=gu.DEV)
        rra.rrs_workspace_init(ws)
        Y = torch.empty(M, N, dtype=torch.float32, device=gu.DEV)
        rra.rrs_linear(X, G, P, wq, Y, ws)
        rra.rrs_linear(X, G, P, wq, Y, ws)     # second call on the same workspace
        torch.cuda.synchronize()
        gu.check_sync_block(ws, K, G, calls=2)
        gu.log(f"  front end: {rra.rrs_frontend_passes(M, K, 0)} launch(es)")
        xq, dx, S = rra.workspace_views(ws, M, K, G)
        fe = oracle.frontend(x, perm_ref, G)
        q_gpu = oracle.unpack_codes(xq.cpu().numpy())
        gu.compare_codes(q_gpu, fe["q"], fe["v"], f"activation codes G={G}")
        gu.rel_close(dx.cpu().numpy(), fe["dx"], gu.SCALE_TOL, "dx")
        gu.rel_close(S.cpu().numpy(), fe["S"], gu.SCALE_TOL, "S")

        ref = oracle.linear_out(fe["q"][rows], fe["dx"][rows], fe["S"], wp["qw"], wp["dw"], G)
        Yg = Y.cpu().numpy()[np.ix_(rows, cols)]
        fe_rows = {"q": fe["q"][rows], "dx": fe["dx"][rows], "S": fe["S"]}
        gu.check_linear_two_way(Yg, ref, q_gpu[rows], qw_gpu, dx.cpu().numpy()[rows], S.cpu().numpy(),
                                dw.cpu().numpy()[cols], G, f"{name} G={G}", fe=fe_rows, wp=wp)
        del ws, Y
    torch.cuda.empty_cache()
