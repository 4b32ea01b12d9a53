"""GPU parity of the component switches end to end (RRS rebuttal page,
"Incomplete ablation study": online smoothing, reordering and rotation as
separable parts) and of the one-launch front end's failure path.

Runtime Smooth alone skips the rotation on both sides (calibration on the
raw channels, weights reordered without H, no 1/K in the output); the
rotation alone keeps S = 1 (the per-channel A4W4 baseline). Each variant
runs through rrs_calibrate_perm_ex, rrs_prepare_weights_ex and
rrs_linear_ex and is compared with the oracle's rrs_linear(rotate=...,
smooth=...) by the same rules as the full method."""
import numpy as np
import pytest
import torch

import oracle
import rotated_runtime_activation_amd as rra
import workloads
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

NR, NS, TP, GU = rra.RRS_FLAG_NO_ROTATE, rra.RRS_FLAG_NO_SMOOTH, rra.RRS_FLAG_TWO_PASS, rra.RRS_FLAG_TEST_GIVE_UP

# (M, K, N, G, flags): one-row-per-wave (300, 1024), row-per-workgroup
# (64 x 8192, few-token GEMM), the three launches (TWO_PASS), tiled GEMM,
# and the Kronecker rotation's K
CASES = [
    (48, 1024, 130, 64, 0), (48, 1024, 130, 64, NR), (48, 1024, 130, 64, NS), (48, 1024, 130, 64, NR | NS),
    (300, 4096, 96, 128, NR), (300, 4096, 96, 128, NS),
    (64, 8192, 64, 128, NR), (64, 8192, 64, 32, NS),
    (500, 2048, 300, 32, NR | TP), (200, 512, 260, 128, NR),
    (20, 1792, 40, 64, NR), (20, 1792, 40, 64, NS), (300, 1536, 50, 128, NR | TP),
]


def _flags_name(flags):
    return "+".join(n for f, n in ((NR, "no_rotate"), (NS, "no_smooth"), (TP, "two_pass")) if flags & f) or "rrs"


@pytest.mark.parametrize("M,K,N,G,flags", CASES)
def test_linear_ablation(M, K, N, G, flags):
    rotate, smooth = not flags & NR, not flags & NS
    gu.log(f"[ablation {_flags_name(flags)}] M={M} K={K} N={N} G={G} "
           f"front end {rra.rrs_frontend_passes(M, K, flags)} launch(es), gemm form {rra.rrs_gemm_form(M, K, N, G)}")
    x, xc, w = workloads.random_case(M * 31 + K + flags, M, K, N)

    # calibration on the GPU: without the rotation the channel maxima are
    # fp16 values, compared exactly, so the order is unique up to exact ties
    # (broken by index on both sides)
    perm_ref = oracle.calibrate_perm(xc, rotate=rotate)
    perm = torch.empty(K, dtype=torch.int32, device=gu.DEV)
    cws = torch.empty(rra.rrs_calibrate_workspace_bytes(K), dtype=torch.uint8, device=gu.DEV)
    rra.rrs_calibrate_perm_ex(gu.to_dev(xc), None, flags & NR, perm, cws)
    torch.cuda.synchronize()
    pg = perm.cpu().numpy()
    if not rotate:
        assert np.array_equal(pg, perm_ref)
    else:
        c = np.abs(oracle.rotate_rows(xc)).max(axis=0)
        diff = pg != perm_ref
        assert np.all(np.abs(c[pg[diff]] - c[perm_ref[diff]]) <= 1e-5 * c[perm_ref[diff]])

    ref = oracle.rrs_linear(x, w, perm_ref, G, rotate=rotate, smooth=smooth)
    wq = torch.empty(rra.rrs_weight_bytes(K, N), dtype=torch.uint8, device=gu.DEV)
    rra.rrs_prepare_weights_ex(gu.to_dev(w), gu.to_dev(perm_ref), None, flags & NR, wq)
    ws = torch.zeros(rra.rrs_workspace_bytes(M, K, G), dtype=torch.uint8, device=gu.DEV)
    rra.rrs_workspace_init(ws)
    Y = torch.empty(M, N, dtype=torch.float32, device=gu.DEV)
    rra.rrs_linear_ex(gu.to_dev(x), G, gu.to_dev(perm_ref), None, flags, wq, Y, ws)
    torch.cuda.synchronize()
    assert ws[8:12].view(torch.int32).item() == 0, "error word set"

    codes, dw = rra.weight_views(wq, K, N)
    qw_gpu = oracle.unpack_codes(codes.cpu().numpy())
    gu.compare_codes(qw_gpu, ref["wp"]["qw"], ref["wp"]["uw"], "weight codes")
    gu.rel_close(dw.cpu().numpy(), ref["wp"]["dw"], gu.SCALE_TOL, "dw")
    xq, dx, S = rra.workspace_views(ws, M, K, G)
    q_gpu = oracle.unpack_codes(xq.cpu().numpy())
    gu.compare_codes(q_gpu, ref["fe"]["q"], ref["fe"]["v"], "activation codes")
    gu.rel_close(dx.cpu().numpy(), ref["fe"]["dx"], gu.SCALE_TOL, "dx")
    gu.rel_close(S.cpu().numpy(), ref["fe"]["S"], gu.SCALE_TOL, "S")
    if not smooth:
        assert np.all(S.cpu().numpy() == 1.0)
    gu.check_linear_two_way(Y.cpu().numpy(), ref, q_gpu, qw_gpu, dx.cpu().numpy(), S.cpu().numpy(),
                            dw.cpu().numpy(), G, _flags_name(flags), rotated=rotate)


def test_ablation_ex_entry_points_match_plain():
    """flags = 0 through the _ex entry points is the full method: the same
    bits as rrs_calibrate_perm, rrs_prepare_weights and rrs_linear."""
    M, K, N, G = 40, 2048, 70, 128
    x, xc, w = workloads.random_case(77, M, K, N)
    X, W, XC = gu.to_dev(x), gu.to_dev(w), gu.to_dev(xc)
    cws = torch.empty(rra.rrs_calibrate_workspace_bytes(K), dtype=torch.uint8, device=gu.DEV)
    p1 = torch.empty(K, dtype=torch.int32, device=gu.DEV)
    p2 = torch.empty_like(p1)
    rra.rrs_calibrate_perm(XC, p1, cws)
    rra.rrs_calibrate_perm_ex(XC, None, 0, p2, cws)
    w1 = torch.empty(rra.rrs_weight_bytes(K, N), dtype=torch.uint8, device=gu.DEV)
    w2 = torch.empty_like(w1)
    rra.rrs_prepare_weights(W, p1, w1)
    rra.rrs_prepare_weights_ex(W, p1, None, 0, w2)
    ws = torch.zeros(rra.rrs_workspace_bytes(M, K, G), dtype=torch.uint8, device=gu.DEV)
    rra.rrs_workspace_init(ws)
    Y1 = torch.empty(M, N, dtype=torch.float32, device=gu.DEV)
    Y2 = torch.empty_like(Y1)
    rra.rrs_linear(X, G, p1, w1, Y1, ws)
    rra.rrs_linear_ex(X, G, p1, None, 0, w1, Y2, ws)
    torch.cuda.synchronize()
    (c1, d1), (c2, d2) = rra.weight_views(w1, K, N), rra.weight_views(w2, K, N)  # not the padding
    assert torch.equal(p1, p2) and torch.equal(c1, c2) and torch.equal(d1, d2) and torch.equal(Y1, Y2)


# ------------------------------------------------------ failure path
# Shapes taking each one-launch form: one row per workgroup (K = 4096,
# M <= 256), one row per wave (fused_kernel), and the Kronecker one-launch
# form (K = 1792, few rows); each also as a grid of a single workgroup,
# which exchanges no maxima but honours the test flag and the error word
# the same way (M = 1 at K = 4096 and 1792, M = 16 at K = 256).
GIVE_UP_CASES = [(64, 4096, 128), (1000, 4096, 128), (40, 1024, 64), (16, 1792, 64),
                 (1, 4096, 128), (16, 256, 64), (1, 1792, 64)]


@pytest.mark.parametrize("M,K,G", GIVE_UP_CASES)
def test_wait_give_up_is_visible(M, K, G):
    """A one-launch front end whose grid-wide wait gives up (forced from the
    host with the test flag: every workgroup gives up after one poll, and
    every kernel ends normally) sets the workspace's error word, marks its
    token scales (and S) with NaN, and every rrs_linear on that workspace
    then writes NaN into all of Y until rrs_workspace_init; after it, the
    same call is correct again."""
    N = 96
    assert rra.rrs_frontend_passes(M, K, 0) == 1
    gu.log(f"[give up] M={M} K={K} G={G}")
    x, xc, w = workloads.random_case(M + K, M, K, N)
    perm = oracle.calibrate_perm(xc)
    X, P = gu.to_dev(x), gu.to_dev(perm)
    wq = gu.prepare_weights(w, perm)
    ws = torch.zeros(rra.rrs_workspace_bytes(M, K, G), dtype=torch.uint8, device=gu.DEV)
    rra.rrs_workspace_init(ws)
    _, dx, S = rra.workspace_regions(ws, M, K, G)
    Y = torch.empty(M, N, dtype=torch.float32, device=gu.DEV)

    # the front end alone: error word, NaN scales
    sync = torch.zeros(rra.rrs_sync_bytes(K, G), dtype=torch.uint8, device=gu.DEV)
    rra.rrs_workspace_init(sync)
    xq1 = gu.xq_empty(M, K)
    dx1 = torch.empty(M, dtype=torch.float32, device=gu.DEV)
    S1 = torch.empty(K // G, dtype=torch.float32, device=gu.DEV)
    rra.rrs_frontend(X, G, P, xq1, dx1, S1, sync, GU)
    torch.cuda.synchronize()
    assert sync[8:12].view(torch.int32).item() != 0, "error word not set"
    assert torch.isnan(dx1).all() and torch.isnan(S1).all()

    # the layer: Y is NaN, and stays NaN on the same workspace
    rra.rrs_linear_ex(X, G, P, None, GU, wq, Y, ws)
    torch.cuda.synchronize()
    assert torch.isnan(Y).all()
    rra.rrs_linear(X, G, P, wq, Y, ws)
    torch.cuda.synchronize()
    assert torch.isnan(Y).all(), "a later call on the failed workspace must stay visible"

    # re-initialised: correct again
    rra.rrs_workspace_init(ws)
    rra.rrs_linear(X, G, P, wq, Y, ws)
    torch.cuda.synchronize()
    assert ws[8:12].view(torch.int32).item() == 0
    ref = oracle.rrs_linear(x, w, perm, G)
    q_gpu = oracle.unpack_codes(rra.workspace_views(ws, M, K, G)[0].cpu().numpy())
    gu.compare_codes(q_gpu, ref["fe"]["q"], ref["fe"]["v"], "codes after init")
    codes, dw = rra.weight_views(wq, K, N)
    gu.check_linear_two_way(Y.cpu().numpy(), ref, q_gpu, oracle.unpack_codes(codes.cpu().numpy()),
                            dx.cpu().numpy(), S.cpu().numpy(), dw.cpu().numpy(), G, "after init")


def test_error_word_set_from_host_poisons_y():
    """The GEMM of rrs_linear reads the error word whatever set it: written
    from the host here, Y is NaN on both GEMM kernels (few tokens, tiled)."""
    K, N, G = 2048, 300, 128
    for M in (16, 700):
        gu.log(f"[error word] M={M} form={rra.rrs_gemm_form(M, K, N, G)}")
        x, xc, w = workloads.random_case(M, M, K, N)
        perm = oracle.calibrate_perm(xc)
        wq = gu.prepare_weights(w, perm)
        ws = torch.zeros(rra.rrs_workspace_bytes(M, K, G), dtype=torch.uint8, device=gu.DEV)
        rra.rrs_workspace_init(ws)
        ws[8:12].view(torch.int32).fill_(1)
        Y = torch.zeros(M, N, dtype=torch.float32, device=gu.DEV)
        rra.rrs_linear(gu.to_dev(x), G, gu.to_dev(perm), wq, Y, ws)
        torch.cuda.synchronize()
        assert torch.isnan(Y).all()
