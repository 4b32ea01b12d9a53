"""GPU parity of the signed rotation X D H (AGC-OR page, Sec. 4.1 / Sec. 4.6;
reading R18) against the oracle: front end (both forms, butterfly and
matrix-core rotations), weight preparation H D W, calibration and the whole
layer (run on an MI355X: -m gpu)."""
import numpy as np
import pytest
import torch

import oracle
import rotated_runtime_activation_amd as rra
import workloads
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _signs(K, seed):
    bits = np.random.default_rng(seed).integers(0, 2**32, size=K // 32, dtype=np.uint64).astype(np.uint32)
    return bits, oracle.signs_from_bits(bits, K)


def _dev_bits(bits):
    return gu.to_dev(bits.view(np.int32))


def _case(M, K, N=8):
    x, xc, w = workloads.random_case(M * 31 + K, M, K, N)
    bits, d = _signs(K, K + M)
    perm = oracle.calibrate_perm(xc, d)
    return x, w, perm, bits, d


@pytest.mark.parametrize("form", ["one-launch", "multi-launch"])
@pytest.mark.parametrize("M,K,G", [(16, 256, 64), (7, 2048, 64), (40, 4096, 128), (5, 8192, 256),
                                   (65, 8192, 32), (300, 512, 128), (300, 2048, 128), (260, 1024, 64),
                                   (1, 8192, 128)])
def test_frontend_signed(M, K, G, form):
    flags = rra.RRS_FLAG_TWO_PASS if form == "multi-launch" else 0
    gu.log(f"[frontend signed] M={M} K={K} G={G} {form}")
    x, _, perm, bits, d = _case(M, K)
    fe = oracle.frontend(x, perm, G, d=d)
    xq = gu.xq_empty(M, K)
    dx = torch.empty(M, dtype=torch.float32, device=gu.DEV)
    S = torch.empty(K // G, dtype=torch.float32, device=gu.DEV)
    ws = torch.zeros(rra.rrs_sync_bytes(K, G), dtype=torch.uint8, device=gu.DEV)
    rra.rrs_frontend_signed(gu.to_dev(x), G, gu.to_dev(perm), _dev_bits(bits), xq, dx, S, ws, flags)
    torch.cuda.synchronize()
    gu.check_sync_block(ws, K, G)
    gu.compare_codes(oracle.unpack_codes(gu.xq_codes(xq, M, K)), fe["q"], fe["v"], "signed codes")
    gu.rel_close(dx.cpu().numpy(), fe["dx"], gu.SCALE_TOL, "signed dx")
    gu.rel_close(S.cpu().numpy(), fe["S"], gu.SCALE_TOL, "signed S")


def test_frontend_signed_all_plus_matches_plain():
    """An all-clear mask is the plain rotation: bit-identical outputs."""
    gu.log("[frontend signed] all-plus mask vs plain")
    M, K, G = 33, 4096, 128
    x, _, perm, _, _ = _case(M, K)
    zero = torch.zeros(K // 32, dtype=torch.int32, device=gu.DEV)
    outs = []
    for signed in (False, True):
        xq = gu.xq_empty(M, K)
        dx = torch.empty(M, dtype=torch.float32, device=gu.DEV)
        S = torch.empty(K // G, dtype=torch.float32, device=gu.DEV)
        ws = torch.zeros(rra.rrs_sync_bytes(K, G), dtype=torch.uint8, device=gu.DEV)
        if signed:
            rra.rrs_frontend_signed(gu.to_dev(x), G, gu.to_dev(perm), zero, xq, dx, S, ws)
        else:
            rra.rrs_frontend(gu.to_dev(x), G, gu.to_dev(perm), xq, dx, S, ws)
        outs.append((rra.codes_matrix(xq, M, K), dx, S))
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a, b)


@pytest.mark.parametrize("K,N", [(256, 64), (4096, 130), (8192, 33), (1024, 7)])
def test_prepare_weights_signed(K, N):
    gu.log(f"[weights signed] K={K} N={N}")
    _, w, perm, bits, d = _case(4, K, N)
    wq = torch.empty(rra.rrs_weight_bytes(K, N), dtype=torch.uint8, device=gu.DEV)
    rra.rrs_prepare_weights_signed(gu.to_dev(w), gu.to_dev(perm), _dev_bits(bits), wq)
    torch.cuda.synchronize()
    codes, dw = rra.weight_views(wq, K, N)
    ref = oracle.prepare_weights(w, perm, d)
    gu.compare_codes(oracle.unpack_codes(codes.cpu().numpy()), ref["qw"], ref["uw"], "signed weight codes")
    gu.rel_close(dw.cpu().numpy(), ref["dw"], gu.SCALE_TOL, "signed dw")


@pytest.mark.parametrize("T,K", [(128, 256), (512, 4096), (100, 8192)])
def test_calibrate_perm_signed(T, K):
    gu.log(f"[calibrate signed] T={T} K={K}")
    wl = workloads.Workload(30_000 + K, "cal", T, K, 8, (K,), 8, 20.0, "count", 3, 500.0, 0.02, T)
    xc = workloads.make_activations(wl, T, wl.seed_base + workloads.ROLE_CALIB)
    bits, d = _signs(K, 7 * K)
    ref = oracle.calibrate_perm(xc, d)
    perm = torch.empty(K, dtype=torch.int32, device=gu.DEV)
    ws = torch.empty(rra.rrs_calibrate_workspace_bytes(K), dtype=torch.uint8, device=gu.DEV)
    rra.rrs_calibrate_perm_signed(gu.to_dev(xc), _dev_bits(bits), perm, ws)
    torch.cuda.synchronize()
    got = perm.cpu().numpy()
    assert np.array_equal(np.sort(got), np.arange(K))
    c = np.abs(oracle.rotate_rows(xc, d)).max(axis=0)
    cs = c[got]
    assert np.all(cs[:-1] >= cs[1:] * (1 - 1e-5) - 1e-30)
    same = got == ref
    if not same.all():
        idx = np.nonzero(~same)[0]
        assert np.all(np.abs(c[got[idx]] - c[ref[idx]]) <= 1e-5 * c[ref[idx]])
    gu.log(f"  perm positions differing from the oracle (near-ties): {int((~same).sum())}")


@pytest.mark.parametrize("M,K,N,G", [(16, 4096, 256, 128), (3, 8192, 129, 128), (130, 1024, 260, 64),
                                     (64, 8192, 96, 256),
                                     # one row per wave past 256 rows (fused_kernel, signed)
                                     (300, 2048, 64, 128), (260, 1024, 40, 32)])
def test_linear_signed(M, K, N, G):
    gu.log(f"[linear signed] M={M} K={K} N={N} G={G} form={rra.rrs_gemm_form(M, K, N, G)}")
    x, w, perm, bits, d = _case(M, K, N)
    ref = oracle.rrs_linear(x, w, perm, G, d)
    db = _dev_bits(bits)
    wq = torch.empty(rra.rrs_weight_bytes(K, N), dtype=torch.uint8, device=gu.DEV)
    rra.rrs_prepare_weights_signed(gu.to_dev(w), gu.to_dev(perm), db, wq)
    ws = torch.zeros(rra.rrs_workspace_bytes(M, K, G), dtype=torch.uint8, device=gu.DEV)
    rra.rrs_workspace_init(ws)
    Y = torch.empty(M, N, dtype=torch.float32, device=gu.DEV)
    rra.rrs_linear_signed(gu.to_dev(x), G, gu.to_dev(perm), db, wq, Y, ws)
    torch.cuda.synchronize()
    xq, dx, S = rra.workspace_views(ws, M, K, G)
    q_gpu = oracle.unpack_codes(xq.cpu().numpy())
    gu.compare_codes(q_gpu, ref["fe"]["q"], ref["fe"]["v"], "signed linear codes")
    codes, dw = rra.weight_views(wq, K, N)
    qw_gpu = oracle.unpack_codes(codes.cpu().numpy())
    gu.compare_codes(qw_gpu, ref["wp"]["qw"], ref["wp"]["uw"], "signed weight codes")
    gu.check_linear_two_way(Y.cpu().numpy(), ref, q_gpu, qw_gpu, dx.cpu().numpy(), S.cpu().numpy(),
                            dw.cpu().numpy(), G, "signed linear")


@pytest.mark.parametrize("M,K,N,G", [(64, 8192, 4096, 128), (7, 4096, 4096, 64)])
def test_linear_signed_prefetch_same_bits(M, K, N, G):
    """The signed layer with few tokens (its front end reads the weight codes
    ahead of the GEMM) gives the bits of rrs_frontend_signed followed by
    rrs_gemm."""
    gu.log(f"[signed linear prefetch] M={M} K={K} N={N} G={G}")
    x, w, perm, bits, _ = _case(M, K, N)
    X, P, db = gu.to_dev(x), gu.to_dev(perm), _dev_bits(bits)
    wq = torch.empty(rra.rrs_weight_bytes(K, N), dtype=torch.uint8, device=gu.DEV)
    rra.rrs_prepare_weights_signed(gu.to_dev(w), P, db, wq)
    ws = torch.zeros(rra.rrs_workspace_bytes(M, K, G), dtype=torch.uint8, device=gu.DEV)
    rra.rrs_workspace_init(ws)
    Y1 = torch.empty(M, N, dtype=torch.float32, device=gu.DEV)
    rra.rrs_linear_signed(X, G, P, db, wq, Y1, ws)
    torch.cuda.synchronize()
    gu.check_sync_block(ws, K, G, calls=1)
    xq1, dx1, S1 = (t.clone() for t in rra.workspace_regions(ws, M, K, G))
    sw = torch.zeros(rra.rrs_sync_bytes(K, G), dtype=torch.uint8, device=gu.DEV)
    rra.rrs_workspace_init(sw)
    xq2 = gu.xq_empty(M, K)
    dx2 = torch.empty(M, dtype=torch.float32, device=gu.DEV)
    S2 = torch.empty(K // G, dtype=torch.float32, device=gu.DEV)
    rra.rrs_frontend_signed(X, G, P, db, xq2, dx2, S2, sw)
    Y2 = torch.empty_like(Y1)
    rra.rrs_gemm(xq2, dx2, S2, G, wq, Y2)
    torch.cuda.synchronize()
    assert torch.equal(rra.codes_matrix(xq1, M, K), rra.codes_matrix(xq2, M, K))
    assert torch.equal(dx1, dx2) and torch.equal(S1, S2)
    assert torch.equal(Y1, Y2)
