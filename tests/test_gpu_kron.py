"""GPU parity of the Kronecker rotation H_m (x) H_n for K = m 2^k,
m in {12, 20, 28} (reading R19), against the oracle: front end (with
ablations and signs), weight preparation, calibration, the grouped GEMM at
such K (including an odd number of groups, where the two halves of K meet
off the middle) and the whole layer (run on an MI355X: -m gpu)."""
import numpy as np
import pytest
import torch

import oracle
import rotated_runtime_activation_amd as rra
import workloads
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _case(M, K, N=8):
    x, xc, w = workloads.random_case(M * 131 + K, M, K, N)
    perm = oracle.calibrate_perm(xc)
    return x, w, perm


# (M, K, G): every m, n from 64 to the largest built, odd group counts
KRON_FE = [
    (16, 768, 64), (5, 1280, 256), (33, 1792, 128), (7, 3072, 1024), (40, 5120, 32),
    (3, 14336, 128), (130, 14336, 2048), (9, 12288, 4096), (2, 10240, 512), (300, 1536, 64),
    (300, 12288, 128), (270, 5120, 64),
]


@pytest.mark.parametrize("M,K,G", KRON_FE)
def test_frontend_kron(M, K, G):
    gu.log(f"[frontend kron] M={M} K={K} G={G} (m, n) = {oracle.kron_split(K)}: {rra.rrs_frontend_passes(M, K, 0)} launches")
    x, _, perm = _case(M, K)
    gu.check_frontend(x, perm, G)


@pytest.mark.parametrize("flags", [rra.RRS_FLAG_NO_ROTATE, rra.RRS_FLAG_NO_SMOOTH])
def test_frontend_kron_ablations(flags):
    M, K, G = 21, 3584, 128   # 28 * 128
    gu.log(f"[frontend kron ablation] flags={flags} M={M} K={K} G={G}")
    x, _, perm = _case(M, K)
    gu.check_frontend(x, perm, G, flags)


@pytest.mark.parametrize("M,K,G", [(11, 1792, 64), (6, 14336, 256), (9, 12288, 128), (5, 5120, 64),
                                   (3, 1536, 32), (300, 14336, 128), (1, 14336, 128)])
def test_frontend_kron_signed(M, K, G):
    gu.log(f"[frontend kron signed] M={M} K={K} G={G}")
    x, _, perm = _case(M, K)
    bits = np.random.default_rng(K).integers(0, 2**32, size=K // 32, dtype=np.uint64).astype(np.uint32)
    d = oracle.signs_from_bits(bits, K)
    fe = oracle.frontend(x, perm, G, d=d)
    xq = gu.xq_empty(M, K)
    dx = torch.empty(M, dtype=torch.float32, device=gu.DEV)
    S = torch.empty(K // G, dtype=torch.float32, device=gu.DEV)
    ws = torch.zeros(rra.rrs_sync_bytes(K, G), dtype=torch.uint8, device=gu.DEV)
    rra.rrs_frontend_signed(gu.to_dev(x), G, gu.to_dev(perm), gu.to_dev(bits.view(np.int32)), xq, dx, S, ws)
    torch.cuda.synchronize()
    gu.compare_codes(oracle.unpack_codes(gu.xq_codes(xq, M, K)), fe["q"], fe["v"], "kron signed codes")
    gu.rel_close(dx.cpu().numpy(), fe["dx"], gu.SCALE_TOL, "kron signed dx")
    gu.rel_close(S.cpu().numpy(), fe["S"], gu.SCALE_TOL, "kron signed S")


@pytest.mark.parametrize("K,N", [(768, 40), (1792, 7), (14336, 96), (12288, 33), (5120, 24), (1536, 17)])
def test_prepare_weights_kron(K, N):
    gu.log(f"[weights kron] K={K} N={N}")
    _, w, perm = _case(4, K, N)
    wq = gu.prepare_weights(w, perm)
    torch.cuda.synchronize()
    codes, dw = rra.weight_views(wq, K, N)
    ref = oracle.prepare_weights(w, perm)
    gu.compare_codes(oracle.unpack_codes(codes.cpu().numpy()), ref["qw"], ref["uw"], "kron weight codes")
    gu.rel_close(dw.cpu().numpy(), ref["dw"], gu.SCALE_TOL, "kron dw")


@pytest.mark.parametrize("T,K", [(64, 768), (200, 14336), (100, 12288), (50, 3072)])
def test_calibrate_perm_kron(T, K):
    gu.log(f"[calibrate kron] T={T} K={K}")
    wl = workloads.Workload(40_000 + K, "cal", T, K, 8, (K,), 8, 20.0, "count", 3, 500.0, 0.02, T)
    xc = workloads.make_activations(wl, T, wl.seed_base + workloads.ROLE_CALIB)
    ref = oracle.calibrate_perm(xc)
    perm = torch.empty(K, dtype=torch.int32, device=gu.DEV)
    ws = torch.empty(rra.rrs_calibrate_workspace_bytes(K), dtype=torch.uint8, device=gu.DEV)
    rra.rrs_calibrate_perm(gu.to_dev(xc), perm, ws)
    torch.cuda.synchronize()
    got = perm.cpu().numpy()
    assert np.array_equal(np.sort(got), np.arange(K))
    c = np.abs(oracle.rotate_rows(xc)).max(axis=0)
    cs = c[got]
    assert np.all(cs[:-1] >= cs[1:] * (1 - 1e-5) - 1e-30)
    same = got == ref
    if not same.all():
        idx = np.nonzero(~same)[0]
        assert np.all(np.abs(c[got[idx]] - c[ref[idx]]) <= 1e-5 * c[ref[idx]])


@pytest.mark.parametrize("M,N,K,G", [(33, 130, 14336, 2048), (130, 64, 1792, 128), (5, 260, 12288, 32),
                                     (64, 40, 14336, 1024),
                                     # few-token kernel at K = m 2^k (odd and even round counts)
                                     (64, 130, 14336, 128), (1, 33, 14336, 256), (40, 96, 12288, 512),
                                     (100, 70, 10240, 64), (3, 64, 6144, 128)])
def test_gemm_kron(M, N, K, G):
    gu.log(f"[gemm kron] M={M} N={N} K={K} G={G} groups={K // G} form={rra.rrs_gemm_form(M, K, N, G)}")
    g = np.random.default_rng(M + N + K)
    q = g.integers(-7, 8, size=(M, K)).astype(np.int8)
    qw = g.integers(-7, 8, size=(N, K)).astype(np.int8)
    dx = (g.random(M) + 0.1).astype(np.float32)
    dw = (g.random(N) * 0.01 + 1e-3).astype(np.float32)
    S = (g.random(K // G) * 100 + 1).astype(np.float32)
    xq = gu.xq_buffer(oracle.pack_codes(q))
    wq = gu.weight_buffer_from_codes(oracle.pack_codes(qw), dw)
    ref = oracle.linear_out(q, dx.astype(np.float64), S.astype(np.float64), qw, dw.astype(np.float64), G)
    Y = torch.empty(M, N, dtype=torch.float32, device=gu.DEV)
    rra.rrs_gemm(xq, gu.to_dev(dx), gu.to_dev(S), G, wq, Y)
    P = torch.empty(M, N, K // G, dtype=torch.int32, device=gu.DEV)
    rra.rrs_gemm_partials(xq, M, K, N, G, wq, 0, M, 0, N, P)
    torch.cuda.synchronize()
    assert np.array_equal(P.cpu().numpy(), oracle.group_partials(q, qw, G))
    err = gu.y_error(Y.cpu().numpy(), ref)
    gu.log(f"  Y err/C = {err:.3e} (bound {gu.y_tol(K, G):.2e})")
    assert err <= gu.y_tol(K, G)


@pytest.mark.parametrize("M,K,N,G", [(48, 14336, 130, 128), (7, 1280, 64, 64),
                                     # one-launch Kronecker front end, few-token GEMM with 5 waves over 4 slices
                                     (200, 5120, 96, 128)])
def test_linear_kron(M, K, N, G):
    gu.log(f"[linear kron] M={M} K={K} N={N} G={G}")
    x, w, perm = _case(M, K, N)
    ref = oracle.rrs_linear(x, w, perm, G)
    wq = gu.prepare_weights(w, perm)
    ws = torch.zeros(rra.rrs_workspace_bytes(M, K, G), dtype=torch.uint8, device=gu.DEV)
    rra.rrs_workspace_init(ws)
    Y = torch.empty(M, N, dtype=torch.float32, device=gu.DEV)
    rra.rrs_linear(gu.to_dev(x), G, gu.to_dev(perm), wq, Y, ws)
    torch.cuda.synchronize()
    xq, dx, S = rra.workspace_views(ws, M, K, G)
    q_gpu = oracle.unpack_codes(xq.cpu().numpy())
    gu.compare_codes(q_gpu, ref["fe"]["q"], ref["fe"]["v"], "kron linear codes")
    codes, dw = rra.weight_views(wq, K, N)
    qw_gpu = oracle.unpack_codes(codes.cpu().numpy())
    gu.compare_codes(qw_gpu, ref["wp"]["qw"], ref["wp"]["uw"], "kron weight codes")
    gu.check_linear_two_way(Y.cpu().numpy(), ref, q_gpu, qw_gpu, dx.cpu().numpy(), S.cpu().numpy(),
                            dw.cpu().numpy(), G, "kron linear")


@pytest.mark.parametrize("M,K,G,signed", [(37, 14336, 128, False), (300, 1536, 64, False), (11, 1792, 64, True),
                                          (1, 14336, 256, False), (2, 12288, 4096, False), (257, 10240, 512, True),
                                          (3, 768, 256, False), (40, 5120, 32, False), (64, 7168, 1024, True)])
def test_frontend_kron_row_area(M, K, G, signed):
    """With an rrs_linear-sized workspace the stats pass keeps the rotated,
    reordered rows in its row area and the quantise pass streams them: the
    same bits as the form that rotates every row twice, the rows themselves
    close to the exact ones, and no row area used when xq lies in it."""
    gu.log(f"[frontend kron rows] M={M} K={K} G={G} signed={signed}")
    x, _, perm = _case(M, K)
    X, P = gu.to_dev(x), gu.to_dev(perm)
    dsign_np = (np.random.default_rng(K + M).integers(0, 2**32, size=K // 32, dtype=np.uint64)
                .astype(np.uint32)) if signed else None
    D = gu.to_dev(dsign_np.view(np.int32)) if signed else None

    # three launches forced: the row area belongs to that form (few rows
    # otherwise take the one-launch form, compared with it at the end)
    def run(xq, dx, S, ws, flags=rra.RRS_FLAG_TWO_PASS):
        if signed:
            rra.rrs_frontend_signed(X, G, P, D, xq, dx, S, ws, flags)
        else:
            rra.rrs_frontend(X, G, P, xq, dx, S, ws, flags)
        torch.cuda.synchronize()

    # rotate twice: a workspace of the synchronisation block alone
    xq_a = gu.xq_empty(M, K)
    dx_a = torch.empty(M, dtype=torch.float32, device=gu.DEV)
    S_a = torch.empty(K // G, dtype=torch.float32, device=gu.DEV)
    ws_a = torch.zeros(rra.rrs_sync_bytes(K, G), dtype=torch.uint8, device=gu.DEV)
    run(xq_a, dx_a, S_a, ws_a)

    # stored rows: a whole rrs_linear workspace, outputs in its own views
    nbytes = rra.rrs_workspace_bytes(M, K, G)
    ws_b = torch.zeros(nbytes, dtype=torch.uint8, device=gu.DEV)
    xq_b, dx_b, S_b = rra.workspace_regions(ws_b, M, K, G)
    run(xq_b, dx_b, S_b, ws_b)
    row_off = nbytes - (4 * M * K + 255) // 256 * 256
    rows = ws_b[row_off:].view(torch.float32).view(M, K).cpu().numpy().astype(np.float64)

    codes_a = rra.codes_matrix(xq_a, M, K)
    assert torch.equal(codes_a, rra.codes_matrix(xq_b, M, K)), "codes differ between the two forms"
    assert torch.equal(dx_a.view(torch.int32), dx_b.view(torch.int32)), "dx differs between the two forms"
    assert torch.equal(S_a.view(torch.int32), S_b.view(torch.int32)), "S differs between the two forms"

    fe = oracle.frontend(x, perm, G, d=oracle.signs_from_bits(dsign_np, K)) if signed else oracle.frontend(x, perm, G)
    gu.compare_codes(oracle.unpack_codes(gu.xq_codes(xq_b, M, K)), fe["q"], fe["v"], "kron rows codes")
    gu.rel_close(dx_b.cpu().numpy(), fe["dx"], gu.SCALE_TOL, "kron rows dx")
    gu.rel_close(S_b.cpu().numpy(), fe["S"], gu.SCALE_TOL, "kron rows S")
    scale = np.maximum(np.abs(fe["Zp"]).max(axis=1, keepdims=True), 1e-30)
    err = float((np.abs(rows - fe["Zp"]) / scale).max())
    gu.log(f"  stored rows: max |row - Zp| / max|Zp row| = {err:.3e}")
    assert err <= 1e-5

    # xq inside the row area: the library must not keep rows there
    ws_c = torch.zeros(nbytes, dtype=torch.uint8, device=gu.DEV)
    xq_c = ws_c[row_off: row_off + rra.rrs_codes_bytes(M, K)]
    dx_c = torch.empty(M, dtype=torch.float32, device=gu.DEV)
    S_c = torch.empty(K // G, dtype=torch.float32, device=gu.DEV)
    run(xq_c, dx_c, S_c, ws_c)
    assert torch.equal(codes_a, rra.codes_matrix(xq_c, M, K)) and torch.equal(dx_a, dx_c) and torch.equal(S_a, S_c)

    # the default form (one launch for up to one row per CU): the same bits
    ws_d = torch.zeros(nbytes, dtype=torch.uint8, device=gu.DEV)
    xq_d, dx_d, S_d = rra.workspace_regions(ws_d, M, K, G)
    gu.log(f"  default form: {rra.rrs_frontend_passes(M, K, 0)} launch(es)")
    run(xq_d, dx_d, S_d, ws_d, 0)
    assert torch.equal(codes_a, rra.codes_matrix(xq_d, M, K)) and torch.equal(dx_a, dx_d) and torch.equal(S_a, S_d)
    gu.check_sync_block(ws_d, K, G)


def test_frontend_kron_workspace_reuse():
    """One synchronisation block across Kronecker calls of several sizes,
    one-launch (few rows) and three-launch (more rows, or forced) mixed: the
    epoch counts the one-launch calls and every call matches the oracle."""
    K, G = 1792, 64
    ws = torch.zeros(rra.rrs_sync_bytes(K, G), dtype=torch.uint8, device=gu.DEV)
    rra.rrs_workspace_init(ws)
    one = 0
    for M, flags in [(5, 0), (200, 0), (1, 0), (300, 0), (64, rra.RRS_FLAG_TWO_PASS), (64, 0), (256, 0)]:
        passes = rra.rrs_frontend_passes(M, K, flags)
        gu.log(f"[kron workspace reuse] M={M} flags={flags}: {passes} launch(es)")
        x, _, perm = _case(M, K)
        fe = oracle.frontend(x, perm, G)
        xq = gu.xq_empty(M, K)
        dx = torch.empty(M, dtype=torch.float32, device=gu.DEV)
        S = torch.empty(K // G, dtype=torch.float32, device=gu.DEV)
        rra.rrs_frontend(gu.to_dev(x), G, gu.to_dev(perm), xq, dx, S, ws, flags)
        torch.cuda.synchronize()
        one += passes == 1
        gu.compare_codes(oracle.unpack_codes(gu.xq_codes(xq, M, K)), fe["q"], fe["v"], "kron reuse codes")
        gu.rel_close(dx.cpu().numpy(), fe["dx"], gu.SCALE_TOL, "kron reuse dx")
        gu.rel_close(S.cpu().numpy(), fe["S"], gu.SCALE_TOL, "kron reuse S")
        words = ws.view(torch.int32).cpu().numpy()
        assert words[2] == 0, "a bounded wait gave up (error word set)"
        assert words[3] == one, f"epoch {words[3]} after {one} one-launch call(s)"
    assert one >= 4, "few-row calls take the one-launch form"
