"""GPU parity of each stage of the HIP path against the CPU oracle, on small
and ragged shapes that span several tiles (run on an MI355X: -m gpu)."""
import numpy as np
import pytest
import torch

import oracle
import rotated_runtime_activation_amd as rra
import workloads
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

# (M, K, G): K sweep 64..8192, G sweep 32..K, ragged token counts (not a
# multiple of the rows a wavefront handles when K < 4096, or of the GEMM tile)
FE_SHAPES = [
    (16, 256, 128), (1, 64, 32), (3, 64, 64), (17, 128, 32), (64, 256, 256), (5, 512, 128),
    (33, 1024, 1024), (7, 2048, 64), (2, 4096, 128), (9, 4096, 4096), (3, 4096, 32),
    (3, 8192, 128), (65, 8192, 32), (2, 8192, 8192), (300, 512, 64),
]


def _case(M, K, N=8, seed=None):
    seed = seed if seed is not None else M * 7919 + K
    x, xc, w = workloads.random_case(seed, M, K, N)
    perm = oracle.calibrate_perm(xc)
    return x, w, perm


@pytest.mark.parametrize("form", ["one-launch", "multi-launch"])
@pytest.mark.parametrize("M,K,G", FE_SHAPES)
def test_frontend(M, K, G, form):
    flags = rra.RRS_FLAG_TWO_PASS if form == "multi-launch" else 0
    passes = rra.rrs_frontend_passes(M, K, flags)
    gu.log(f"[frontend] M={M} K={K} G={G} {form}: {passes} launch(es)")
    assert passes == (3 if flags else 1)
    x, _, perm = _case(M, K)
    gu.check_frontend(x, perm, G, flags)


# Token counts at and past what the one-launch front end holds on chip (two
# blocks of 4096 elements per wave at K <= 4096, one block of 8192 at
# K = 8192): past it the same call falls back to three launches, whose
# passes loop each wave over several blocks (ragged at the end).
@pytest.mark.parametrize("M,K,G", [(4096, 4096, 128), (4200, 4096, 128), (8300, 2048, 64),
                                   (768, 8192, 128), (800, 8192, 256), (8192, 4096, 128), (2000, 8192, 64)])
def test_frontend_capacity(M, K, G):
    passes = rra.rrs_frontend_passes(M, K, 0)
    gu.log(f"[frontend capacity] M={M} K={K} G={G}: {passes} launch(es)")
    x, _, perm = _case(M, K)
    gu.check_frontend(x, perm, G)


# One row per workgroup (K = 1024 .. 8192, up to 256 rows) and the step to
# one row per wave past it; group sizes from 32 to a single group of K.
@pytest.mark.parametrize("M,K,G", [(1, 8192, 128), (255, 8192, 32), (256, 8192, 8192), (257, 8192, 128),
                                   (1, 4096, 4096), (256, 4096, 64), (257, 4096, 128),
                                   (1, 2048, 64), (256, 2048, 2048), (257, 2048, 128),
                                   (1, 1024, 1024), (255, 1024, 32), (64, 1024, 128),
                                   # past 256 rows at K = 1024: one row per wave (fused_kernel)
                                   (257, 1024, 128), (300, 1024, 32)])
@pytest.mark.parametrize("flags", [0, rra.RRS_FLAG_NO_SMOOTH, rra.RRS_FLAG_NO_ROTATE])
def test_frontend_rows_boundary(M, K, G, flags):
    gu.log(f"[frontend rows] M={M} K={K} G={G} flags={flags}: {rra.rrs_frontend_passes(M, K, flags)} launch(es)")
    assert rra.rrs_frontend_passes(M, K, flags) == 1
    x, _, perm = _case(M, K)
    gu.check_frontend(x, perm, G, flags)


def test_frontend_rows_workspace_reuse():
    """The row-per-workgroup form and the one-row-per-wave form share the
    synchronisation block's epoch and partial rows: calls of both in a row,
    with a smoothing-free call between."""
    K, G = 8192, 128
    ws = torch.zeros(rra.rrs_sync_bytes(K, G), dtype=torch.uint8, device=gu.DEV)
    rra.rrs_workspace_init(ws)
    calls = 0
    for M, flags in [(64, 0), (700, 0), (3, 0), (64, rra.RRS_FLAG_NO_SMOOTH), (256, 0), (300, 0), (1, 0)]:
        gu.log(f"[rows workspace reuse] M={M} flags={flags}")
        x, _, perm = _case(M, K)
        fe = oracle.frontend(x, perm, G, smooth=not (flags & 2))
        xq = gu.xq_empty(M, K)
        dx = torch.empty(M, dtype=torch.float32, device=gu.DEV)
        S = torch.empty(K // G, dtype=torch.float32, device=gu.DEV)
        rra.rrs_frontend(gu.to_dev(x), G, gu.to_dev(perm), xq, dx, S, ws, flags)
        torch.cuda.synchronize()
        if not flags and rra.rrs_frontend_passes(M, K, 0) == 1:
            calls += 1
        gu.check_sync_block(ws, K, G, calls)
        gu.compare_codes(oracle.unpack_codes(gu.xq_codes(xq, M, K)), fe["q"], fe["v"], "rows reuse codes")
        gu.rel_close(S.cpu().numpy(), fe["S"], gu.SCALE_TOL, "rows reuse S")


@pytest.mark.parametrize("M,K,G", [(40, 512, 64), (5, 4096, 128), (3, 8192, 256)])
@pytest.mark.parametrize("flags", [rra.RRS_FLAG_NO_ROTATE, rra.RRS_FLAG_NO_SMOOTH,
                                   rra.RRS_FLAG_NO_ROTATE | rra.RRS_FLAG_NO_SMOOTH])
def test_frontend_ablations(M, K, G, flags):
    gu.log(f"[frontend ablation] flags={flags} M={M} K={K} G={G}")
    x, _, perm = _case(M, K)
    gu.check_frontend(x, perm, G, flags)


def test_frontend_random_perm():
    gu.log("[frontend] shuffled permutation M=50 K=1024 G=128")
    x, _, _ = _case(50, 1024)
    gu.check_frontend(x, workloads.shuffled_perm(1024, 3), 128)


def test_frontend_zero_rows_and_groups():
    gu.log("[frontend] zero rows / all-zero input")
    K, G = 512, 64
    x, _, perm = _case(12, K)
    x[[0, 5, 11]] = 0
    fe, xq, dx, S, q, _ = gu.check_frontend(x, perm, G)
    assert np.all(dx[[0, 5, 11]] == 0) and not q[[0, 5, 11]].any()
    # all zero: every group scale guarded to 1, all codes 0
    z = np.zeros((7, K), dtype=np.float16)
    xq, dx, S = gu.frontend(z, perm, G)
    assert not xq.any() and not dx.any() and np.all(S == 1.0)
    # zero groups without rotation: groups with no nonzero channel -> 1
    z[:, perm[:G]] = 1.5
    gu.check_frontend(z, perm, G, rra.RRS_FLAG_NO_ROTATE)


def test_frontend_extreme_values():
    """fp16 extremes: spikes at +-65504 on two tokens (the two-outlier-token
    case the RRS summary lists as a limitation) and subnormal inputs."""
    gu.log("[frontend] fp16 extremes")
    K, G = 4096, 128
    x, _, perm = _case(20, K)
    x[3, 17] = np.float16(65504)
    x[11, 2000] = np.float16(-65504)
    x[5] = np.float16(6e-8)        # subnormal row
    gu.check_frontend(x, perm, G)


@pytest.mark.parametrize("K,N", [(256, 256), (64, 7), (512, 130), (4096, 300), (8192, 129)])
def test_prepare_weights(K, N):
    gu.log(f"[weights] K={K} N={N}")
    _, w, perm = _case(4, K, N)
    wq = gu.prepare_weights(w, perm)
    torch.cuda.synchronize()
    codes, dw = rra.weight_views(wq, K, N)
    ref = oracle.prepare_weights(w, perm)
    gu.compare_codes(oracle.unpack_codes(codes.cpu().numpy()), ref["qw"], ref["uw"], "weight codes")
    gu.rel_close(dw.cpu().numpy(), ref["dw"], gu.SCALE_TOL, "dw")


def test_prepare_weights_zero_column():
    gu.log("[weights] zero column")
    _, w, perm = _case(4, 512, 9)
    w[:, 4] = 0
    wq = gu.prepare_weights(w, perm)
    codes, dw = rra.weight_views(wq, 512, 9)
    torch.cuda.synchronize()
    assert not codes[4].any().item() and dw[4].item() == 0.0


# (M, N, K, G) for the grouped GEMM, fed oracle codes. M <= 64 with G >= 64
# runs the few-token kernel (K split over 8 waves, groups cut between
# waves: (32, 40, 128, 64), (48, 70, 1024, 256), (64, 33, 4096, 4096)).
GEMM_SHAPES = [
    (16, 256, 256, 128), (1, 1, 64, 32), (130, 200, 512, 32), (64, 64, 64, 64),
    (257, 129, 1024, 256), (128, 128, 4096, 4096), (33, 300, 2048, 128), (5, 17, 8192, 512),
    (1, 4096, 8192, 128), (32, 40, 128, 64), (48, 70, 1024, 256), (64, 33, 4096, 4096),
    (17, 257, 512, 64),
    # few-token kernel over several 64-token slices (grid y), ragged last slice
    (65, 260, 8192, 128), (200, 33, 2048, 64), (256, 300, 4096, 256), (500, 64, 4096, 128),
    # few-token kernel at G = 32 (two groups per k-step)
    (64, 260, 4096, 32), (130, 64, 8192, 32), (1, 33, 2048, 32),
    # few-token kernel with 4 .. 7 waves (K not a multiple of 2048)
    (64, 130, 5120, 128), (1, 96, 3072, 64), (33, 70, 7168, 256), (64, 40, 1024, 128),
    (130, 64, 2560, 512), (20, 50, 3072, 1024), (7, 33, 1536, 32),
]


# One shape for each few-token GEMM instantiation the shapes above leave
# out: token blocks (1 up to 32 tokens, else 2) x load rounds in flight (1
# for an odd, 2 for an even round count per wave) x the G class (32; 64;
# 128; 256 and up) x waves per workgroup (4 .. 8, fixed by K). The exact
# and partials tests run them bit for bit.
FEW_TOKEN_CLASSES = [
    (20, 41, 1024, 32), (20, 41, 1792, 32), (20, 41, 1024, 64), (20, 41, 1536, 64), (20, 41, 1792, 64),
    (20, 41, 2048, 64), (20, 41, 1024, 128), (20, 41, 1536, 128), (20, 41, 1792, 128), (20, 41, 2048, 128),
    (20, 41, 1024, 256), (20, 41, 1536, 256), (20, 41, 1792, 256), (20, 41, 2048, 256), (20, 41, 2560, 32),
    (20, 41, 3072, 32), (20, 41, 3584, 32), (20, 41, 4096, 32), (20, 41, 2560, 64), (20, 41, 3584, 64),
    (20, 41, 4096, 64), (20, 41, 2560, 128), (20, 41, 3072, 128), (20, 41, 3584, 128), (20, 41, 2560, 256),
    (20, 41, 3584, 256), (50, 42, 1024, 32), (50, 42, 1536, 32), (50, 42, 1792, 32), (50, 42, 2048, 32),
    (50, 42, 1024, 64), (50, 42, 1536, 64), (50, 42, 1792, 64), (50, 42, 1536, 128), (50, 42, 1792, 128),
    (50, 42, 1536, 256), (50, 42, 1792, 256), (50, 42, 2048, 256), (50, 42, 2560, 32), (50, 42, 3072, 32),
    (50, 42, 3584, 32), (50, 42, 2560, 64), (50, 42, 3072, 64), (50, 42, 3584, 64), (50, 42, 4096, 64),
    (50, 42, 3072, 128), (50, 42, 3584, 128), (50, 42, 3072, 256),
]

# The tiled kernel's instantiations with both sets of waves on K: G = 32
# (16 x 16 x 32 MFMA), G = 64 and 128 (rescale inside the product loop),
# G >= 256 (groups over several stages), one group split between the two
# sets (integer halves added before the scale), and an odd group count at a
# Kronecker K (set 1 takes the larger share).
TILED_CLASSES = [
    (700, 130, 1024, 32), (130, 260, 512, 64), (600, 300, 4096, 128), (130, 300, 512, 256),
    (700, 64, 2048, 2048), (600, 260, 1792, 256), (515, 257, 8192, 512),
]


def _random_codes(seed, M, N, K):
    g = np.random.default_rng(seed)
    q = g.integers(-7, 8, size=(M, K)).astype(np.int8)
    qw = g.integers(-7, 8, size=(N, K)).astype(np.int8)
    q[0, :] = 7      # extreme partials +-49 G
    qw[0, :] = -7
    return q, qw


@pytest.mark.parametrize("M,N,K,G", GEMM_SHAPES + FEW_TOKEN_CLASSES + TILED_CLASSES)
def test_gemm_partials_exact(M, N, K, G):
    """rrs_gemm_partials runs the instantiation rrs_gemm runs for the shape
    (its K split and rescale points, the accumulator multiplied by 0 where
    it would be rescaled): its partials must equal the int64 brute force."""
    gu.log(f"[gemm partials] M={M} N={N} K={K} G={G} form={rra.rrs_gemm_form(M, K, N, G)}")
    q, qw = _random_codes(M + N + K, M, N, K)
    xq = gu.xq_buffer(oracle.pack_codes(q))
    wq = gu.weight_buffer_from_codes(oracle.pack_codes(qw), np.ones(N))
    ref = oracle.group_partials(q, qw, G)
    for (m0, m1, n0, n1) in {(0, M, 0, N), (M // 2, M, N // 3, N), (M - 1, M, N - 1, N)}:
        P = torch.empty(m1 - m0, n1 - n0, K // G, dtype=torch.int32, device=gu.DEV)
        rra.rrs_gemm_partials(xq, M, K, N, G, wq, m0, m1, n0, n1, P)
        torch.cuda.synchronize()
        got = P.cpu().numpy()
        assert np.array_equal(got, ref[m0:m1, n0:n1]), \
            f"partials differ in window {(m0, m1, n0, n1)}: {int((got != ref[m0:m1, n0:n1]).sum())} entries"


@pytest.mark.parametrize("M,N,K,G", GEMM_SHAPES)
def test_gemm_output(M, N, K, G):
    gu.log(f"[gemm Y] M={M} N={N} K={K} G={G} form={rra.rrs_gemm_form(M, K, N, G)}")
    q, qw = _random_codes(M * 3 + N + K, M, N, K)
    g = np.random.default_rng(K + M)
    dx = (g.random(M) + 0.1).astype(np.float32)
    dw = (g.random(N) * 0.01 + 1e-3).astype(np.float32)
    S = (g.random(K // G) * 100 + 1).astype(np.float32)
    ref = oracle.linear_out(q, dx.astype(np.float64), S.astype(np.float64), qw, dw.astype(np.float64), G)
    Y = torch.empty(M, N, dtype=torch.float32, device=gu.DEV)
    rra.rrs_gemm(gu.xq_buffer(oracle.pack_codes(q)), gu.to_dev(dx), gu.to_dev(S), G,
                 gu.weight_buffer_from_codes(oracle.pack_codes(qw), dw), Y)
    torch.cuda.synchronize()
    err = gu.y_error(Y.cpu().numpy(), ref)
    gu.log(f"  Y err/C = {err:.3e} (bound {gu.y_tol(K, G):.2e})")
    assert err <= gu.y_tol(K, G)


def _exact_codes(seed, M, N, K):
    """Random codes whose worst output keeps every partial sum of the
    product chain below 2^18 units (|q qw| summed over K), so that with the
    group scales powers of two up to 8 every fp32 value on the chain is an
    exact multiple of 2^-21 below 8."""
    q, qw = _random_codes(seed, M, N, K)
    if 49 * K >= 1 << 18:  # the all-7 rows would exceed it: moderate them
        q[0, :] = 3
        qw[0, :] = -3
    worst = (np.abs(q.astype(np.int64)) @ np.abs(qw.astype(np.int64)).T).max()
    assert worst < 1 << 18
    return q, qw


@pytest.mark.parametrize("M,N,K,G", GEMM_SHAPES + FEW_TOKEN_CLASSES + TILED_CLASSES)
def test_gemm_exact_through_product_kernels(M, N, K, G):
    """The kernels that produce Y, checked bit for bit: with dx = dw = 1 and
    group scales that are powers of two (neighbouring groups always
    different: a product counted in the wrong group changes the sum), every
    rescale, partial sum and epilogue product is exact in fp32 up to the one
    product by the output scale: Y = fl32(X fl32(2^18 / K)) with X =
    2^-18 sum_g S_g P_g exact (for K a power of two, K Y = sum_g S_g P_g
    exactly). A dropped, doubled or misplaced product anywhere in the main
    loop, the K split or the epilogue shows as a mismatch."""
    gu.log(f"[gemm exact Y] M={M} N={N} K={K} G={G} form={rra.rrs_gemm_form(M, K, N, G)}")
    q, qw = _exact_codes(M * 5 + N + K, M, N, K)
    ng = K // G
    S = np.array([2.0 ** ((3 * g + M) % 4) for g in range(ng)], dtype=np.float32)
    Y = torch.empty(M, N, dtype=torch.float32, device=gu.DEV)
    rra.rrs_gemm(gu.xq_buffer(oracle.pack_codes(q)), gu.to_dev(np.ones(M, np.float32)), gu.to_dev(S), G,
                 gu.weight_buffer_from_codes(oracle.pack_codes(qw), np.ones(N)), Y)
    torch.cuda.synchronize()
    total = (oracle.group_partials(q, qw, G) * S.astype(np.int64)[None, None, :]).sum(axis=2)
    assert np.abs(total).max() < 1 << 24          # X is exact in fp32
    x32 = (total.astype(np.float64) * 2.0 ** -18).astype(np.float32)
    want = x32 * (np.float32(2.0 ** 18) / np.float32(K))  # one fp32 rounding
    if K & (K - 1) == 0:
        assert np.array_equal(want.astype(np.float64) * K, total)
    got = Y.cpu().numpy()
    bad = got != want
    assert not bad.any(), f"{int(bad.sum())} outputs differ, first {np.argwhere(bad)[:3].tolist()}"


@pytest.mark.parametrize("M,K,N,G", [(16, 256, 256, 128), (45, 1024, 300, 64), (3, 8192, 129, 32),
                                     (130, 4096, 260, 4096), (1, 64, 1, 32)])
def test_linear_end_to_end(M, K, N, G):
    gu.log(f"[linear] M={M} K={K} N={N} G={G}")
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
    gu.compare_codes(q_gpu, ref["fe"]["q"], ref["fe"]["v"], "linear codes")
    codes, dw = rra.weight_views(wq, K, N)
    qw_gpu = oracle.unpack_codes(codes.cpu().numpy())
    gu.compare_codes(qw_gpu, ref["wp"]["qw"], ref["wp"]["uw"], "weight codes")
    gu.check_linear_two_way(Y.cpu().numpy(), ref, q_gpu, qw_gpu, dx.cpu().numpy(), S.cpu().numpy(),
                            dw.cpu().numpy(), G, "linear")


def test_determinism():
    gu.log("[determinism] two identical rrs_linear calls")
    M, K, N, G = 200, 4096, 512, 128
    x, w, perm = _case(M, K, N)
    wq = gu.prepare_weights(w, perm)
    ws = torch.zeros(rra.rrs_workspace_bytes(M, K, G), dtype=torch.uint8, device=gu.DEV)
    rra.rrs_workspace_init(ws)
    X, P = gu.to_dev(x), gu.to_dev(perm)
    Y1 = torch.empty(M, N, dtype=torch.float32, device=gu.DEV)
    Y2 = torch.empty_like(Y1)
    rra.rrs_linear(X, G, P, wq, Y1, ws)
    xq1 = rra.workspace_views(ws, M, K, G)[0].clone()
    rra.rrs_linear(X, G, P, wq, Y2, ws)
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y2)
    assert torch.equal(xq1, rra.workspace_views(ws, M, K, G)[0])


@pytest.mark.parametrize("M,K,N,G", [(64, 8192, 8192, 128), (1, 8192, 4096, 32), (16, 4096, 4096, 128),
                                     (100, 2048, 4096, 64), (192, 8192, 8192, 128), (200, 1024, 2048, 128),
                                     (2048, 4096, 4096, 128), (700, 1024, 1000, 64), (4096, 4096, 512, 128)])
def test_linear_prefetch_same_bits(M, K, N, G):
    """rrs_linear's front end reads the GEMM's weight codes ahead: with few
    tokens on extra workgroups where enough compute units are idle (at
    M = 192, K = N = 8192 it does not), before the tiled GEMM in the
    one-launch form's own threads (with one block per wave: not at M = 4096,
    K = 4096). The layer's outputs must be the bits of rrs_frontend followed
    by rrs_gemm, which never read ahead, and the grid-wide wait must not give
    up."""
    gu.log(f"[linear prefetch] M={M} K={K} N={N} G={G}")
    x, w, perm = _case(M, K, N)
    wq = gu.prepare_weights(w, perm)
    X, P = gu.to_dev(x), gu.to_dev(perm)
    ws = torch.zeros(rra.rrs_workspace_bytes(M, K, G), dtype=torch.uint8, device=gu.DEV)
    rra.rrs_workspace_init(ws)
    Y1 = torch.empty(M, N, dtype=torch.float32, device=gu.DEV)
    rra.rrs_linear(X, G, P, wq, Y1, ws)
    torch.cuda.synchronize()
    gu.check_sync_block(ws, K, G, calls=1 if rra.rrs_frontend_passes(M, K, 0) == 1 else 0)
    xq1, dx1, S1 = (t.clone() for t in rra.workspace_regions(ws, M, K, G))
    sw = torch.zeros(rra.rrs_sync_bytes(K, G), dtype=torch.uint8, device=gu.DEV)
    rra.rrs_workspace_init(sw)
    xq2 = gu.xq_empty(M, K)
    dx2 = torch.empty(M, dtype=torch.float32, device=gu.DEV)
    S2 = torch.empty(K // G, dtype=torch.float32, device=gu.DEV)
    rra.rrs_frontend(X, G, P, xq2, dx2, S2, sw)
    Y2 = torch.empty_like(Y1)
    rra.rrs_gemm(xq2, dx2, S2, G, wq, Y2)
    torch.cuda.synchronize()
    # the codes of the M rows (an odd M leaves the pad row of the last pair unwritten)
    assert torch.equal(rra.codes_matrix(xq1, M, K), rra.codes_matrix(xq2, M, K))
    assert torch.equal(dx1, dx2) and torch.equal(S1, S2)
    assert torch.equal(Y1, Y2)


def test_frontend_workspace_reuse_across_sizes():
    """One synchronisation block serves calls of different token counts in a
    row (the one-launch form's grid changes size between calls: rows of
    workgroups a smaller call does not use keep older epoch tags and must
    not be read), on both forms and after a smoothing-free call."""
    K, G = 4096, 128
    ws = torch.zeros(rra.rrs_sync_bytes(K, G), dtype=torch.uint8, device=gu.DEV)
    rra.rrs_workspace_init(ws)
    calls = 0
    for M, flags in [(2048, 0), (64, 0), (1000, 0), (300, rra.RRS_FLAG_TWO_PASS), (2048, 0),
                     (5, rra.RRS_FLAG_NO_SMOOTH), (777, 0)]:
        gu.log(f"[workspace reuse] M={M} flags={flags}")
        x, _, perm = _case(M, K)
        fe = oracle.frontend(x, perm, G, smooth=not (flags & 2))
        xq = gu.xq_empty(M, K)
        dx = torch.empty(M, dtype=torch.float32, device=gu.DEV)
        S = torch.empty(K // G, dtype=torch.float32, device=gu.DEV)
        rra.rrs_frontend(gu.to_dev(x), G, gu.to_dev(perm), xq, dx, S, ws, flags)
        torch.cuda.synchronize()
        if not flags and rra.rrs_frontend_passes(M, K, 0) == 1:
            calls += 1
        gu.check_sync_block(ws, K, G, calls)
        gu.compare_codes(oracle.unpack_codes(gu.xq_codes(xq, M, K)), fe["q"], fe["v"], "reuse codes")
        gu.rel_close(S.cpu().numpy(), fe["S"], gu.SCALE_TOL, "reuse S")


@pytest.mark.parametrize("T,K", [(128, 256), (512, 4096), (100, 8192), (3, 64)])
def test_calibrate_perm(T, K):
    gu.log(f"[calibrate] T={T} K={K}")
    wl = workloads.Workload(20_000 + K, "cal", T, K, 8, (K,), 8, 20.0, "count", 3, 500.0, 0.02, T)
    xc = workloads.make_activations(wl, T, wl.seed_base + workloads.ROLE_CALIB)
    ref = oracle.calibrate_perm(xc)
    perm = torch.empty(K, dtype=torch.int32, device=gu.DEV)
    ws = torch.empty(rra.rrs_calibrate_workspace_bytes(K), dtype=torch.uint8, device=gu.DEV)
    rra.rrs_calibrate_perm(gu.to_dev(xc), perm, ws)
    torch.cuda.synchronize()
    got = perm.cpu().numpy()
    assert np.array_equal(np.sort(got), np.arange(K))
    # the order is unique where channel maxima differ by more than fp32
    # rounding of the rotation; near-ties may swap
    c = np.abs(oracle.fwht(xc)).max(axis=0)
    cs = c[got]
    assert np.all(cs[:-1] >= cs[1:] * (1 - 1e-5) - 1e-30)
    same = got == ref
    if not same.all():
        idx = np.nonzero(~same)[0]
        assert np.all(np.abs(c[got[idx]] - c[ref[idx]]) <= 1e-5 * c[ref[idx]])
    gu.log(f"  perm positions differing from the oracle (near-ties): {int((~same).sum())}")
