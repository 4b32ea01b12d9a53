"""Pins of the CPU oracle against the pages' definitions, closed forms,
invariants, a hand-worked example and brute force (CPU only)."""
import numpy as np
import pytest
import scipy.linalg

import oracle
import workloads
from tests import pins


# ------------------------------------------------------------------ FWHT
@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 64, 256, 1024])
def test_hadamard_orthogonality(n):
    H = pins.hadamard_popcount(n)
    assert np.array_equal(H @ H.T, n * np.eye(n))


@pytest.mark.parametrize("n", [2, 8, 64, 512])
def test_popcount_matrix_is_scipy_sylvester(n):
    assert np.array_equal(pins.hadamard_popcount(n), scipy.linalg.hadamard(n))


def test_fwht_bit_exact_vs_explicit_matmul():
    assert pins.fwht_matches_explicit(oracle.fwht)


def test_fwht_unit_vectors():
    assert pins.fwht_unit_vectors(oracle.fwht)


@pytest.mark.parametrize("n", [4096, 8192])
def test_fwht_sampled_columns_large(n):
    g = np.random.default_rng(n)
    x = (g.standard_normal((3, n)) * np.where(g.random(n) < 0.01, 300, 1)).astype(np.float16)
    z = oracle.fwht(x)
    for j in g.choice(n, size=6, replace=False):
        col = pins.hadamard_column(n, int(j))
        assert np.array_equal(z[:, j], x.astype(np.float64) @ col)


def test_fwht_involution_and_parseval():
    g = np.random.default_rng(3)
    x = g.standard_normal((4, 2048)).astype(np.float16).astype(np.float64)
    z = oracle.fwht(x)
    assert np.array_equal(oracle.fwht(z), 2048 * x)
    assert np.allclose((z * z).sum(1), 2048 * (x * x).sum(1), rtol=1e-13)


def test_fwht_rejects_non_power_of_two():
    with pytest.raises(ValueError):
        oracle.fwht(np.ones((2, 12)))


# -------------------------------------------------------------- front end
def test_frontend_golden():
    assert pins.frontend_matches_golden(oracle.frontend)


def test_weights_golden():
    assert pins.weights_match_golden(oracle.prepare_weights)


def test_gemm_golden():
    assert pins.gemm_matches_golden(oracle.group_partials, oracle.linear_out)


def test_pack_golden_and_roundtrip():
    assert pins.pack_matches_golden(oracle.pack_codes)
    q = np.random.default_rng(0).integers(-7, 8, size=(5, 64)).astype(np.int8)
    assert np.array_equal(oracle.unpack_codes(oracle.pack_codes(q)), q)


def test_unrounded_output_equals_xw():
    assert pins.unrounded_output_is_xw(oracle.frontend, oracle.prepare_weights, oracle.linear_out)


def _case(seed=5, M=40, K=512, G=64):
    wl = workloads.WORKLOADS["tiny"]
    x, xc, w = workloads.random_case(seed, M, K, 16)
    perm = oracle.calibrate_perm(xc)
    return x, perm, G


def test_invariants_I1_I2_I3_I4():
    x, perm, G = _case()
    fe = oracle.frontend(x, perm, G)
    U, r, q, S = fe["U"], fe["r"], fe["q"], fe["S"]
    K = x.shape[1]
    # I1: every group reaches |U| == 1 exactly (x / x == 1 in IEEE).
    Ug = np.abs(U).reshape(U.shape[0], K // G, G)
    assert np.all(Ug.max(axis=(0, 2)) == 1.0)
    # I2: smoothing bounds every entry by 1.
    assert np.abs(U).max() <= 1.0
    # I3: each nonzero row has a +-7 code at its |U| argmax.
    am = np.argmax(np.abs(U), axis=1)
    assert np.all(np.abs(q[np.arange(len(q)), am]) == 7)
    # I4: RTN error at most half a step.
    err = np.abs(U - (r[:, None] / 7) * q)
    assert np.all(err <= r[:, None] / 14 * (1 + 1e-12))


def test_I5_single_group_is_per_token_rtn():
    """G = K: S is one scalar, so the codes are plain per-token symmetric RTN
    of the rotated, reordered row ([AGC-OR] Sec. 3.1 quantiser)."""
    x, perm, _ = _case()
    K = x.shape[1]
    fe = oracle.frontend(x, perm, K)
    Zp = pins.hadamard_popcount(K)
    Zp = (x.astype(np.float64) @ Zp)[:, perm]
    delta = np.abs(Zp).max(axis=1) / 7
    ref = np.clip(np.rint(Zp / delta[:, None]), -7, 7)
    # the two formulas differ by float64 rounding of the divide chain; compare
    # away from .5 boundaries
    ok = ~oracle.near_half(fe["v"], 1e-9)
    assert np.array_equal(fe["q"][ok], ref[ok])


def test_I6_single_token():
    x, perm, G = _case(M=1)
    fe = oracle.frontend(x[:1], perm, G)
    assert fe["r"][0] == 1.0


def test_unsmoothing_roundtrip_exact_for_power_of_two_scales():
    # Group maxima that are powers of two make U * S == Zp exact (the
    # rotation is switched off so the smoothed values are chosen directly).
    K, G = 64, 16
    g = np.random.default_rng(9)
    X = g.integers(-31, 32, size=(6, K)).astype(np.float64) / 64.0
    X[0, ::G] = [1.0, 2.0, 0.5, 4.0]   # one power-of-two maximum per group
    X = X.astype(np.float16)
    perm = np.arange(K, dtype=np.int32)
    fe = oracle.frontend(X, perm, G, rotate=False)
    assert np.array_equal(fe["S"], [1.0, 2.0, 0.5, 4.0])
    assert np.array_equal(fe["U"] * np.repeat(fe["S"], G), fe["Zp"])


def test_unsmoothing_roundtrip_one_ulp_general():
    x, perm, G = _case(seed=11)
    fe = oracle.frontend(x, perm, G)
    back = fe["U"] * np.repeat(fe["S"], G)
    assert np.all(np.abs(back - fe["Zp"]) <= np.spacing(np.abs(fe["Zp"])) + 0)


def test_reorder_identity():
    """sum_j Zp[:, j] Wp[j, :] / K == X W  ([RRS-rebuttal] reorder answer)."""
    g = np.random.default_rng(2)
    K, N = 256, 10
    x = g.standard_normal((7, K)).astype(np.float16)
    W = (g.standard_normal((K, N)) * 0.02).astype(np.float16)
    perm = g.permutation(K).astype(np.int32)
    Zp = oracle.fwht(x)[:, perm]
    Wp_t = oracle.prepare_weights(W, perm)["Wp_t"]
    lhs = Zp @ Wp_t.T / K
    assert np.allclose(lhs, x.astype(np.float64) @ W.astype(np.float64), rtol=1e-12, atol=1e-15)


def test_zero_row_and_zero_group_guards():
    K, G = 128, 32
    x = np.zeros((3, K), dtype=np.float16)
    x[1, 5] = 2.0
    perm = np.arange(K, dtype=np.int32)
    fe = oracle.frontend(x, perm, G, rotate=False)
    # groups 1..3 are all zero over all tokens -> scale 1 (R9)
    assert np.array_equal(fe["S"], [2.0, 1.0, 1.0, 1.0])
    assert fe["r"][0] == 0 and fe["dx"][0] == 0 and not fe["q"][0].any()
    assert fe["q"][1, 5] == 7


def test_ablation_switches():
    x, perm, G = _case()
    fe = oracle.frontend(x, perm, G, rotate=False)
    assert np.array_equal(fe["Z"], x.astype(np.float64))
    fe = oracle.frontend(x, perm, G, smooth=False)
    assert np.all(fe["S"] == 1.0)


def test_calibrate_perm_order_brute_force():
    g = np.random.default_rng(4)
    K = 32
    xc = g.integers(-3, 4, size=(6, K)).astype(np.float16)   # many ties
    perm = oracle.calibrate_perm(xc)
    c = np.abs(xc.astype(np.float64) @ pins.hadamard_popcount(K)).max(axis=0)
    ref = sorted(range(K), key=lambda k: (-c[k], k))
    assert list(perm) == ref


def test_weights_per_channel_properties():
    g = np.random.default_rng(6)
    K, N = 256, 9
    W = (g.standard_normal((K, N)) * 0.02).astype(np.float16)
    W[:, 3] = 0
    perm = g.permutation(K).astype(np.int32)
    wp = oracle.prepare_weights(W, perm)
    qw = wp["qw"]
    assert not qw[3].any() and wp["dw"][3] == 0
    nz = [n for n in range(N) if n != 3]
    assert np.all(np.abs(qw[nz]).max(axis=1) == 7)
    assert np.all(np.abs(qw) <= 7)


# ------------------------------------------------------------------- GEMM
def test_partials_vs_int64_brute_force():
    g = np.random.default_rng(7)
    for (M, N, K, G) in [(5, 7, 64, 32), (3, 4, 256, 128), (2, 3, 128, 128)]:
        q = g.integers(-7, 8, size=(M, K)).astype(np.int8)
        qw = g.integers(-7, 8, size=(N, K)).astype(np.int8)
        q[0] = 7
        qw[0] = -7     # extreme partials
        P = oracle.group_partials(q, qw, G)
        assert np.array_equal(P, oracle.group_partials_int64(q, qw, G))
        assert np.abs(P).max() <= 49 * G
        assert P[0, 0, 0] == -49 * G


def test_output_magnitude_bounds_output():
    g = np.random.default_rng(8)
    q = g.integers(-7, 8, size=(4, 128)).astype(np.int8)
    qw = g.integers(-7, 8, size=(5, 128)).astype(np.int8)
    out = oracle.linear_out(q, g.random(4), g.random(2) + 0.5, qw, g.random(5), 64)
    assert np.all(np.abs(out["Y"]) <= out["C"] * (1 + 1e-12))


def test_quantisation_error_is_bounded_and_rrs_beats_rs_on_spikes():
    """Non-gating context check of the pages' qualitative claim: on spiky
    synthetic activations, rotation + runtime smooth at G=128 has lower output
    error than runtime smooth without rotation ([RRS-summary] "Surprising
    findings"; reported, asserted only as an ordering)."""
    wl = workloads.WORKLOADS["tiny"]
    x = workloads.runtime_x(wl)
    w = workloads.weights(wl)
    perm = oracle.calibrate_perm(workloads.calib_x(wl))
    ref = x.astype(np.float64) @ w.astype(np.float64)
    res = oracle.rrs_linear(x, w, perm, 128)
    err_rrs = np.linalg.norm(res["Y"] - ref) / np.linalg.norm(ref)
    # RS without rotation: identity "rotation" on both sides.
    fe = oracle.frontend(x, perm, 128, rotate=False)
    Wp = w.astype(np.float64).T[:, perm]
    a = np.abs(Wp).max(axis=1)
    qw = oracle.rtn_codes(7 * Wp / a[:, None])
    y_rs = oracle.linear_out(fe["q"], fe["dx"], fe["S"], qw, a / 7, 128)["Y"] * x.shape[1]
    err_rs = np.linalg.norm(y_rs - ref) / np.linalg.norm(ref)
    assert err_rrs < 0.2
    assert err_rrs < err_rs


def test_rotation_spares_the_victims_of_a_spike():
    """Non-gating context check of the pages' qualitative claim about spike
    outliers and the victim effect ([RRS-summary] "Approach"; [RRS-rebuttal]
    "Novelty"): in a token with a spike, smoothing without rotation rounds
    most of the other channels to code 0, while the rotation spreads the
    spike over every channel first. Reported, asserted only as an ordering."""
    wl = workloads.WORKLOADS["tiny"]
    x = workloads.runtime_x(wl)
    perm = oracle.calibrate_perm(workloads.calib_x(wl))
    spiky = np.abs(x.astype(np.float64)).max(axis=1) >= 0.99 * wl.spike_value
    assert spiky.any()
    zeros_rrs = int((oracle.frontend(x, perm, 128)["q"][spiky] == 0).sum())
    zeros_rs = int((oracle.frontend(x, perm, 128, rotate=False)["q"][spiky] == 0).sum())
    print(f"zero codes in {int(spiky.sum())} spike tokens: {zeros_rrs} with rotation, {zeros_rs} without")
    assert zeros_rrs < zeros_rs


def test_scale_match_statistic():
    assert oracle.scale_match_u(np.ones(16)) == 1.0
    t = np.zeros(16)
    t[0] = 4.0
    assert oracle.scale_match_u(t) == 4.0


def test_pack_layout_feeds_fp8_subnormals():
    """The packing reading R10 is chosen so that, per 32-bit word, w & 0x87878787
    and rotr(w, 4) & 0x87878787 are the even and odd codes as sign-magnitude
    bytes (fp8 e4m3 subnormals +-|q| * 2^-9); checked on every code pair."""
    g = np.random.default_rng(12)
    q = g.integers(-7, 8, size=(64, 8)).astype(np.int8)
    b = oracle.pack_codes(q)
    w = b.view("<u4")[:, 0].astype(np.uint64)
    lo = w & 0x87878787
    hi = (((w >> 4) | (w << 28)) & 0xFFFFFFFF) & 0x87878787

    def dec(x, j):
        byte = (x >> (8 * j)) & 0xFF
        return np.where(byte & 0x80, -(byte & 7).astype(np.int64), (byte & 7).astype(np.int64))
    for j in range(4):
        assert np.array_equal(dec(lo, j), q[:, 2 * j])
        assert np.array_equal(dec(hi, j), q[:, 2 * j + 1])


# ---- signed rotation (x D H; [AGC-OR] Sec. 4.1 / Sec. 4.6, reading R18)
def test_signed_rotation_explicit_and_inverse():
    assert pins.signed_rotation_matches_explicit(oracle.rotate_rows)
    assert pins.signed_rotation_inverts(oracle.rotate_rows)


def test_signed_rotation_all_plus_is_plain():
    x, perm, G = _case()
    K = x.shape[1]
    assert np.array_equal(oracle.rotate_rows(x, np.ones(K)), oracle.fwht(x))
    a = oracle.frontend(x, perm, G)
    b = oracle.frontend(x, perm, G, d=np.ones(K))
    assert np.array_equal(a["q"], b["q"]) and np.array_equal(a["S"], b["S"])


def test_signed_unrounded_output_equals_xw():
    import functools
    d = np.where(np.random.default_rng(9).random(128) < 0.5, -1.0, 1.0)
    fe = functools.partial(oracle.frontend, d=d)
    pw = functools.partial(oracle.prepare_weights, d=d)
    assert pins.unrounded_output_is_xw(fe, pw, oracle.linear_out)


def test_signed_weights_are_h_d_w():
    g = np.random.default_rng(11)
    K, N = 64, 6
    W = (g.standard_normal((K, N)) * 0.05).astype(np.float16)
    d = np.where(g.random(K) < 0.5, -1.0, 1.0)
    perm = g.permutation(K).astype(np.int32)
    wp = oracle.prepare_weights(W, perm, d)
    ref = scipy.linalg.hadamard(K).astype(np.float64) @ (d[:, None] * W.astype(np.float64))
    assert np.array_equal(wp["Wp_t"], ref[perm, :].T)


def test_signs_from_bits_brute_force():
    g = np.random.default_rng(12)
    K = 96
    bits = g.integers(0, 2**32, size=K // 32, dtype=np.uint64).astype(np.uint32)
    d = oracle.signs_from_bits(bits, K)
    for j in range(K):
        word = int(bits[j // 32])
        assert d[j] == (-1.0 if (word >> (j % 32)) & 1 else 1.0)


# ---- Kronecker rotation for K = m 2^k (reading R19)
def test_paley_orders_are_hadamard():
    assert pins.paley_is_hadamard(oracle.hadamard_paley)


def test_kron_rotation_explicit():
    assert pins.kron_rotation_matches_explicit(oracle.hadamard_rows, oracle.hadamard_paley)


def test_kron_split():
    assert oracle.kron_split(4096) == (1, 4096)
    assert oracle.kron_split(14336) == (28, 512)
    assert oracle.kron_split(768) == (12, 64)
    assert oracle.kron_split(5120) == (20, 256)
    for bad in (100, 11008, 14 * 3):
        with pytest.raises(ValueError):
            oracle.kron_split(bad)


@pytest.mark.parametrize("K,G", [(768, 64), (1792, 128)])
def test_kron_unrounded_output_equals_xw(K, G):
    assert pins.unrounded_output_is_xw(oracle.frontend, oracle.prepare_weights, oracle.linear_out, K=K, G=G)


def test_kron_signed_rotation_explicit():
    g = np.random.default_rng(14)
    m, n = 20, 64
    x = g.standard_normal((3, m * n)).astype(np.float16)
    d = np.where(g.random(m * n) < 0.5, -1.0, 1.0)
    ref = (x.astype(np.float64) * d) @ np.kron(oracle.hadamard_paley(m), scipy.linalg.hadamard(n).astype(np.float64))
    assert np.array_equal(oracle.rotate_rows(x, d), ref)


# ------------------------------------------------------ exemption window
def test_near_half_window():
    assert pins.near_half_window(oracle.near_half)
    assert pins.near_half_window(oracle.near_half, w=1e-3)


# ------------------------------------- ablations: RS alone, rotation alone
def test_unrotated_unrounded_output_equals_xw():
    for G in (1, 32, 96):
        assert pins.unrounded_output_is_xw_unrotated(oracle.frontend, oracle.prepare_weights,
                                                     oracle.linear_out, G=G)


def test_unrotated_weights_are_reordered_raw_columns():
    """Without the rotation the weight side is W's rows in perm order,
    quantised per output channel: a hand check on a tiny matrix."""
    W = np.array([[0.5, -1.0], [2.0, 0.25], [-1.0, 0.0], [0.0, 0.5]], dtype=np.float16)
    perm = np.array([2, 0, 3, 1], dtype=np.int32)
    wp = oracle.prepare_weights(W, perm, rotate=False)
    # column 0 reordered: [-1, 0.5, 0, 2], max 2 -> 7 x / 2 = [-3.5, 1.75, 0, 7]
    # -> rne: [-4, 2, 0, 7]; column 1: [0, -1, 0.5, 0.25], max 1 -> [0, -7, 3.5, 1.75] -> [0, -7, 4, 2]
    assert np.array_equal(wp["qw"], [[-4, 2, 0, 7], [0, -7, 4, 2]])
    assert np.array_equal(wp["a"], [2.0, 1.0])


def test_calibrate_perm_unrotated_brute_force():
    g = np.random.default_rng(9)
    K = 24
    xc = g.integers(-4, 5, size=(5, K)).astype(np.float16)
    perm = oracle.calibrate_perm(xc, rotate=False)
    c = np.abs(xc.astype(np.float64)).max(axis=0)
    assert list(perm) == sorted(range(K), key=lambda k: (-c[k], k))
    with pytest.raises(ValueError):
        oracle.calibrate_perm(xc, d=np.ones(K), rotate=False)


def test_G1_is_per_channel_runtime_smooth():
    """G = 1: every reordered channel has its own scale, its |max| over the
    call's tokens (per-channel Runtime Smooth); without the rotation the
    smoothed activations are the raw channels divided by that max."""
    x, perm, _ = _case(seed=11, M=30, K=256, G=64)
    x[:, 7] = 0                                   # one all-zero channel -> scale 1
    fe = oracle.frontend(x, perm, 1, rotate=False)
    xp = x.astype(np.float64)[:, perm]
    c = np.abs(xp).max(axis=0)
    assert np.array_equal(fe["S"], np.where(c > 0, c, 1.0))
    assert np.array_equal(fe["U"], xp / np.where(c > 0, c, 1.0)[None, :])
    nz = c > 0
    assert np.all(np.abs(fe["U"][:, nz]).max(axis=0) == 1.0)
    fe_r = oracle.frontend(x, perm, 1)
    assert np.all(np.abs(fe_r["U"]).max(axis=0)[np.abs(fe_r["Zp"]).max(axis=0) > 0] == 1.0)


def test_rs_without_rotation_degrades_with_group_size():
    """Non-gating context check of the pages' qualitative claim that Runtime
    Smooth without the rotation loses accuracy as the group grows while the
    rotated form barely moves ([RRS-summary] "Surprising findings" and
    "Limitations"): ordering only, on the tiny workload."""
    wl = workloads.WORKLOADS["tiny"]
    x, w, xc = workloads.runtime_x(wl), workloads.weights(wl), workloads.calib_x(wl)
    ref = x.astype(np.float64) @ w.astype(np.float64)

    def err(G, rotate):
        perm = oracle.calibrate_perm(xc, rotate=rotate)
        y = oracle.rrs_linear(x, w, perm, G, rotate=rotate)["Y"]
        return np.linalg.norm(y - ref) / np.linalg.norm(ref)

    rs = [err(G, False) for G in (1, 32, 128)]
    rrs = [err(G, True) for G in (1, 32, 128)]
    assert rs[0] < rs[1] < rs[2]
    assert rrs[2] < rs[2]
    assert max(rrs) - min(rrs) < rs[2] - rs[0]


def test_rotation_only_is_per_token_rtn_of_rotated_rows():
    """smooth=False (S = 1) is the per-channel A4W4 baseline: the codes are
    per-token round-to-nearest of the rotated, reordered row."""
    x, perm, G = _case(seed=12)
    fe = oracle.frontend(x, perm, G, smooth=False)
    zp = pins.hadamard_popcount(x.shape[1])
    z = (x.astype(np.float64) @ zp)[:, perm]
    r = np.abs(z).max(axis=1)
    assert np.array_equal(fe["q"], np.clip(np.rint(7 * z / r[:, None]), -7, 7).astype(np.int8))
