"""Planted mistakes in the oracle (CPU only): each plausible slip must make at
least one pin fail, so the pins are shown to be sensitive to it."""
import numpy as np

import oracle
from oracle import rrs_ref
from tests import pins


def _fwht_wrong_sign(x):
    y = np.array(x, dtype=np.float64, copy=True)
    n = y.shape[-1]
    lead = y.shape[:-1]
    h = 1
    while h < n:
        y = y.reshape(lead + (n // (2 * h), 2, h))
        a, b = y[..., 0, :], y[..., 1, :]
        y = np.stack((a + b, b - a), axis=-2)        # slip: b - a
        h *= 2
    return y.reshape(lead + (n,))


def _fwht_bit_reversed(x):
    # a valid Hadamard-type transform, but outputs in bit-reversed order
    z = oracle.fwht(x)
    n = z.shape[-1]
    bits = n.bit_length() - 1
    idx = [int(format(i, f"0{bits}b")[::-1], 2) if bits else 0 for i in range(n)]
    return z[..., idx]


def test_fwht_mutants_fail():
    assert not pins.fwht_matches_explicit(_fwht_wrong_sign)
    assert not pins.fwht_unit_vectors(_fwht_wrong_sign)
    # bit-reversal keeps e_0 -> ones but fails the explicit matrix check
    assert not pins.fwht_matches_explicit(_fwht_bit_reversed)


def _with(monkeypatch, name, fn):
    monkeypatch.setattr(rrs_ref, name, fn)


def test_inverse_perm_mutant_fails():
    def frontend_inv(X, perm, G, **kw):
        return rrs_ref.frontend.__wrapped__(X, oracle.invert_perm(perm), G, **kw)
    rrs_ref.frontend.__wrapped__ = rrs_ref.frontend
    try:
        assert not pins.frontend_matches_golden(frontend_inv)
    finally:
        del rrs_ref.frontend.__wrapped__


def test_round_half_away_mutant_fails(monkeypatch):
    _with(monkeypatch, "rtn_codes",
          lambda v: np.clip(np.sign(v) * np.floor(np.abs(v) + 0.5), -7, 7).astype(np.int8))
    assert not pins.frontend_matches_golden(rrs_ref.frontend)


def test_mean_instead_of_max_group_scale_fails():
    def frontend_mean(X, perm, G, **kw):
        fe = oracle.frontend(X, perm, G, **kw)
        K = X.shape[1]
        S = fe["c"].reshape(K // G, G).mean(axis=1)
        U = fe["Zp"] / np.repeat(S, G)
        r = np.abs(U).max(axis=1)
        v = 7 * U / r[:, None]
        return {**fe, "S": S, "U": U, "r": r, "dx": r / 7, "v": v, "q": oracle.rtn_codes(v)}
    # the golden case has constant groups (mean == max); the invariants catch it
    assert pins.frontend_invariants(oracle.frontend)
    assert not pins.frontend_invariants(frontend_mean)


def test_dropped_output_scale_fails():
    def linear_out_no_invK(q, dx, S, qw, dw, G):
        out = oracle.linear_out(q, dx, S, qw, dw, G)
        return {"Y": out["Y"] * q.shape[1], "C": out["C"]}
    assert not pins.unrounded_output_is_xw(oracle.frontend, oracle.prepare_weights, linear_out_no_invK)
    assert not pins.gemm_matches_golden(oracle.group_partials, linear_out_no_invK)


def test_weight_scale_not_divided_by_7_fails():
    def prep_bad(W, perm):
        wp = oracle.prepare_weights(W, perm)
        return {**wp, "dw": wp["a"]}
    assert not pins.weights_match_golden(prep_bad)
    assert not pins.unrounded_output_is_xw(oracle.frontend, prep_bad, oracle.linear_out)


def test_weight_rows_not_reordered_fails():
    def prep_noperm(W, perm):
        return oracle.prepare_weights(W, np.arange(len(perm), dtype=np.int32))
    assert not pins.weights_match_golden(prep_noperm)
    assert not pins.unrounded_output_is_xw(oracle.frontend, prep_noperm, oracle.linear_out)


def test_transposed_partials_fail():
    def partials_t(q, qw, G):
        P = oracle.group_partials(q, qw, G)
        return P[:, :, ::-1]                    # groups in the wrong order
    assert not pins.gemm_matches_golden(partials_t, oracle.linear_out)


def test_swapped_nibbles_fail():
    def pack_swapped(q):
        q = np.asarray(q).astype(np.int16)
        return ((q[..., 1::2] & 0xF) | ((q[..., 0::2] & 0xF) << 4)).astype(np.uint8)
    assert not pins.pack_matches_golden(pack_swapped)


def test_odd_sign_in_own_byte_fails():
    def pack_no_roll(q):
        q = np.asarray(q).astype(np.int16)
        w = q.reshape(q.shape[:-1] + (q.shape[-1] // 8, 4, 2))
        a, b = w[..., 0], w[..., 1]
        byte = np.abs(a) | (np.abs(b) << 4) | ((a < 0) << 7) | ((b < 0) << 3)
        return byte.reshape(q.shape[:-1] + (q.shape[-1] // 2,)).astype(np.uint8)
    assert not pins.pack_matches_golden(pack_no_roll)


def test_signs_after_rotation_mutant_fails():
    # slip: x H D instead of x D H
    def rot_after(x, d=None):
        z = oracle.fwht(x)
        return z if d is None else z * np.asarray(d, dtype=np.float64)
    assert not pins.signed_rotation_matches_explicit(rot_after)


def test_signs_ignored_mutant_fails():
    assert not pins.signed_rotation_matches_explicit(lambda x, d=None: oracle.fwht(x))


def test_kron_order_mutant_fails():
    # slip: H_n (x) H_m instead of H_m (x) H_n
    def rows_swapped(x):
        x = np.asarray(x, dtype=np.float64)
        m, n = oracle.kron_split(x.shape[-1])
        y = np.einsum("...ij,ja->...ia", x.reshape(x.shape[:-1] + (n, m)), oracle.hadamard_paley(m))
        return oracle.fwht(np.swapaxes(y, -1, -2)).swapaxes(-1, -2).reshape(x.shape)
    assert not pins.kron_rotation_matches_explicit(rows_swapped, oracle.hadamard_paley)


def test_kron_transposed_factor_mutant_fails():
    # slip: H_m^T in place of H_m (Paley I matrices are not symmetric)
    assert not pins.kron_rotation_matches_explicit(oracle.hadamard_rows, lambda m: oracle.hadamard_paley(m).T)


def test_paley_wrong_character_mutant_fails():
    # slip: Jacobsthal matrix with chi(i - j) and no border sign change
    def bad(m):
        H = oracle.hadamard_paley(m)
        H[1:, 0] = 1.0
        return H
    assert not pins.paley_is_hadamard(bad, orders=(12,))


def test_near_half_mutants_fail():
    # distance to the nearest integer instead of the nearest half
    assert not pins.near_half_window(lambda v, w=1e-5: np.abs(np.abs(v) - np.rint(np.abs(v))) < w)
    # a boundary off by a half step (k instead of k + 1/2 past the floor)
    assert not pins.near_half_window(lambda v, w=1e-5: np.abs(np.abs(v) - np.floor(np.abs(v))) < w)
    # window ten times too wide
    assert not pins.near_half_window(lambda v, w=1e-5: oracle.near_half(v, 10 * w), 1e-5)


def test_unrotated_output_with_1_over_K_fails():
    def linear_out_always_k(q, dx, S, qw, dw, G, rotated=True):
        return oracle.linear_out(q, dx, S, qw, dw, G, rotated=True)
    assert not pins.unrounded_output_is_xw_unrotated(oracle.frontend, oracle.prepare_weights, linear_out_always_k)


def test_unrotated_weights_still_rotated_fails():
    def prep_always_rotated(W, perm, d=None, rotate=True):
        return oracle.prepare_weights(W, perm, d)
    assert not pins.unrounded_output_is_xw_unrotated(oracle.frontend, prep_always_rotated, oracle.linear_out,
                                                     K=128)
