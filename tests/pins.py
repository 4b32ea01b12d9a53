"""Pin checks for the oracle, written so that each takes the oracle function
under test as an argument. ``test_oracle_*.py`` call them on the real oracle
(they must pass) and on planted mistakes (they must fail), which shows that a
plausible slip -- a flipped sign, an inverted permutation, a dropped scale, a
different rounding rule -- cannot pass unnoticed.

Every reference value here comes from something other than the oracle: the
popcount definition of the Sylvester Hadamard matrix, scipy's Hadamard
routine, a hand-worked example (tests/golden/), closed forms and invariants.
"""
from __future__ import annotations

import json
import os

import numpy as np
import scipy.linalg

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def hadamard_popcount(n: int) -> np.ndarray:
    """H[i, j] = (-1)^popcount(i & j), built entry by entry from the bit
    definition (not by the butterfly recursion)."""
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    a = i & j
    pc = np.zeros_like(a)
    while np.any(a):
        pc += a & 1
        a >>= 1
    return np.where(pc % 2 == 0, 1.0, -1.0)


def hadamard_column(n: int, j: int) -> np.ndarray:
    i = np.arange(n)
    pc = np.array([bin(int(v)).count("1") for v in (i & j)])
    return np.where(pc % 2 == 0, 1.0, -1.0)


def load_golden(name: str = "rrs_k8_worked.json") -> dict:
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------- FWHT pins
def fwht_matches_explicit(fwht, sizes=(2, 4, 8, 16, 32, 64, 128, 256), seed=0) -> bool:
    """fwht(x) == x @ H bit-exactly for fp16 inputs (both are exact)."""
    g = np.random.default_rng(seed)
    for n in sizes:
        H = hadamard_popcount(n)
        x = (g.standard_normal((5, n)) * 3).astype(np.float16).astype(np.float64)
        if not np.array_equal(fwht(x), x @ H):
            return False
    return True


def fwht_unit_vectors(fwht, n=64) -> bool:
    """e_i -> row i of H; all-ones -> n e_0."""
    H = hadamard_popcount(n)
    if not np.array_equal(fwht(np.eye(n)), H):
        return False
    e0 = np.zeros(n)
    e0[0] = n
    return np.array_equal(fwht(np.ones(n)), e0)


# ----------------------------------------------------------- golden pins
def frontend_matches_golden(frontend) -> bool:
    gd = load_golden()
    e = gd["expect"]
    X = np.array(gd["X"], dtype=np.float16)
    perm = np.array(gd["perm"], dtype=np.int32)
    fe = frontend(X, perm, gd["G"])
    return (np.array_equal(fe["Z"], np.array(e["Z"]))
            and np.array_equal(fe["Zp"], np.array(e["Zp"]))
            and np.array_equal(fe["S"], np.array(e["S"], dtype=float))
            and np.array_equal(fe["r"], np.array(e["r"]))
            and np.allclose(fe["dx"], np.array(e["dx"]), rtol=1e-15, atol=0)
            and np.allclose(fe["v"], np.array(e["v"]), rtol=1e-15, atol=0)
            and np.array_equal(fe["q"], np.array(e["q"])))


def weights_match_golden(prepare_weights) -> bool:
    gd = load_golden()
    e = gd["expect"]
    W = np.array(gd["W"], dtype=np.float16)
    perm = np.array(gd["perm"], dtype=np.int32)
    wp = prepare_weights(W, perm)
    return (np.array_equal(wp["qw"], np.array(e["qw"]))
            and np.array_equal(wp["a"], np.array(e["a"]))
            and np.allclose(wp["dw"], np.array(e["dw"]), rtol=1e-15, atol=0))


def gemm_matches_golden(group_partials, linear_out) -> bool:
    gd = load_golden()
    e = gd["expect"]
    G = gd["G"]
    q = np.array(e["q"], dtype=np.int8)
    qw = np.array(e["qw"], dtype=np.int8)
    P = group_partials(q, qw, G)
    out = linear_out(q, np.array(e["dx"]), np.array(e["S"], dtype=float), qw,
                     np.array(e["dw"]), G)
    return (np.array_equal(P, np.array(e["P"]))
            and np.allclose(out["Y"], np.array(e["Y"]), rtol=1e-14, atol=1e-14))


def pack_matches_golden(pack_codes) -> bool:
    gd = load_golden()
    e = gd["expect"]
    return (np.array_equal(pack_codes(np.array(e["q"])), np.array(e["xq_bytes"], dtype=np.uint8))
            and np.array_equal(pack_codes(np.array(e["qw"])), np.array(e["wq_bytes"], dtype=np.uint8)))


# ------------------------------------------------- closed-form identities
def unrounded_output_is_xw(frontend, prepare_weights, linear_out, seed=1,
                           M=12, K=128, N=20, G=32) -> bool:
    """Without rounding (feed the pre-rounding values v and uw in place of the
    codes), the scale bookkeeping must give back X W exactly up to float64
    rounding: (1/K) (r/7) (a/7) sum_g S_g sum_j v uw = Zp Wp / K = X W
    ([RRS-rebuttal] reorder identity; [AGC-OR] Sec. 3.1 transform pair)."""
    g = np.random.default_rng(seed)
    X = (g.standard_normal((M, K)) * np.where(g.random(K) < 0.1, 20, 1)).astype(np.float16)
    W = (g.standard_normal((K, N)) * 0.02).astype(np.float16)
    perm = g.permutation(K).astype(np.int32)
    fe = frontend(X, perm, G)
    wp = prepare_weights(W, perm)
    out = linear_out(fe["v"], fe["dx"], fe["S"], wp["uw"], wp["dw"], G)
    ref = X.astype(np.float64) @ W.astype(np.float64)
    return bool(np.allclose(out["Y"], ref, rtol=1e-10, atol=1e-12 * np.abs(ref).max()))


def frontend_invariants(frontend, seed=5, M=40, K=512, G=64) -> bool:
    """I1: each group reaches |U| == 1 exactly; I2: |U| <= 1; I3: each nonzero
    row has a +-7 code at its |U| argmax; I4: |U - (r/7) q| <= r/14."""
    import workloads
    from oracle import calibrate_perm  # the permutation is an input here
    x, xc, _ = workloads.random_case(seed, M, K, 16)
    perm = calibrate_perm(xc)
    fe = frontend(x, perm, G)
    U, r, q = fe["U"], fe["r"], fe["q"]
    Ug = np.abs(U).reshape(M, K // G, G)
    am = np.argmax(np.abs(U), axis=1)
    return bool(np.all(Ug.max(axis=(0, 2)) == 1.0)
                and np.abs(U).max() <= 1.0
                and np.all(np.abs(q[np.arange(M), am]) == 7)
                and np.all(np.abs(U - (r[:, None] / 7) * q) <= r[:, None] / 14 * (1 + 1e-12)))


def signed_rotation_matches_explicit(rotate_rows, sizes=(2, 8, 64, 256), seed=3) -> bool:
    """Signed rotation x D H against the explicit product with scipy's
    Sylvester Hadamard and diag(d) ([AGC-OR] Sec. 4.1; reading R18). fp16
    inputs make both sides exact in float64."""
    g = np.random.default_rng(seed)
    for n in sizes:
        x = g.standard_normal((5, n)).astype(np.float16)
        d = np.where(g.random(n) < 0.5, -1.0, 1.0)
        ref = (x.astype(np.float64) * d) @ scipy.linalg.hadamard(n).astype(np.float64)
        if not np.array_equal(rotate_rows(x, d), ref):
            return False
    return True


def signed_rotation_inverts(rotate_rows, n=512, seed=4) -> bool:
    """(x D H) H / n then D gives x back exactly (H H = n I, D D = I)."""
    g = np.random.default_rng(seed)
    x = g.standard_normal((3, n)).astype(np.float16).astype(np.float64)
    d = np.where(g.random(n) < 0.5, -1.0, 1.0)
    z = rotate_rows(x, d)
    back = (z @ scipy.linalg.hadamard(n).astype(np.float64)) / n * d
    return bool(np.array_equal(back, x))


def paley_is_hadamard(hadamard_paley, orders=(12, 20, 28)) -> bool:
    """H H^T = m I with +-1 entries: the defining property of a Hadamard matrix
    (reading R19)."""
    for m in orders:
        H = hadamard_paley(m)
        if H.shape != (m, m) or not np.all(np.abs(H) == 1.0):
            return False
        if not np.array_equal(H @ H.T, m * np.eye(m)):
            return False
    return True


def kron_rotation_matches_explicit(hadamard_rows, hadamard_paley, cases=((12, 64), (20, 64), (28, 64), (12, 128)),
                                   seed=13) -> bool:
    """x H_K for K = m n against the explicit dense Kronecker product
    kron(H_m, H_n) with scipy's Sylvester H_n (fp16 inputs: exact)."""
    g = np.random.default_rng(seed)
    for m, n in cases:
        x = g.standard_normal((4, m * n)).astype(np.float16)
        ref = x.astype(np.float64) @ np.kron(hadamard_paley(m), scipy.linalg.hadamard(n).astype(np.float64))
        if not np.array_equal(hadamard_rows(x), ref):
            return False
    return True


# ------------------------------------------------- parity exemption window
def near_half_window(near_half, w=1e-5) -> bool:
    """The exemption rule of the code comparisons: a pre-rounding value is
    exempt exactly when |v| lies within w of k + 1/2 for an integer k (either
    neighbouring code is then correct). Values are chosen by hand: on both
    sides of several boundaries and for both signs, just inside the window
    (exempt), at twice the window and on integers (not exempt)."""
    inside = [2.5, 2.5 + w / 2, 2.5 - w / 2, -3.5 + w / 2, -3.5 - w / 2, 0.5 + 0.9 * w, 6.5 - 0.9 * w]
    outside = [3.0, 2.5 + 2 * w, 2.5 - 2 * w, -3.5 - 2 * w, 0.0, 1.0, -7.0, 7.0, 0.5 + 1.5 * w,
               3.0 - w / 2, -2.0 + w / 2]
    if w == 1e-5:  # literal values at the window the comparisons use
        inside += [2.499995, -3.500004]
        outside += [2.49, 2.5001]
    a = near_half(np.array(inside, dtype=np.float64), w)
    b = near_half(np.array(outside, dtype=np.float64), w)
    return bool(np.all(a) and not np.any(b))


def unrounded_output_is_xw_unrotated(frontend, prepare_weights, linear_out, seed=2,
                                     M=10, K=96, N=12, G=1) -> bool:
    """Runtime Smooth without the rotation (the ablation): with the
    pre-rounding values in place of the codes, dx dw sum_g S_g sum_j v uw =
    Zp Wp = X W exactly up to float64 rounding, with no 1/K (no Hadamard
    pair). The reorder identity of [RRS-rebuttal] on the raw channels."""
    g = np.random.default_rng(seed)
    X = (g.standard_normal((M, K)) * np.where(g.random(K) < 0.1, 20, 1)).astype(np.float16)
    W = (g.standard_normal((K, N)) * 0.02).astype(np.float16)
    perm = g.permutation(K).astype(np.int32)
    fe = frontend(X, perm, G, rotate=False)
    wp = prepare_weights(W, perm, rotate=False)
    out = linear_out(fe["v"], fe["dx"], fe["S"], wp["uw"], wp["dw"], G, rotated=False)
    ref = X.astype(np.float64) @ W.astype(np.float64)
    return bool(np.allclose(out["Y"], ref, rtol=1e-10, atol=1e-12 * np.abs(ref).max()))
