"""CPU oracle for the Rotated Runtime Smooth (RRS) A4W4 linear layer.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the HIP
path (``rotated_runtime_activation_amd``) and imports nothing from it.

Plain, slow, obviously correct: NumPy in float64, steps in the order the pages
give them, no blocking or fusion. Sources ("pages"):

* [RRS-summary]  atlas.scime.ai summary of "Rotated Runtime Smooth:
  Training-Free Activation Smoother for accurate INT4 inference",
  paragraphs "Approach" and "Problem".
* [RRS-rebuttal] paperhub.cn page of the same paper (authors' rebuttal):
  "Novelty" answer (reorder + group-wise scales aligned with the GEMM),
  "Description of the reorder process" answer (equation Y = X W^T as a sum of
  per-channel outer products, invariant under a consistent channel reorder).
* [RRS-groovesquid] groovesquid.com summary, medium-difficulty summary
  (RS smooths with runtime maxima; the rotation narrows spike outliers).
* [AGC-OR] paperpeel.com page of "Understanding LLM Quantization through
  Activation-Guided Compensation and Orthogonal Residuals": Sec. 3.1 (output
  preserving transform Z = XP, V = W P^-T; per-token quantiser Q_A), Sec. 3.2
  (normalised Hadamard), App. B.1 (Delta_t = ||Z_t||_inf / q_A,
  q_A = 2^(b-1) - 1), Sec. 5 "Quantization and calibration" (per-token
  symmetric activations, per-output-channel symmetric weights).

Readings taken where the pages are silent, each with a label (R1, R2, ...):
R1 group scale = max over the group's channels of the per-channel max over
tokens; R2 the max runs over all tokens of the call; R3/R4 Sylvester Hadamard
in natural order, unnormalised, with the exact 1/K folded into the output;
R5 rotate, then reorder, then smooth; R6 round half to even; R7 no clipping;
R8 codes in [-7, 7]; R9 zero group -> scale 1, zero row -> codes 0 and scale 0;
R10 4-bit sign-magnitude packing, 8 codes per 32-bit word (layout in
``pack_codes``); R11 weights RTN per output
channel; R12 the group scale multiplies each group's integer partial;
R18 the signed rotation variant is Z = X D H with D = diag(d), d in {+1, -1}^K
given by the caller, and the weights take H D W ([AGC-OR] Sec. 4.1, the
transform family P = Lambda^-1 D H^T with Lambda = I; Sec. 4.6 "Signed online
rotation": sign flips before the online Hadamard rotation);
R19 for K = m 2^k with m in {12, 20, 28} (no power of two) the rotation is
the Kronecker product H_K = H_m (x) H_{2^k}, H_m from Paley's constructions
(I for q = 11, 19; II for q = 13) and Sylvester H_{2^k}; x indexed i 2^k + j
(i < m). H_m need not be symmetric, so the weights take H_K^T W (which is
W^T H_K row by row: the same row transform as the activations).

Every function below is pinned by ``tests/test_oracle_*.py`` against something
other than itself (explicit Hadamard matrices, scipy's Hadamard, closed forms,
a hand-worked example in ``tests/golden/``, int64 brute force, invariants).
"""
from __future__ import annotations

from typing import Dict

import numpy as np

QMAX = 7  # q_A = 2^(4-1) - 1 for 4-bit symmetric codes ([AGC-OR] App. B.1)


# ----------------------------------------------------------------- rotation
def fwht(x: np.ndarray) -> np.ndarray:
    """Unnormalised Sylvester Walsh-Hadamard transform along the last axis,
    in float64: returns x @ H_n with H_n[i, j] = (-1)^popcount(i & j).

    The rotation of [RRS-summary] "Approach" / [RRS-groovesquid]; normalised
    form in [AGC-OR] Sec. 3.2 (the 1/sqrt(n) is applied by the callers as an
    exact 1/n on the output, reading R3).

    Exact for fp16 inputs: every fp16 value is an integer multiple of 2^-24
    below 2^16 in magnitude, so every +-1 partial sum of n <= 2^13 of them is a
    multiple of 2^-24 below 2^29 and fits float64's 53-bit significand; no
    butterfly rounds.
    """
    y = np.array(x, dtype=np.float64, copy=True)
    n = y.shape[-1]
    if n & (n - 1):
        raise ValueError("length must be a power of two")
    lead = y.shape[:-1]
    h = 1
    while h < n:
        y = y.reshape(lead + (n // (2 * h), 2, h))
        a = y[..., 0, :]
        b = y[..., 1, :]
        y = np.stack((a + b, a - b), axis=-2)
        h *= 2
    return y.reshape(lead + (n,))


KRON_ORDERS = (12, 20, 28)


def _legendre(a: int, q: int) -> int:
    a %= q
    if a == 0:
        return 0
    return 1 if pow(a, (q - 1) // 2, q) == 1 else -1


def hadamard_paley(m: int) -> np.ndarray:
    """A Hadamard matrix of order m in {12, 20, 28} (reading R19), from
    Paley's constructions with the quadratic character chi of GF(q), q prime:
    construction I for q = m - 1 = 11, 19 (q = 3 mod 4): with the Jacobsthal
    matrix Q[i, j] = chi(j - i), H = I + [[0, 1^T], [-1, Q]]; construction II
    for q = 13 (q = 1 mod 4), m = 2 (q + 1): with the symmetric conference
    matrix C = [[0, 1^T], [1, Q]], H = [[C + I, C - I], [C - I, -C - I]].
    Pinned by H H^T = m I in the tests."""
    if m in (12, 20):
        q = m - 1
        Q = np.array([[_legendre(j - i, q) for j in range(q)] for i in range(q)], dtype=np.float64)
        S = np.zeros((m, m))
        S[0, 1:] = 1.0
        S[1:, 0] = -1.0
        S[1:, 1:] = Q
        return np.eye(m) + S
    if m == 28:
        q = 13
        Q = np.array([[_legendre(j - i, q) for j in range(q)] for i in range(q)], dtype=np.float64)
        C = np.zeros((q + 1, q + 1))
        C[0, 1:] = 1.0
        C[1:, 0] = 1.0
        C[1:, 1:] = Q
        I = np.eye(q + 1)
        return np.block([[C + I, C - I], [C - I, -C - I]])
    raise ValueError("Hadamard orders built here: 12, 20, 28")


def kron_split(K: int):
    """(m, n) with K = m n, n a power of two and m = 1 (K a power of two) or
    m in KRON_ORDERS; ValueError otherwise."""
    if K > 0 and K & (K - 1) == 0:
        return 1, K
    for m in KRON_ORDERS:
        if K % m == 0:
            n = K // m
            if n & (n - 1) == 0:
                return m, n
    raise ValueError(f"K = {K} is neither a power of two nor m 2^k with m in {KRON_ORDERS}")


def hadamard_rows(x: np.ndarray) -> np.ndarray:
    """x @ H_K along the last axis: Sylvester H_K for a power of two (``fwht``),
    else H_m (x) H_n with K = m n (reading R19): H_n over each run of n
    consecutive channels, then H_m across the runs."""
    x = np.asarray(x, dtype=np.float64)
    K = x.shape[-1]
    m, n = kron_split(K)
    if m == 1:
        return fwht(x)
    lead = x.shape[:-1]
    y = fwht(x.reshape(lead + (m, n)))                 # sum_j x[i, j] H_n[j, b]
    y = np.einsum("...ib,ia->...ab", y, hadamard_paley(m))  # sum_i (.)[i, b] H_m[i, a]
    return y.reshape(lead + (K,))


def rotate_rows(x: np.ndarray, d=None) -> np.ndarray:
    """The online rotation of the activations: x H, or with a sign vector d
    (+1 / -1 per input channel) the signed rotation x D H of [AGC-OR]
    Sec. 4.1 / Sec. 4.6 (reading R18); H = H_K of ``hadamard_rows``.
    Flipping signs of fp16 values is exact."""
    x = np.asarray(x, dtype=np.float64)
    if d is None:
        return hadamard_rows(x)
    d = np.asarray(d, dtype=np.float64)
    if d.shape != (x.shape[-1],) or not np.all(np.abs(d) == 1.0):
        raise ValueError("d must be a +-1 vector over the channels")
    return hadamard_rows(x * d)


def signs_from_bits(bits: np.ndarray, K: int) -> np.ndarray:
    """+-1 vector from the boundary's sign bitmask (K bits, little-endian
    32-bit words; bit j set means d_j = -1)."""
    b = np.asarray(bits, dtype=np.uint32)
    j = np.arange(K)
    neg = (b[j // 32] >> (j % 32).astype(np.uint32)) & 1
    return np.where(neg == 1, -1.0, 1.0)


# ------------------------------------------------------------------ reorder
def calibrate_perm(x_cal: np.ndarray, d=None, rotate: bool = True) -> np.ndarray:
    """Fixed channel order from a calibration batch (reading R5/R15).

    Rotate the calibration activations (with the layer's sign vector, if
    any), take each channel's |max| over the calibration tokens, and order
    channels by that max, largest first, ties by lower channel index. perm[j]
    is the source channel of position j, so outlier channels gather into the
    leading groups and normal channels into the rest ([RRS-rebuttal]
    "Novelty": reorder to collect outliers and normal values).
    ``rotate=False`` orders the raw channels (Runtime Smooth without the
    rotation, the ablation of [RRS-rebuttal] "Incomplete ablation study").
    """
    if not rotate and d is not None:
        raise ValueError("the sign vector belongs to the rotation")
    z = rotate_rows(x_cal, d) if rotate else np.asarray(x_cal, dtype=np.float64)
    c = np.max(np.abs(z), axis=0)
    return np.argsort(-c, kind="stable").astype(np.int32)


def invert_perm(perm: np.ndarray) -> np.ndarray:
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.size, dtype=perm.dtype)
    return inv


# ---------------------------------------------------------------- quantizer
def rtn_codes(v: np.ndarray) -> np.ndarray:
    """Round half to even, clamp to [-7, 7] (R6, R8)."""
    return np.clip(np.rint(v), -QMAX, QMAX).astype(np.int8)


def prepare_weights(W: np.ndarray, perm: np.ndarray, d=None, rotate: bool = True) -> Dict[str, np.ndarray]:
    """Offline weight side for Y = X W with W [K, N].

    Output-preserving transform ([AGC-OR] Sec. 3.1): rotating the activations
    by H is undone by H^T applied to the weights, and H is symmetric, so the
    rotated weight is Wz = H W (each column transformed); with signs
    (Z = X D H) it is Wz = H D W, since D D = I (reading R18). The reorder applies
    the same permutation to the weight rows ([RRS-rebuttal], reorder answer).
    Each output channel is quantised symmetric per channel with
    Delta_w = max|col| / 7 ([AGC-OR] Sec. 5; R11).

    Returns qw int8 [N, K] (K in permuted order), a = max|Wp| per output
    channel (float64 [N]), dw = a / 7, and the pre-rounding values uw [N, K].
    ``rotate=False`` skips the transform (Wz = W; the weight side of Runtime
    Smooth without rotation).
    """
    W = np.asarray(W)
    if not rotate and d is not None:
        raise ValueError("the sign vector belongs to the rotation")
    # [N, K]: row n is (H D W)[:, n], or W[:, n] without the rotation
    Wz_t = rotate_rows(W.T, d) if rotate else W.T.astype(np.float64)
    Wp_t = Wz_t[:, perm]                # Wp[j, n] = Wz[perm[j], n]
    a = np.max(np.abs(Wp_t), axis=1)    # per output channel
    safe = np.where(a > 0, a, 1.0)
    uw = np.where(a[:, None] > 0, QMAX * Wp_t / safe[:, None], 0.0)
    qw = rtn_codes(uw)
    return {"qw": qw, "a": a, "dw": a / QMAX, "uw": uw, "Wp_t": Wp_t}


def frontend(X: np.ndarray, perm: np.ndarray, G: int, *, rotate: bool = True,
             smooth: bool = True, d=None) -> Dict[str, np.ndarray]:
    """Activation side: rotate, reorder, runtime group-wise smoothing,
    per-token symmetric INT4 ([RRS-summary] "Approach"; [RRS-rebuttal]
    "Novelty"; [AGC-OR] Sec. 3.1 and App. B.1).

    Steps, in the pages' order:
      Z  = X H                                   (rotation)
      Zp[:, j] = Z[:, perm[j]]                   (fixed reorder)
      c_j = max_t |Zp[t, j]|                     (runtime channel max, R1/R2)
      S_g = max_{j in group g} c_j, 0 -> 1       (group-wise scale, R9)
      U  = Zp / S_g(j)                           (smoothing divide)
      r_t = max_j |U[t, j]|; Delta_t = r_t / 7   (per-token scale)
      v  = 7 U / r_t;  q = clamp(rne(v), -7, 7)  (codes; zero row -> 0)

    ``rotate=False`` gives Runtime Smooth without rotation and
    ``smooth=False`` gives rotation only (S = 1): the ablations of
    [RRS-rebuttal] "Incomplete ablation study". ``d`` (a +-1 vector) makes
    the rotation the signed one, Z = X D H (reading R18).
    """
    X = np.asarray(X)
    M, K = X.shape
    if K % G:
        raise ValueError("G must divide K")
    if not rotate and d is not None:
        raise ValueError("the sign vector belongs to the rotation")
    Z = rotate_rows(X, d) if rotate else X.astype(np.float64)
    Zp = Z[:, perm]
    c = np.max(np.abs(Zp), axis=0) if M else np.zeros(K)
    if smooth:
        S = np.max(c.reshape(K // G, G), axis=1)
        S = np.where(S > 0, S, 1.0)
    else:
        S = np.ones(K // G)
    U = Zp / np.repeat(S, G)[None, :]
    r = np.max(np.abs(U), axis=1) if K else np.zeros(M)
    safe = np.where(r > 0, r, 1.0)
    v = np.where(r[:, None] > 0, QMAX * U / safe[:, None], 0.0)
    q = rtn_codes(v)
    return {"Z": Z, "Zp": Zp, "c": c, "S": S, "U": U, "r": r, "dx": r / QMAX,
            "v": v, "q": q}


# --------------------------------------------------------------------- GEMM
def group_partials(q: np.ndarray, qw: np.ndarray, G: int) -> np.ndarray:
    """Exact per-group integer partials P[t, n, g] = sum_{j in g} q[t,j] qw[n,j].

    Computed as float64 matmuls on integer-valued operands: every partial sum
    is an integer of magnitude <= 49 * G < 2^53, so the result is exact in any
    summation order. Pinned against an int64 brute force in the tests.
    """
    M, K = q.shape
    N = qw.shape[0]
    ng = K // G
    qa = q.astype(np.float64).reshape(M, ng, G)
    qb = qw.astype(np.float64).reshape(N, ng, G)
    P = np.empty((M, N, ng), dtype=np.int64)
    for g in range(ng):
        P[:, :, g] = np.rint(qa[:, g, :] @ qb[:, g, :].T).astype(np.int64)
    return P


def group_partials_int64(q: np.ndarray, qw: np.ndarray, G: int) -> np.ndarray:
    """Brute-force int64 version of ``group_partials`` (small inputs)."""
    M, K = q.shape
    N = qw.shape[0]
    P = np.zeros((M, N, K // G), dtype=np.int64)
    for t in range(M):
        for n in range(N):
            prod = q[t].astype(np.int64) * qw[n].astype(np.int64)
            P[t, n] = prod.reshape(K // G, G).sum(axis=1)
    return P


def linear_out(q: np.ndarray, dx: np.ndarray, S: np.ndarray, qw: np.ndarray,
               dw: np.ndarray, G: int, rotated: bool = True) -> Dict[str, np.ndarray]:
    """Output of the A4W4 GEMM with group rescale (reading R12):

      Y[t, n] = (1/K) * dx_t * dw_n * sum_g S_g * P[t, n, g]

    (1/K is the product of the two 1/sqrt(K) normalisations of H, R3; codes
    made without the rotation, ``rotated=False``, carry no such factor.)
    Also returns the cancellation-free magnitude
      C[t, n] = (1/K) * |dx_t| * |dw_n| * sum_g S_g * |P[t, n, g]|
    used by the output tolerance (R13). Accumulates over groups without
    materialising P for all groups at once.
    """
    M, K = q.shape
    N = qw.shape[0]
    ng = K // G
    qa = q.astype(np.float64).reshape(M, ng, G)
    qb = qw.astype(np.float64).reshape(N, ng, G)
    acc = np.zeros((M, N))
    mag = np.zeros((M, N))
    for g in range(ng):
        P = qa[:, g, :] @ qb[:, g, :].T   # exact integers
        acc += S[g] * P
        mag += S[g] * np.abs(P)
    scale = (dx[:, None] * dw[None, :]) / (K if rotated else 1)
    return {"Y": scale * acc, "C": np.abs(scale) * mag}


def rrs_linear(X: np.ndarray, W: np.ndarray, perm: np.ndarray, G: int, d=None, *,
               rotate: bool = True, smooth: bool = True) -> Dict[str, np.ndarray]:
    """The whole RRS A4W4 linear: weights prepared offline, then the runtime
    front end and the grouped integer GEMM (signed rotation when d is given).
    ``rotate`` and ``smooth`` switch the two components off for the
    ablations of [RRS-rebuttal] "Incomplete ablation study": Runtime Smooth
    alone (no rotation on either side) and the rotation alone (S = 1, the
    per-channel A4W4 baseline)."""
    wp = prepare_weights(W, perm, d, rotate=rotate)
    fe = frontend(X, perm, G, rotate=rotate, smooth=smooth, d=d)
    out = linear_out(fe["q"], fe["dx"], fe["S"], wp["qw"], wp["dw"], G, rotated=rotate)
    return {"fe": fe, "wp": wp, **out}


# ----------------------------------------------------------------- packing
def pack_codes(q: np.ndarray) -> np.ndarray:
    """4-bit sign-magnitude packing along the last axis (reading R10; the
    pages fix no layout). Codes come in words of 8 (4 bytes, little endian);
    with a_j = code 2j and b_j = code 2j+1 of a word, byte j holds
      bits 0-2: |a_j|,  bit 7: sign of a_j,
      bits 4-6: |b_j|,  and bit 3 of byte (j+1) mod 4 holds the sign of b_j.
    Zero is stored with a clear sign bit; the last axis must be a multiple
    of 8."""
    q = np.asarray(q).astype(np.int16)
    if q.shape[-1] % 8:
        raise ValueError("code rows must be a multiple of 8")
    w = q.reshape(q.shape[:-1] + (q.shape[-1] // 8, 4, 2))
    a, b = w[..., 0], w[..., 1]
    sa = (a < 0).astype(np.int16)
    sb = (b < 0).astype(np.int16)
    byte = np.abs(a) | (np.abs(b) << 4) | (sa << 7) | (np.roll(sb, 1, axis=-1) << 3)
    return byte.reshape(q.shape[:-1] + (q.shape[-1] // 2,)).astype(np.uint8)


def unpack_codes(bts: np.ndarray) -> np.ndarray:
    """Inverse of ``pack_codes`` (a stored sign on a zero magnitude reads as
    zero)."""
    bts = np.asarray(bts).astype(np.int16)
    w = bts.reshape(bts.shape[:-1] + (bts.shape[-1] // 4, 4))
    ma, mb = w & 7, (w >> 4) & 7
    sa = (w >> 7) & 1
    sb = np.roll((w >> 3) & 1, -1, axis=-1)
    a = np.where(sa == 1, -ma, ma)
    b = np.where(sb == 1, -mb, mb)
    out = np.stack((a, b), axis=-1).reshape(bts.shape[:-1] + (2 * bts.shape[-1],))
    return out.astype(np.int8)


# ---------------------------------------------------------- parity helpers
def near_half(v: np.ndarray, window: float = 1e-5) -> np.ndarray:
    """Codes whose pre-rounding value lies within ``window`` of a .5 boundary:
    either neighbouring integer is an acceptable code there. The distance is
    taken from |v| to the nearest k + 1/2 (k = floor |v|), so the rule is the
    same for both signs."""
    a = np.abs(v)
    return np.abs(a - (np.floor(a) + 0.5)) < window


def scale_match_u(t: np.ndarray) -> np.ndarray:
    """u = max|t| / RMS(t) along the last axis: equals 1 when a row is
    perfectly flat ([RRS-rebuttal] "Experimental support for claims (W4)")."""
    t = np.asarray(t, dtype=np.float64)
    rms = np.sqrt(np.mean(t * t, axis=-1))
    return np.max(np.abs(t), axis=-1) / np.where(rms > 0, rms, 1.0)
