"""Helpers for the GPU parity tests: device marshalling, calls through the
C ABI, and the comparison rules.

Comparison rules (codes are integers decided by floating point):
* a code whose oracle pre-rounding value lies within 1e-5 of a .5 boundary
  is exempt: either neighbour is correct, but a differing code must differ by
  exactly 1; every other code must match bit for bit;
* scales (dx, S, dw) match the exact oracle to a relative 1e-5 (the GPU
  rotation runs in fp32, the oracle's is exact);
* Y is compared relative to the cancellation-free magnitude
  C = (1/K) |dx| |dw| sum_g S_g |P_g| (reading R13) with a bound derived
  from the fp32 arithmetic of the kernels (``y_tol``), in two ways: every
  output against the oracle's GEMM fed the GPU's own codes and scales, and
  the outputs whose row and column carry no exempt code flip against the
  oracle's end-to-end result, widened by the GPU scales' observed relative
  deviation from the exact ones.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import rotated_runtime_activation_amd as rra

DEV = torch.device("cuda:0")
WINDOW = 1e-5
SCALE_TOL = 1e-5
U32 = 2.0 ** -24  # unit roundoff of fp32


def y_tol(K: int, G: int) -> float:
    """Relative bound (times C) on the fp32 rounding of the grouped GEMM's
    output, given exact codes and scales. Along one output's chain the
    kernels round at most: once per matrix instruction that adds into a
    non-integer accumulator (K/64 of them, K/32 at G = 32, where the
    instruction covers 32 codes), twice per group (the ratio S_{g-1}/S_g and
    the rescale by it), and a fixed handful in the epilogue (the two halves'
    or the waves' sums, dx 2^18/K, the products by dx and dw: at most 8).
    Each rounding errs by at most u times a partial magnitude bounded by C,
    so |dY| <= gamma_n C with gamma_n = n u / (1 - n u) (the standard bound
    of a chain of n roundings, u = 2^-24). A group's partial itself is exact
    (integers below 2^24 units), which the partials tests check bit for bit.
    At K = 4096, G = 128 this is 8.1e-6."""
    km = 32 if G == 32 else 64
    n = K // km + 2 * (K // G) + 8
    return n * U32 / (1 - n * U32)


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def prepare_weights(w: np.ndarray, perm: np.ndarray):
    K, N = w.shape
    wq = torch.empty(rra.rrs_weight_bytes(K, N), dtype=torch.uint8, device=DEV)
    rra.rrs_prepare_weights(to_dev(w), to_dev(perm), wq)
    return wq


def weight_buffer_from_codes(qw_packed: np.ndarray, dw: np.ndarray) -> torch.Tensor:
    """Opaque prepared-weight buffer holding the given packed codes [N, K/2]
    (row-major; stored in the layout include/rrs.h documents) and scales
    [N]."""
    N, Kh = qw_packed.shape
    K = 2 * Kh
    buf = torch.zeros(rra.rrs_weight_bytes(K, N), dtype=torch.uint8, device=DEV)
    rra.codes_buffer(to_dev(qw_packed), K, out=rra.weight_codes_region(buf, K, N))
    _, dwv = rra.weight_views(buf, K, N)
    dwv.copy_(to_dev(dw.astype(np.float32)))
    return buf


def xq_buffer(q_packed: np.ndarray) -> torch.Tensor:
    """Activation-code buffer (stored layout) holding the row-major packed
    codes [M, K/2]."""
    return rra.codes_buffer(to_dev(q_packed), 2 * q_packed.shape[1])


def xq_empty(M: int, K: int) -> torch.Tensor:
    """An uninitialised activation-code buffer for M tokens of length K."""
    return torch.empty(rra.rrs_codes_bytes(M, K), dtype=torch.uint8, device=DEV)


def xq_codes(xq: torch.Tensor, M: int, K: int) -> np.ndarray:
    """The row-major packed codes [M, K/2] held in an activation-code buffer."""
    return rra.codes_matrix(xq, M, K).cpu().numpy()


def frontend(x: np.ndarray, perm: np.ndarray, G: int, flags: int = 0):
    M, K = x.shape
    X = to_dev(x)
    xq = xq_empty(M, K)
    dx = torch.empty(M, dtype=torch.float32, device=DEV)
    S = torch.empty(K // G, dtype=torch.float32, device=DEV)
    ws = torch.zeros(rra.rrs_sync_bytes(K, G), dtype=torch.uint8, device=DEV)
    rra.rrs_frontend(X, G, to_dev(perm), xq, dx, S, ws, flags)
    torch.cuda.synchronize()
    check_sync_block(ws, K, G)
    return xq_codes(xq, M, K), dx.cpu().numpy(), S.cpu().numpy()


def check_sync_block(ws, K: int, G: int, calls: int = 1):
    """After `calls` front-end calls on a freshly initialised workspace: the
    error word is clear, the reserved words stay zero (the multi-launch form
    keeps its maxima in the codes buffer), and the one-launch epoch counted
    the one-launch calls (0 or `calls`)."""
    words = ws[: rra.rrs_sync_bytes(K, G)].view(torch.int32).cpu().numpy()
    assert words[2] == 0, "a bounded wait gave up (error word set)"
    assert not words[0:2].any() and not words[4:17408].any(), "reserved synchronisation words written"
    assert words[3] in (0, calls), f"epoch {words[3]} after {calls} call(s)"


def compare_codes(q_gpu: np.ndarray, q_ref: np.ndarray, v_ref: np.ndarray, what: str) -> dict:
    diff = q_gpu.astype(np.int16) != q_ref.astype(np.int16)
    exempt = oracle.near_half(v_ref, WINDOW)
    bad = diff & ~exempt
    stats = {"codes": int(q_ref.size), "exempt": int(exempt.sum()),
             "exempt_differ": int((diff & exempt).sum()), "nonexempt_differ": int(bad.sum())}
    log(f"  {what}: {stats}")
    assert not bad.any(), f"{what}: {int(bad.sum())} non-exempt code mismatches, first at {np.argwhere(bad)[:5].tolist()}"
    if diff.any():
        step = np.abs(q_gpu.astype(np.int16) - q_ref.astype(np.int16))[diff]
        assert np.all(step == 1), f"{what}: exempt codes differ by more than one step"
    assert np.abs(q_gpu).max(initial=0) <= 7, f"{what}: code outside [-7, 7]"
    return stats


def rel_close(a: np.ndarray, ref: np.ndarray, tol: float, what: str) -> float:
    a = np.asarray(a, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    denom = np.where(ref != 0, np.abs(ref), 1.0)
    err = np.where(ref != 0, np.abs(a - ref) / denom, np.abs(a))
    e = float(err.max(initial=0.0))
    log(f"  {what}: max rel err {e:.3e}")
    assert e <= tol, f"{what}: max rel err {e:.3e} > {tol}"
    return e


def check_frontend(x, perm, G, flags=0, what="front end"):
    """GPU front end vs oracle: codes (exemption rule), dx and S."""
    fe = oracle.frontend(x, perm, G, rotate=not (flags & 1), smooth=not (flags & 2))
    xq, dx, S = frontend(x, perm, G, flags)
    q = oracle.unpack_codes(xq)
    stats = compare_codes(q, fe["q"], fe["v"], f"{what} codes")
    rel_close(dx, fe["dx"], SCALE_TOL, f"{what} dx")
    rel_close(S, fe["S"], SCALE_TOL, f"{what} S")
    return fe, xq, dx, S, q, stats


def y_error(Y: np.ndarray, ref: dict) -> float:
    C = ref["C"]
    err = np.abs(Y.astype(np.float64) - ref["Y"]) / np.where(C > 0, C, 1.0)
    err = np.where(C > 0, err, np.abs(Y))
    return float(err.max(initial=0.0))


def check_linear_two_way(Y, ref: dict, q_gpu, qw_gpu, dx_gpu, S_gpu, dw_gpu, G: int, what: str,
                         rotated: bool = True, fe=None, wp=None) -> dict:
    """End-to-end Y of rrs_linear against the oracle, the two ways of the
    parity rule: (1) every output against the oracle's GEMM fed the GPU's
    own codes and scales, within y_tol; (2) outputs whose row has no
    activation-code flip and whose column has no weight-code flip against the
    oracle's own end-to-end Y, within y_tol plus the relative deviation of
    the GPU's dx, dw and S from the exact ones. ``ref`` holds the oracle's Y
    and C for these rows and columns; ``fe`` / ``wp`` its front-end and
    weight results for them (default: ref["fe"], ref["wp"])."""
    fe = ref["fe"] if fe is None else fe
    wp = ref["wp"] if wp is None else wp
    K = q_gpu.shape[1]
    tol = y_tol(K, G)
    Yg = np.asarray(Y, dtype=np.float64)
    f64 = lambda a: np.asarray(a, dtype=np.float64)
    own = oracle.linear_out(q_gpu, f64(dx_gpu), f64(S_gpu), qw_gpu, f64(dw_gpu), G, rotated=rotated)
    e_own = np.abs(Yg - own["Y"])
    ok_own = e_own <= tol * own["C"]
    # relative deviation of the GPU's scales (reading R14 bounds each by 1e-5)
    rel = lambda g, r: np.where(f64(r) != 0, np.abs(f64(g) - f64(r)) / np.where(f64(r) != 0, np.abs(f64(r)), 1), 0)
    e_dx = rel(dx_gpu, fe["dx"])[:, None]
    e_dw = rel(dw_gpu, wp["dw"])[None, :]
    e_S = float(rel(S_gpu, fe["S"]).max(initial=0.0))
    scale_dev = (1 + e_dx) * (1 + e_dw) * (1 + e_S) - 1
    clean_rows = ~(q_gpu != fe["q"]).any(axis=1)
    clean_cols = ~(qw_gpu != wp["qw"]).any(axis=1)
    clean = clean_rows[:, None] & clean_cols[None, :]
    e_ref = np.abs(Yg - ref["Y"])
    ok_ref = e_ref <= ((tol + scale_dev) * (1 + 1e-6)) * ref["C"]
    C_own = np.where(own["C"] > 0, own["C"], 1.0)
    C_ref = np.where(ref["C"] > 0, ref["C"], 1.0)
    stats = {"outputs": int(Yg.size), "tol": tol,
             "own_max_err_over_C": float((e_own / C_own).max(initial=0.0)),
             "clean_outputs": int(clean.sum()), "flipped_rows": int((~clean_rows).sum()),
             "flipped_cols": int((~clean_cols).sum()),
             "ref_max_err_over_C_clean": float((e_ref / C_ref)[clean].max(initial=0.0))}
    log(f"  {what} Y: {stats}")
    assert ok_own.all(), f"{what}: {int((~ok_own).sum())} outputs off the oracle GEMM of the GPU's codes " \
                         f"(first {np.argwhere(~ok_own)[:3].tolist()})"
    assert ok_ref[clean].all(), f"{what}: {int((~ok_ref & clean).sum())} flip-free outputs off the oracle"
    return stats
