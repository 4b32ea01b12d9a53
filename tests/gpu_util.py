"""Helpers for the GPU parity tests: device marshalling, calls through the
C ABI, and the comparison rules.

Comparison rules (codes are integers decided by floating point):
* a code whose oracle pre-rounding value lies within 1e-5 of a .5 boundary
  is exempt: either neighbour is correct, but a differing code must differ by
  exactly 1; every other code must match bit for bit;
* scales (dx, S, dw) match the exact oracle to a relative 1e-5 (the GPU
  rotation runs in fp32, the oracle's is exact);
* Y matches to 1e-3 relative to the cancellation-free magnitude
  C = (1/K) |dx| |dw| sum_g S_g |P_g| of the oracle.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import rotated_runtime_activation_amd as rra

DEV = torch.device("cuda:0")
WINDOW = 1e-5
Y_TOL = 1e-3
SCALE_TOL = 1e-5


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
    and scales [N] (the layout include/rrs.h documents)."""
    N, Kh = qw_packed.shape
    buf = torch.zeros(rra.rrs_weight_bytes(2 * Kh, N), dtype=torch.uint8, device=DEV)
    codes, dwv = rra.weight_views(buf, 2 * Kh, N)
    codes.copy_(to_dev(qw_packed))
    dwv.copy_(to_dev(dw.astype(np.float32)))
    return buf


def frontend(x: np.ndarray, perm: np.ndarray, G: int, flags: int = 0):
    M, K = x.shape
    X = to_dev(x)
    xq = torch.empty(M, K // 2, dtype=torch.uint8, device=DEV)
    dx = torch.empty(M, dtype=torch.float32, device=DEV)
    S = torch.empty(K // G, dtype=torch.float32, device=DEV)
    ws = torch.zeros(rra.rrs_sync_bytes(K, G), dtype=torch.uint8, device=DEV)
    rra.rrs_frontend(X, G, to_dev(perm), xq, dx, S, ws, flags)
    torch.cuda.synchronize()
    check_sync_block(ws, K, G)
    return xq.cpu().numpy(), dx.cpu().numpy(), S.cpu().numpy()


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


def flip_bound(q_gpu, q_ref, qw_gpu, qw_ref, dx, S, dw, G):
    """Largest legitimate |dY| per output from exempt code flips: a flipped
    activation code q[t, j] moves Y[t, n] by (1/K) dx_t dw_n S_g |qw[n, j]|,
    a flipped weight code by (1/K) dx_t dw_n S_g |q[t, j]| (both flipped: the
    sum of the two plus one step)."""
    K = q_ref.shape[1]
    Sj = np.repeat(np.asarray(S, dtype=np.float64), G)[None, :]
    Fa = (q_gpu.astype(np.int16) != q_ref.astype(np.int16)).astype(np.float64)
    Fw = (qw_gpu.astype(np.int16) != qw_ref.astype(np.int16)).astype(np.float64)
    t = (Fa * Sj) @ (np.abs(qw_ref.astype(np.float64)) + Fw).T
    t += (np.abs(q_ref.astype(np.float64)) * Sj) @ Fw.T
    return t * (np.asarray(dx, dtype=np.float64)[:, None] * np.asarray(dw, dtype=np.float64)[None, :]) / K
