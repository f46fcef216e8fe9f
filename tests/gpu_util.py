"""Helpers for the GPU parity tests: move seeded inputs to the device and back."""
import numpy as np
import torch

import synth


def device_tensor(a: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to("cuda")


def host_f64(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return synth.bf16_bits_to_f64(t.view(torch.int16).numpy().view(np.uint16))
    return t.numpy().astype(np.float64)


def as_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    return synth.bf16_bits_to_f64(a) if dtype == "bf16" else a.astype(np.float64)


TOL = {"bf16": {"o": 2e-2, "lse": 1e-3, "grad": 2e-2}, "f32": {"o": 1e-4, "lse": 1e-4, "grad": 1e-4}}


def _bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |x| (8 significant bits)."""
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return 2.0 ** (e - 7)


def bwd_rounding_bound(q, k, v, do, o, lse, scale: float, causal: bool, tol: float = 2e-2):
    """Element-wise bound on |bf16 backward - exact gradient|, derived from the arithmetic the
    bf16 backward does, for one (b, h) (arrays (T, D), float64, o and lse the exact forward).

    The backward ("Lab 06 - Attention kernels", section 4) rounds three quantities to bf16:
      * the forward's output O, which feeds D_i = sum_d dO_id O_id: O carries the bf16 rounding
        of the P~ that multiplied V (relative 2^-9 each) and its own output rounding, so
        |dD_i| <= 2^-8 sum_d |dO_id| (sum_j P_ij |V_jd| + |O_id|);
      * dS = P (dP - D) before the dQ and dK products: relative 2^-9 per entry;
      * P before the dV product: relative 2^-9 per entry.
    A change dD_i moves dS_ij by P_ij dD_i. With u = 2^-8 (twice the half-ulp):
      |d dQ_id| <= scale (u sum_j |dS_ij K_jd| + |dD_i| sum_j P_ij |K_jd|)
      |d dK_jd| <= scale (u sum_i |dS_ij Q_id| + sum_i P_ij |dD_i| |Q_id|)
      |d dV_jd| <= u sum_i P_ij |dO_id|
    plus the flat tolerance `tol` and half a bf16 ulp of the result for the output rounding.
    The fp32 recomputation of S, P and dP adds relative errors near 2^-24, far below these.
    Returns (bound_dq, bound_dk, bound_dv).
    """
    import oracle
    u = 2.0 ** -8
    s = oracle.scores(q, k, scale, causal)
    p = np.exp(s - lse[:, None])
    dp = do @ v.T
    dvec = np.sum(do * o, axis=1)
    ds = p * (dp - dvec[:, None])
    dd = u * np.sum(np.abs(do) * (p @ np.abs(v) + np.abs(o)), axis=1)
    aq, ak = np.abs(q), np.abs(k)
    bq = scale * (u * (np.abs(ds) @ ak) + dd[:, None] * (p @ ak))
    bk = scale * (u * (np.abs(ds).T @ aq) + (p * dd[:, None]).T @ aq)
    bv = u * (p.T @ np.abs(do))
    dq = scale * ds @ k
    dk = scale * ds.T @ q
    dv = p.T @ do
    return tuple(b + tol + 0.5 * _bf16_ulp(g) for b, g in ((bq, dq), (bk, dk), (bv, dv)))


# The scaled E4M3 matrix-core product sums a 64-element block of products to within about
# 2^-11.3 of the largest product in the block (measured; tests/test_fp8_gpu.py pins
# E4M3_SUM_REL = 2^-10 as the bound used here).
E4M3_SUM_REL = 2.0 ** -10


def e4m3_score_error_bound(qd: np.ndarray, kd: np.ndarray, scale: float, chunk: int = 64):
    """Bound on |S_fp8 - S| for one head, S = scale * qd kd^T on the dequantized values
    (qd (Tq, D), kd (Tk, D)): E4M3_SUM_REL * scale * sum over 64-element blocks of the largest
    |q_d k_d| in the block."""
    Tq, D = qd.shape
    nb = D // 64
    out = np.empty((Tq, kd.shape[0]))
    aq, ak = np.abs(qd), np.abs(kd)
    for r0 in range(0, Tq, chunk):
        blk = aq[r0:r0 + chunk, None, :] * ak[None, :, :]          # (rows, Tk, D)
        out[r0:r0 + chunk] = blk.reshape(blk.shape[0], blk.shape[1], nb, 64).max(-1).sum(-1)
    return E4M3_SUM_REL * scale * out


def e4m3_tolerances(qd, kd, v, scale, causal, shift=0):
    """Per-row (O, LSE) tolerances of the E4M3 forward against the oracle on the dequantized
    inputs, for one head: delta_i = the largest score error bound over row i's visible keys
    (bottom-right causal with shift = Tk - Tq); every softmax weight then moves by a factor
    within e^(+-2 delta_i), so |dO_i| <= (e^(2 delta_i) - 1) max_j |V_j| and
    |dLSE_i| <= delta_i, on top of the bf16 tolerances."""
    b = e4m3_score_error_bound(qd, kd, scale)
    Tq, Tk = b.shape
    vis = np.ones((Tq, Tk), dtype=bool)
    if causal:
        vis = np.arange(Tk)[None, :] <= np.arange(Tq)[:, None] + shift
    delta = np.where(vis, b, 0.0).max(axis=1)
    vabs = np.abs(v).max(axis=1)
    vmax = np.where(vis, vabs[None, :], 0.0).max(axis=1)
    return TOL["bf16"]["o"] + np.expm1(2 * delta) * vmax, TOL["bf16"]["lse"] + delta
