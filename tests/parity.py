"""Comparison rules between the HIP path and the oracle, and device upload.

INT8 (W8A8_INT8): int32 accumulators bit-exact; bf16 outputs within one bf16
ulp of the oracle's correctly rounded value (fp32 epilogue vs double).
FP8 (FP8_Dynamic, Block_FP8): normwise relative error <= 1e-2 against the
double-precision value, and elementwise |y_gpu - y| <= 2^-8 * S where
S = sum_k |a_k b_k| * |scales| is the oracle's bound matrix (S == 0 forces
y_gpu == +-0).  The 2^-8 budget covers bf16 output rounding (2^-9 relative)
plus fp32 accumulation in any order with room to spare.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

FMT_CODE = {"fp8": oracle.FMT_E4M3, "int8": oracle.FMT_INT8, "block_fp8": oracle.FMT_E4M3}
FP8_ELEM = 2.0 ** -8
FP8_NORM = 1e-2


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(bits).astype(np.uint16)
    return torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


def ordered(bits: np.ndarray) -> np.ndarray:
    """bf16 bits -> integers ordered like the values (+0 and -0 both 0)."""
    b = np.asarray(bits).astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def to_device(case, device="cuda"):
    """Upload a synth.Case: returns (a_q, a_scale, b_q, b_scale) device tensors."""
    dt = torch.int8 if case.fmt == "int8" else torch.float8_e4m3fn
    a = torch.from_numpy(np.ascontiguousarray(case.A)).to(device).view(dt)
    b = torch.from_numpy(np.ascontiguousarray(case.B)).to(device).view(dt)
    sa = torch.from_numpy(np.ascontiguousarray(case.sA)).to(device)
    sb = torch.from_numpy(np.ascontiguousarray(case.sB)).to(device)
    return a, sa, b, sb


def y_bits(y: torch.Tensor) -> np.ndarray:
    return y.view(torch.int16).cpu().numpy().view(np.uint16)


def oracle_full(case):
    return oracle.scaled_mm(FMT_CODE[case.fmt], case.A, case.sA, case.B, case.sB, block=case.block)


def check_y(fmt: str, y_gpu_bits: np.ndarray, ref_y_bits: np.ndarray, ref_ydbl: np.ndarray,
            ref_bound: np.ndarray, what: str = ""):
    """Assert the output rule of the format; returns a small stats dict."""
    y_gpu_bits = np.asarray(y_gpu_bits)
    assert y_gpu_bits.shape == ref_y_bits.shape, what
    if fmt == "int8":
        d = np.abs(ordered(y_gpu_bits) - ordered(ref_y_bits))
        bad = np.argwhere(d > 1)
        assert bad.size == 0, f"{what}: {len(bad)} outputs beyond 1 ulp, first at {bad[:3].tolist()}"
        return {"ulp_diffs": int((d == 1).sum())}
    yg = bf16_to_f64(y_gpu_bits)
    assert np.isfinite(yg).all(), f"{what}: non-finite outputs"
    err = np.abs(yg - ref_ydbl)
    lim = FP8_ELEM * ref_bound
    bad = np.argwhere(err > lim)
    assert bad.size == 0, (f"{what}: {len(bad)} outputs beyond 2^-8*S, first {bad[:3].tolist()} "
                           f"err={err[tuple(bad[0])]:.3g} lim={lim[tuple(bad[0])]:.3g}")
    nrm = np.linalg.norm(ref_ydbl)
    rel = float(np.linalg.norm(yg - ref_ydbl) / nrm) if nrm > 0 else 0.0
    assert rel <= FP8_NORM, f"{what}: normwise relative error {rel:.3g}"
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(ref_bound > 0, err / ref_bound, 0.0)
    return {"normwise": rel, "max_err_over_S": float(ratio.max()) if ratio.size else 0.0}


def check_case(case, y_gpu: torch.Tensor, ref=None, what: str = ""):
    ref = ref if ref is not None else oracle_full(case)
    return check_y(case.fmt, y_bits(y_gpu), ref.y, ref.ydbl, ref.bound, what or case.tag)


def sample_points(M: int, N: int, n: int, seed: int = 0):
    """Seeded sample of output positions including the four corners."""
    g = np.random.default_rng(seed)
    ms = np.concatenate([[0, 0, M - 1, M - 1], g.integers(0, M, n)])
    ns = np.concatenate([[0, N - 1, 0, N - 1], g.integers(0, N, n)])
    return ms, ns


def check_sampled(case, y_gpu: torch.Tensor, npts: int = 2000, seed: int = 0, what: str = ""):
    ms, ns = sample_points(case.M, case.N, npts, seed)
    ref = oracle.scaled_mm_points(FMT_CODE[case.fmt], case.A, case.sA, case.B, case.sB, ms, ns,
                                  block=case.block)
    yb = y_bits(y_gpu)[ms, ns]
    return check_y(case.fmt, yb, ref.y, ref.ydbl, ref.bound, what or case.tag)
