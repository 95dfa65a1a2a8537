"""Helpers shared by the GPU parity tests: upload, download, the tolerance gate."""

from __future__ import annotations

import sys

import numpy as np

from oracle import bf16_bits_to_f64

# Elementwise bar on bf16 outputs: |gpu - oracle| <= ATOL + RTOL * |oracle|.
ATOL = 1e-2
RTOL = 1e-2
# Tighter whole-tensor gate: bf16 weights (8-bit mantissa) and bf16 output
# rounding give a relative Frobenius error of a few 1e-3; 1e-2 flags a real bug.
REL_FRO_MAX = 1e-2


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(bits: np.ndarray, device="cuda"):
    import torch

    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(device)


def to_host_bits(t) -> np.ndarray:
    import torch

    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def to_host_f64(t) -> np.ndarray:
    return bf16_bits_to_f64(to_host_bits(t))


def upload(inputs: dict, device="cuda") -> dict:
    return {k: to_device(v, device) for k, v in inputs.items()}


def assert_parity(gpu: np.ndarray, ref: np.ndarray, what: str = ""):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite GPU output"
    err = np.abs(gpu - ref)
    bound = ATOL + RTOL * np.abs(ref)
    worst = np.unravel_index(np.argmax(err - bound), err.shape) if err.size else None
    ok = bool(np.all(err <= bound))
    denom = np.linalg.norm(ref)
    rel_fro = float(np.linalg.norm(gpu - ref) / denom) if denom > 0 else float(np.linalg.norm(gpu - ref))
    log(f"  parity {what}: max|err|={err.max() if err.size else 0:.3e} rel_fro={rel_fro:.3e} n={err.size}")
    assert ok, (f"{what}: elementwise bound violated at {worst}: gpu={gpu[worst]} "
                f"oracle={ref[worst]} err={err[worst]:.3e}")
    assert rel_fro <= REL_FRO_MAX, f"{what}: relative Frobenius error {rel_fro:.3e} > {REL_FRO_MAX}"


def spread_pairs(B: int, H: int, n: int, seed: int = 0) -> list:
    """Up to n (b, h) pairs: both ends, one in each eighth of the b*H + h range
    and one of each residue of b*H + h mod 8 (the two ways the decode kernels
    deal (b, h) pairs to the XCDs), then random ones."""
    import numpy as np

    rng = np.random.default_rng(seed)
    BH = B * H
    eighth = max(BH // 8, 1)
    flat = [0, BH - 1]
    for r in range(8):
        flat.append(min(BH - 1, r * BH // 8 + int(rng.integers(eighth))))
        flat.append(min(BH - 1, 8 * int(rng.integers(eighth)) + r))
    while len(set(flat)) < min(n, BH):
        flat.append(int(rng.integers(BH)))
    return [divmod(f, H) for f in list(dict.fromkeys(flat))[:n]]


def spread_heads(H: int) -> list:
    """Four heads spread over [0, H): first, last and two between."""
    return sorted({0, H // 3, 2 * H // 3, H - 1})
