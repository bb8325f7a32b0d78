"""Shared helpers for the GPU parity tests (device upload, tolerance checks)."""
from __future__ import annotations

import sys

import numpy as np

# Tolerances on bf16 outputs against the float64 oracle.
MAX_ABS = 2e-2
REL_L2 = 5e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


def dev_i32(x, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(device)


def host_bits(t) -> np.ndarray:
    import torch
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def compare(got_bits, ref, what="", max_abs=MAX_ABS, rel_l2=REL_L2):
    """Check a bf16 GPU result against a float64 reference; return the stats."""
    got = bf16_to_f64(got_bits)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = got - ref
    mx = float(np.max(np.abs(err))) if err.size else 0.0
    nref = float(np.linalg.norm(ref))
    rl2 = float(np.linalg.norm(err) / nref) if nref > 0 else float(np.linalg.norm(err))
    worst = 0.0
    if got.ndim == 3:
        for h in range(got.shape[1]):
            nr = np.linalg.norm(ref[:, h])
            if nr > 0:
                worst = max(worst, float(np.linalg.norm(err[:, h]) / nr))
    say(f"[parity] {what}: max_abs={mx:.3e} rel_l2={rl2:.3e} worst_head_rel_l2={worst:.3e}")
    assert mx <= max_abs, f"{what}: max abs error {mx} > {max_abs}"
    assert rl2 <= rel_l2, f"{what}: relative L2 error {rl2} > {rel_l2}"
    return mx, rl2, worst
