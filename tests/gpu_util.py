"""Helpers shared by the GPU parity tests (marshalling and error metrics only)."""
import numpy as np


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round float values to bf16 (nearest even), returned as float64."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).bfloat16().double().numpy()


def to_dev_bf16(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).bfloat16().cuda()


def to_dev_f32(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def to_dev_i32(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def host(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().double().numpy()


def rel_l2(a, b) -> float:
    a = np.asarray(a, dtype=np.float64).ravel()
    b = np.asarray(b, dtype=np.float64).ravel()
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / den) if den > 0 else float(np.linalg.norm(a - b))


def cosine(a, b) -> float:
    a = np.asarray(a, dtype=np.float64).ravel()
    b = np.asarray(b, dtype=np.float64).ravel()
    na, nb = np.linalg.norm(a), np.linalg.norm(b)
    if na == 0 and nb == 0:
        return 1.0
    return float(a @ b / (na * nb))


def bf16_rne_bits(a: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even bf16 bit patterns of fp32 values (plain integer arithmetic)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


# Rounding constants of the element-wise error bounds.
U32 = 2.0 ** -24   # fp32 unit roundoff (round to nearest)
BF16 = 2.0 ** -8   # bf16 round to nearest: at most half of a 2^-7 relative spacing


def assert_elementwise(got, ref, tol, what=""):
    """|got - ref| <= tol for every element; the message names the count of violations
    and the worst element (index, values, bound)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    tol = np.broadcast_to(np.asarray(tol, dtype=np.float64), ref.shape)
    err = np.abs(got - ref)
    bad = ~(err <= tol)
    if np.any(bad):
        i = np.unravel_index(int(np.argmax(np.where(bad, err / np.maximum(tol, 1e-300), 0))), ref.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {ref.size} elements outside the bound; worst at {i}: "
                             f"got {got[i]!r}, ref {ref[i]!r}, bound {tol[i]!r}")


def abs_matmul(a, b):
    """|a| @ |b| in float32: the scale of a product's summation error (not a reference value)."""
    return np.abs(np.asarray(a, dtype=np.float32)) @ np.abs(np.asarray(b, dtype=np.float32))
