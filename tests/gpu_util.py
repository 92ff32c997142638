"""Helpers shared by the GPU parity tests (no method arithmetic here)."""
import numpy as np

DEV = "cuda:0"


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    import torch
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    if t.dtype == torch.float16:
        return t.cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float64 (exact: the top half of a binary32)."""
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f16_to_f64(bits: np.ndarray) -> np.ndarray:
    return bits.view(np.float16).astype(np.float64)


def _group_ratio(diff, scale):
    # one entry per head: its max abs error over its max abs reference value
    with np.errstate(invalid="ignore", divide="ignore"):
        rat = np.where(scale > 0, diff / np.where(scale > 0, scale, 1), diff)
    return float(rat.max()) if rat.size else 0.0


def tile_err(got_state, ref_state, NV: int, D: int) -> float:
    """Per (sequence, head) tile: max|got - ref| / max|ref|, maximum over tiles."""
    g = np.asarray(got_state, dtype=np.float64)[:, :NV * D * D].reshape(-1, D * D)
    r = np.asarray(ref_state, dtype=np.float64)[:, :NV * D * D].reshape(-1, D * D)
    return _group_ratio(np.abs(g - r).max(axis=1), np.abs(r).max(axis=1))


def out_err(got, ref, NV: int, D: int) -> float:
    """Per (row, head) output vector: max|got - ref| / max|ref|, maximum over them."""
    g = np.asarray(got, dtype=np.float64)[:, :NV * D].reshape(-1, D)
    r = np.asarray(ref, dtype=np.float64)[:, :NV * D].reshape(-1, D)
    return _group_ratio(np.abs(g - r).max(axis=1), np.abs(r).max(axis=1))


def bf16_ok(got_bits, ref, NV: int, D: int, tol: float) -> float:
    """Worst ratio of |y_hat - y| to the allowed 2^-8 |y| + tol max_head |y| (<= 1 passes)."""
    g = bf16_to_f64(np.asarray(got_bits))[:, :NV * D].reshape(-1, D)
    r = np.asarray(ref, dtype=np.float64)[:, :NV * D].reshape(-1, D)
    allow = 2.0 ** -8 * np.abs(r) + tol * np.abs(r).max(axis=1, keepdims=True)
    allow = np.where(allow > 0, allow, 1e-30)
    return float((np.abs(g - r) / allow).max())
