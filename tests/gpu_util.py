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


def normed_output_errors(got_y, ref_y, ref_state, q, z, gn, NV: int, NK: int, D: int,
                         eps: float):
    """Per-head errors of a gated-norm output y_i = w_i o_i / r, w = gn silu(z),
    r = sqrt(mean(o^2) + eps), o = S' q / sqrt(D), for one decode step whose
    updated state S' is ``ref_state`` (the oracle's).

    Returns three arrays over the (sequence, head) pairs:
      plain  max_i |dy_i| / max_i |y_i|;
      scaled max_i |dy_i| / max_i A_i, with A_i the first-order bound on |dy_i|
             per unit relative error of each summand of o: m_i = sum_j
             |S'_ij q_j| / sqrt(D) bounds the rounding of o_i, and
             A_i = |w_i| m_i / r + |y_i| |m| / (sqrt(D) r);
      kappa  max_i m_i / max_i |o_i|, the head's output condition number (how
             far o is a cancellation of larger terms).
    No method arithmetic on the expected values: y comes from the oracle; S' and
    q only scale the tolerance."""
    B = got_y.shape[0]
    g = np.arange(NV) % NK
    S = np.asarray(ref_state, np.float64)[:, :NV * D * D].reshape(B, NV, D, D)
    qh = np.asarray(q, np.float64)[:, :NK * D].reshape(B, NK, D)[:, g]
    m = np.einsum("bhij,bhj->bhi", np.abs(S), np.abs(qh)) / np.sqrt(D)
    o = np.einsum("bhij,bhj->bhi", S, qh) / np.sqrt(D)
    del S
    r = np.sqrt((o * o).mean(-1, keepdims=True) + eps)
    zz = np.asarray(z, np.float64)[:, :NV * D].reshape(B, NV, D)
    w = np.asarray(gn, np.float64) * zz / (1.0 + np.exp(-zz))
    y = np.asarray(ref_y, np.float64)[:, :NV * D].reshape(B, NV, D)
    dy = np.abs(np.asarray(got_y, np.float64)[:, :NV * D].reshape(B, NV, D) - y)
    A = np.abs(w) * m / r + np.abs(y) * np.sqrt((m * m).sum(-1, keepdims=True)) / (np.sqrt(D) * r)
    plain = (dy.max(-1) / np.abs(y).max(-1)).reshape(-1)
    scaled = (dy.max(-1) / A.max(-1)).reshape(-1)
    kappa = (m.max(-1) / np.abs(o).max(-1)).reshape(-1)
    return plain, scaled, kappa
