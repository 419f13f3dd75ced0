"""Helpers shared by the GPU parity tests (comparison metrics and host<->device moves only)."""
import numpy as np
import torch


def dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    """Stored host array ('bf16' uint16 bits, 'f32', 'f64', ints) -> GPU tensor with the same bytes."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def sin_theta_max(V_hat: np.ndarray, V: np.ndarray, k: int) -> float:
    """sin of the largest principal angle between span(V_hat[:, :k]) and span(V[:, :k]) (fp64)."""
    Vh = np.asarray(V_hat[:, :k], dtype=np.float64)
    Vk = np.asarray(V[:, :k], dtype=np.float64)
    R = Vh - Vk @ (Vk.T @ Vh)
    return float(np.linalg.norm(R, 2))


def check_lambda(lam_hat, lam, tol=1e-5):
    err = np.max(np.abs(np.asarray(lam_hat) - np.asarray(lam))) / abs(lam[0])
    assert err <= tol, "eigenvalue error %.3e lambda_max (limit %.1e)" % (err, tol)
    return err


# Below rel * eps_0 the relative check gives way to an absolute floor that depends on the
# eigensolver's working precision.  C is accumulated and stored in fp32, so tail sums smaller
# than about one fp32 unit of its trace are not resolved by any method that keeps C in fp32:
# rounding the exact C once to fp32 already moves the tail of a rank-deficient spectrum by about
# 1e-8 eps_0 (8.3e-9 eps_0 measured on the 16384 x 512 -> 640 block case), the fp32 accumulation
# of that C over the tokens by 2.2e-8 eps_0 (the same case, LAPACK on the GPU's C), and an fp32
# eigensolver adds rounding of its own of a few 1e-8 eps_0.
#   prec 1 (fp32 tridiagonalisation and back-transformation): 2^-23 eps_0 (1.2e-7);
#   prec 2 (fp64 eigensolver, and the n <= 128 Jacobi path, which always runs in fp64): 2^-24 eps_0
#   (6.0e-8), 2.7 times the accumulation's measured share.
EPS_FLOOR = {1: 2.0 ** -23, 2: 2.0 ** -24}


def check_eps(eps_hat, eps, rel=1e-4, prec=1):
    """eps_k within rel relative where eps_k >= rel * eps_0; elsewhere within EPS_FLOOR[prec] * eps_0."""
    floor = EPS_FLOOR[prec]
    eps_hat = np.asarray(eps_hat, dtype=np.float64)
    eps = np.asarray(eps, dtype=np.float64)
    big = eps >= rel * eps[0]
    e_big = np.max(np.abs(eps_hat[big] - eps[big]) / eps[big]) if big.any() else 0.0
    e_small = np.max(np.abs(eps_hat[~big] - eps[~big])) / eps[0] if (~big).any() else 0.0
    assert e_big <= rel, "eps relative error %.3e (limit %.1e)" % (e_big, rel)
    assert e_small <= floor, "eps tail error %.3e eps_0 (limit %.1e)" % (e_small, floor)
    return e_big, e_small


def gap(lam, k):
    return (lam[k - 1] - lam[k]) / lam[0]
