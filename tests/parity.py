"""Helpers shared by the GPU parity tests: device upload and the tolerance checks.

Tolerance (stated for bf16 I/O with fp32 accumulation): max-abs <= 1e-2 and
relative L2 <= 4e-3 against the fp64 oracle, for O and for the finite LSE
entries; -inf LSE entries must match exactly. A bf16 output cannot be closer
to the exact value than half a bf16 spacing, which exceeds 1e-2 once |O| >= 4,
so for bf16 O the per-element bound is 1e-2 plus half the bf16 spacing at the
exact value (the kernel's own arithmetic error stays within 1e-2; the single
final rounding adds at most half a spacing). fp32 outputs get the plain bound.
"""
import numpy as np
import torch

from oracle import fullcheck as fc

MAX_ABS = 1e-2
REL_L2 = 4e-3


def up(bits: np.ndarray, device="cuda") -> torch.Tensor:
    """uint16 bf16 bit array -> bf16 device tensor (same bits)."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def down(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def half_spacing_bf16(x: np.ndarray) -> np.ndarray:
    ax = np.abs(x)
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -126)))
    return 2.0 ** (e - 8)


def check_o(o_gpu: np.ndarray, o_ref: np.ndarray, bf16: bool, what: str = "O") -> dict:
    err = np.abs(o_gpu - o_ref)
    bound = MAX_ABS + (half_spacing_bf16(o_ref) if bf16 else 0.0)
    nref = np.linalg.norm(o_ref)
    rel = np.linalg.norm(o_gpu - o_ref) / nref if nref > 0 else np.linalg.norm(o_gpu)
    worst = np.unravel_index(np.argmax(err - bound), err.shape) if err.size else None
    info = {"max_abs": float(err.max()) if err.size else 0.0, "rel_l2": float(rel),
            "floor": float(np.abs(o_ref - bf16_round(o_ref)).max()) if bf16 and err.size else 0.0}
    assert np.isfinite(o_gpu).all(), f"{what}: non-finite output"
    assert (err <= bound).all(), (f"{what}: |err| {err[worst]:.4e} > bound {np.broadcast_to(bound, err.shape)[worst]:.4e} "
                                  f"at {worst} (gpu {o_gpu[worst]}, ref {o_ref[worst]}); {info}")
    assert rel <= REL_L2, f"{what}: rel-L2 {rel:.3e} > {REL_L2}; {info}"
    return info


def check_lse(l_gpu: np.ndarray, l_ref: np.ndarray, what: str = "LSE") -> dict:
    ninf = np.isneginf(l_ref)
    assert np.array_equal(np.isneginf(l_gpu), ninf), f"{what}: -inf pattern differs"
    g, r = l_gpu[~ninf], l_ref[~ninf]
    if g.size == 0:
        return {"max_abs": 0.0, "rel_l2": 0.0}
    assert np.isfinite(g).all(), f"{what}: non-finite entries"
    err = np.abs(g - r)
    rel = np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300)
    assert err.max() <= MAX_ABS, f"{what}: max-abs {err.max():.4e} > {MAX_ABS}"
    assert rel <= REL_L2, f"{what}: rel-L2 {rel:.3e} > {REL_L2}"
    return {"max_abs": float(err.max()), "rel_l2": float(rel)}


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float64 to the nearest bf16 value (ties to even) -- used only for reporting the floor."""
    f, e = np.frexp(x)
    sp = np.ldexp(1.0, np.maximum(e, -125) - 8)
    return np.rint(x / sp) * sp


def check_grad(g_gpu: np.ndarray, g_ref: np.ndarray, a_ref: np.ndarray, r_ref: np.ndarray, what: str) -> dict:
    """Gradient check (bf16 output), with the bound of oracle.fullcheck.grad_bound. The
    tolerance stated for O and LSE does not cover gradients; this one follows from the
    arithmetic. Besides the output rounding, bf16 roundings (unit roundoff u = 2^-8) of one
    factor of every product term enter each gradient element: dS for dQ, P for dV, and for
    dK both the rounding of dS and, at d = 128, that of the P it is formed from; D_i is
    formed from the bf16 O the forward returns. a_ref and r_ref (oracle, abs_terms) are the
    element's worst-case and root-sum-square first-order sensitivities to relative changes
    of those factors, so k roundings give an error of at most k u a_ref and, independent
    and uniform in [-u, u], an RMS of sqrt(k) (u / sqrt(3)) r_ref. fp32 arithmetic and the
    fp32 LSE add far less and are covered by the forward's 1e-2. Per element:
    |err| <= 1e-2 + half a bf16 spacing at the exact value + k 2^-8 a_ref.
    Per tensor, the forward's rel-L2 bar plus twice the expected RMS of the roundings:
    ||err||_2 <= 4e-3 ||g_ref||_2 + 2 sqrt(k) (2^-8 / sqrt(3)) ||r_ref||_2.
    """
    k = fc.GRAD_ROUNDINGS[what]
    err = np.abs(g_gpu - g_ref)
    bound = fc.grad_bound(g_ref, a_ref, k)
    nref = np.linalg.norm(g_ref)
    rel = np.linalg.norm(g_gpu - g_ref) / nref if nref > 0 else np.linalg.norm(g_gpu)
    rel_bound = fc.grad_rel_bound(nref, np.linalg.norm(r_ref), k)
    worst = np.unravel_index(np.argmax(err - bound), err.shape) if err.size else None
    info = {"max_abs": float(err.max()) if err.size else 0.0, "rel_l2": float(rel), "rel_l2_bound": float(rel_bound),
            "max_err_over_bound": float((err / bound).max()) if err.size else 0.0}
    assert np.isfinite(g_gpu).all(), f"{what}: non-finite output"
    assert (err <= bound).all(), (f"{what}: |err| {err[worst]:.4e} > bound {bound[worst]:.4e} at {worst} "
                                  f"(gpu {g_gpu[worst]}, ref {g_ref[worst]}, abs-terms {a_ref[worst]:.4e}); {info}")
    assert rel <= rel_bound, f"{what}: rel-L2 {rel:.3e} > {rel_bound:.3e}; {info}"
    return info
