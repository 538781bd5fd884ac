"""Shared helpers for the parity tests: tolerances and comparison rules.

Tolerances (written here, used by every GPU parity test):
  * block indices: identical to the oracle, except that a swap between a
    GPU-only and an oracle-only block is excused when the oracle's pooled
    scores of the two differ by at most 1e-4 relative (near-ties);
  * outputs: max-abs <= 1e-2 and ||o - o_ref|| / ||o_ref|| <= 1e-2 for bf16
    inputs, 1e-4 for both with fp32 inputs; lse within 2e-3 (bf16) / 1e-5
    (fp32) absolute.
"""
from __future__ import annotations

import numpy as np
import torch

TIE_REL = 1e-4
TOL = {torch.bfloat16: dict(max_abs=1e-2, rel_l2=1e-2, lse=2e-3),
       torch.float32: dict(max_abs=1e-4, rel_l2=1e-4, lse=1e-5)}


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


def compare_index_rows(gpu_ids, ora_ids, pooled, diags, force_local=True):
    """Check GPU block lists against the oracle row by row.

    gpu_ids/ora_ids [rows, h_kv, k] int; pooled: list (per row) of
    [h_kv, diag+1] oracle pooled scores.  Returns (n_exact, n_excused);
    raises AssertionError on any other difference."""
    gpu_ids = np.asarray(gpu_ids)
    ora_ids = np.asarray(ora_ids)
    n_exact = n_excused = 0
    for t in range(ora_ids.shape[0]):
        for r in range(ora_ids.shape[1]):
            g = gpu_ids[t, r]
            o = ora_ids[t, r]
            if np.array_equal(g, o):
                n_exact += 1
                continue
            gv, ov = g[g >= 0], o[o >= 0]
            assert len(gv) == len(ov), f"row {t} group {r}: {g} vs oracle {o}"
            assert np.all(np.diff(gv) > 0), f"row {t} group {r}: not ascending {g}"
            assert np.all(g[len(gv):] == -1)
            if force_local:
                assert diags[t] in gv, f"row {t} group {r}: diagonal {diags[t]} missing in {g}"
            m = pooled[t][r]
            assert gv.max() <= diags[t]
            only_g = sorted(set(gv.tolist()) - set(ov.tolist()))
            only_o = sorted(set(ov.tolist()) - set(gv.tolist()))
            for x in only_g:
                for y in only_o:
                    a, b = m[x], m[y]
                    assert abs(a - b) <= TIE_REL * max(abs(a), abs(b)), (
                        f"row {t} group {r}: GPU picked {x} ({a}) over {y} ({b}); lists {g} vs {o}")
            n_excused += 1
    return n_exact, n_excused


def compare_out(o_gpu, o_ref, dtype, what="o", rel_elem=0.0):
    """Outputs within the tolerance.  ``rel_elem`` adds rel_elem * |o_ref| to
    the max-abs bound of each element: for inputs whose outputs reach well
    above 1 (the MXFP8 tests' block scales reach 2^4), a bf16 output carries a
    rounding error of up to 2^-9 of its own magnitude, which a fixed absolute
    bound does not cover."""
    tol = TOL[dtype]
    og = np64(o_gpu) if isinstance(o_gpu, torch.Tensor) else np.asarray(o_gpu, np.float64)
    orf = np.asarray(o_ref, np.float64)
    assert og.shape == orf.shape, (og.shape, orf.shape)
    assert np.all(np.isfinite(og)), f"{what}: non-finite values"
    err = np.abs(og - orf)
    max_abs = float(err.max()) if err.size else 0.0
    rel = float(np.linalg.norm(og - orf) / max(np.linalg.norm(orf), 1e-30))
    if rel_elem > 0.0:
        excess = err - rel_elem * np.abs(orf)
        max_abs = float(excess.max()) if excess.size else 0.0
    assert max_abs <= tol["max_abs"], f"{what}: max-abs {max_abs:.3e} > {tol['max_abs']}"
    assert rel <= tol["rel_l2"], f"{what}: relative L2 {rel:.3e} > {tol['rel_l2']}"
    return max_abs, rel


def compare_lse(l_gpu, l_ref, dtype):
    """lse within the tolerance; rows with no visible key must be -inf on both sides."""
    tol = TOL[dtype]["lse"]
    lg = np64(l_gpu)
    lr = np.asarray(l_ref, np.float64)
    empty = np.isneginf(lr)
    assert np.array_equal(np.isneginf(lg), empty), "lse: -inf rows differ"
    err = np.zeros_like(lr)
    err[~empty] = np.abs(lg[~empty] - lr[~empty])
    assert float(err.max()) <= tol, f"lse: max-abs {float(err.max()):.3e} > {tol}"
    return float(err.max())


# Gradients (bf16 outputs of fp32 accumulations whose operands P and dS are
# rounded to bf16 for the MFMA): relative to the gradient's own scale.
GRAD_TOL = {"max_rel_to_max": 1e-2, "rel_l2": 1e-2}


def compare_grad(g_gpu, g_ref, what="grad"):
    gg = np64(g_gpu) if isinstance(g_gpu, torch.Tensor) else np.asarray(g_gpu, np.float64)
    gr = np.asarray(g_ref, np.float64)
    assert gg.shape == gr.shape, (gg.shape, gr.shape)
    assert np.all(np.isfinite(gg)), f"{what}: non-finite values"
    scale = float(np.abs(gr).max()) if gr.size else 0.0
    err = np.abs(gg - gr)
    max_err = float(err.max()) if err.size else 0.0
    rel = float(np.linalg.norm(gg - gr) / max(np.linalg.norm(gr), 1e-30))
    assert max_err <= GRAD_TOL["max_rel_to_max"] * max(scale, 1e-30), \
        f"{what}: max error {max_err:.3e} > {GRAD_TOL['max_rel_to_max']} x max|ref| {scale:.3e}"
    assert rel <= GRAD_TOL["rel_l2"], f"{what}: relative L2 {rel:.3e} > {GRAD_TOL['rel_l2']}"
    return max_err / max(scale, 1e-30), rel
