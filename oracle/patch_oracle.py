"""CPU oracle of Kamera patch formation.  TEST INFRASTRUCTURE ONLY.

Only ``tests/`` and the ``cpu_baseline`` leg of ``bench.py`` may import this
module.  The product path never imports, calls or links it, and it imports
nothing from the product package.

Source: "Kamera: Unified Position-Invariant Multimodal KV Cache for
Training-Free Reuse", technical summaries on gist.science (paper 2606.23581),
section 2 "Methodology: the Kamera operator", "Patch application" bullet: the
rank-m patch is computed once, from one forward pass conditioned on [A, B],
followed by a singular value decomposition that keeps the top-m factors.
Section 1 names the quantity the patch stands for, the deficit
KV(B|A) - KV(B|empty).

The forward pass needs model weights and is not part of this oracle: its
output KV(B|A) (the rows of chunk B prefilled after A, at their positions in
that context) is an input.  What remains has a plain definition, written out
here in float64:

* the deficit in the destination frame, i.e. the reuse equation solved for
  the patch (it must restore KV(B|A) exactly after the relocation):

      Delta = KV(B|A) - R(delta) KV(B|empty)

  with R(delta) the same exact RoPE re-rotation the reuse oracle applies
  (stream 0 only; values and c_KV are not rotated);
* its truncated SVD, Delta ~ U_m Sigma_m V_m^T, returned as the factors the
  reuse operator consumes: U = U_m Sigma_m (T x m) and V = V_m (F x m);
* conventions that make the factors unique where the SVD is (distinct
  singular values): each column of V has its largest-magnitude entry (the
  first such entry on a tie) positive; columns whose singular value is at most
  1e-6 of the largest are returned as zeros (their contribution is far below
  the bfloat16 resolution of the patch).

The orbit patch (section 3, "Three cheap window operations", Reorder: one
patch, averaged over permutations, serves every ordering of a cached set) is
read the same way: the patch is added after R(delta) in every order, so the
deficit it stands for is the mean over the sampled orders of each order's
deficit in its own destination frame,

      Delta_orbit = (1/P) sum_p [ KV_p(B|A_p) - R(delta_p) KV(B|empty) ],

and the orbit patch is its rank-m truncated SVD.  With P = 1 it is the plain
patch.

Nothing is blocked, fused or reordered beyond that definition; numpy's SVD is
the library routine that serves as the decomposition step.
"""

from __future__ import annotations

import numpy as np

from . import kamera_oracle as ko

NEGLIGIBLE = 1e-6   # singular values <= NEGLIGIBLE * sigma_1 give zero columns


def deficit_f64(canon, target, delta: int, layout: "ko.Layout", rotate: bool) -> np.ndarray:
    """Delta = KV(B|A) - R(delta) KV(B|empty) for one (chunk, layer, stream) block [T, F].

    Kamera summary, section 1 (the deficit) and section 2 (reuse equation):
    R(delta) KV(B|empty) + Delta reproduces KV(B|A) exactly.
    """
    c = np.asarray(canon, np.float64)
    rel = ko.relocate_f64(c, delta, layout) if rotate else c
    return np.asarray(target, np.float64) - rel


def truncated_svd_factors(d: np.ndarray, m: int):
    """Top-m factors of d [T, F]: (U_m Sigma_m [T, m], V_m [F, m], sigma [min(T, F)]).

    Kamera summary, section 2, "Patch application": an SVD extracts the top-m
    factors.  Sign and negligible-column conventions: see the module header.
    """
    d = np.asarray(d, np.float64)
    T, F = d.shape
    uu, sig, vt = np.linalg.svd(d, full_matrices=False)
    k = min(m, sig.size)
    U = np.zeros((T, m))
    V = np.zeros((F, m))
    top = sig[0] if sig.size else 0.0
    for i in range(k):
        if not (sig[i] > NEGLIGIBLE * top):
            break
        u_i, v_i = uu[:, i], vt[i]
        if v_i[int(np.argmax(np.abs(v_i)))] < 0:
            u_i, v_i = -u_i, -v_i
        U[:, i] = u_i * sig[i]
        V[:, i] = v_i
    return U, V, sig


def form_patch_f64(canon, target, delta: int, layout: "ko.Layout", rotate: bool, m: int):
    """(U, V, sigma) of the rank-m patch of one block, float64."""
    return truncated_svd_factors(deficit_f64(canon, target, delta, layout, rotate), m)


def form_patch_bits(canon_bits, target_bits, delta: int, layout: "ko.Layout", rotate: bool, m: int):
    """The rank-m patch of one block from bfloat16 rows: (u_bits [T, m], v_bits [F, m], U, V, sigma).

    Inputs are widened exactly; each factor element is rounded once to
    bfloat16 (nearest even), the storage format the reuse operator reads.
    """
    U, V, sig = form_patch_f64(ko.bf16_bits_to_f64(canon_bits), ko.bf16_bits_to_f64(target_bits),
                               delta, layout, rotate, m)
    return ko.f64_to_bf16_bits(U), ko.f64_to_bf16_bits(V), U, V, sig


def orbit_deficit_f64(canon, targets, deltas, layout: "ko.Layout", rotate: bool) -> np.ndarray:
    """Mean over the views p of KV_p(B|A_p) - R(delta_p) KV(B|empty), one block [T, F].

    Kamera summary, section 3, Reorder: one orbit patch, averaged over
    permutations, serves every ordering of the cached set.
    """
    acc = None
    for t, d in zip(targets, deltas):
        x = deficit_f64(canon, t, d, layout, rotate)
        acc = x if acc is None else acc + x
    return acc / len(targets)


def form_orbit_patch_f64(canon, targets, deltas, layout: "ko.Layout", rotate: bool, m: int):
    """(U, V, sigma) of the rank-m orbit patch of one block, float64."""
    return truncated_svd_factors(orbit_deficit_f64(canon, targets, deltas, layout, rotate), m)


def form_orbit_patch_bits(canon_bits, target_bits, deltas, layout: "ko.Layout", rotate: bool, m: int):
    """The orbit patch from bfloat16 rows: (u_bits, v_bits, U, V, sigma); target_bits [P, T, F]."""
    U, V, sig = form_orbit_patch_f64(ko.bf16_bits_to_f64(canon_bits),
                                     [ko.bf16_bits_to_f64(t) for t in target_bits], deltas, layout, rotate, m)
    return ko.f64_to_bf16_bits(U), ko.f64_to_bf16_bits(V), U, V, sig
