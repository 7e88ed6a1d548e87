"""Pins of the patch-formation oracle (oracle/patch_oracle.py) on the CPU.

Every pin compares the oracle with something other than itself: a deficit
built from a known spectrum (orthonormal P, Q from QR of seeded Gaussians and
chosen singular values), the closed form of the Eckart-Young residual,
standard RoPE written as a complex rotation (independent of the oracle's
relocation), and the reuse oracle closing the loop.  ``test_planted_mistakes``
breaks the formation oracle on purpose and checks that a pin catches each
mistake.
"""

import math

import numpy as np
import pytest

from oracle import kamera_oracle as ko
from oracle import patch_oracle as po

SIG = np.array([8.0, 5.0, 3.0, 2.0, 1.2, 0.7])   # distinct, r = 6


def _layout(H=2, D=64, o=0, R=None, base=1e4, style=ko.ROPE_HALF):
    return ko.Layout(num_layers=1, num_heads=H, head_dim=D, rope_offset=o,
                     rope_dim=D if R is None else R, rope_base=base, num_streams=2, rope_style=style)


def _rope(x, pos, lay):
    """Standard RoPE of raw keys x[T, F] at positions pos[T]: each pair (a, b)
    becomes (a + ib) exp(i pos theta_j), theta_j = base^(-2j/R) by math.pow."""
    y = np.array(x, np.float64)
    o, R, D = lay.rope_offset, lay.rope_dim, lay.head_dim
    for h in range(lay.num_heads):
        for j in range(R // 2):
            if lay.rope_style == ko.ROPE_HALF:
                ia, ib = h * D + o + j, h * D + o + j + R // 2
            else:
                ia, ib = h * D + o + 2 * j, h * D + o + 2 * j + 1
            z = (x[:, ia] + 1j * x[:, ib]) * np.exp(1j * np.asarray(pos, np.float64) * math.pow(lay.rope_base, -2.0 * j / R))
            y[:, ia], y[:, ib] = z.real, z.imag
    return y


def _spectrum_case(T=96, lay=None, seed=0):
    """canon = RoPE_p(k), target = RoPE_{p+delta}(k) + P diag(SIG) Q^T."""
    lay = lay or _layout()
    F = lay.row_width
    rng = np.random.default_rng(seed)
    P, _ = np.linalg.qr(rng.standard_normal((T, SIG.size)))
    Q, _ = np.linalg.qr(rng.standard_normal((F, SIG.size)))
    k = rng.standard_normal((T, F))
    p0, delta = 37, -1234
    pos = p0 + np.arange(T)
    canon = _rope(k, pos, lay)
    deficit = P @ np.diag(SIG) @ Q.T
    target = _rope(k, pos + delta, lay) + deficit
    return lay, canon, target, delta, P, Q, deficit


# ---------------------------------------------------------------------------
# Pins (each returns True when the oracle agrees)
# ---------------------------------------------------------------------------

def pin_top_m_of_known_spectrum():
    lay, canon, target, delta, P, Q, deficit = _spectrum_case()
    m = 4
    U, V, sig = po.form_patch_f64(canon, target, delta, lay, True, m)
    want = P[:, :m] @ np.diag(SIG[:m]) @ Q[:, :m].T          # Eckart-Young: the top-m part
    ok = np.allclose(U @ V.T, want, atol=1e-9)
    ok &= np.allclose(np.linalg.norm(U, axis=0), SIG[:m], rtol=1e-9)        # ||U_i|| = sigma_i
    ok &= np.allclose(V.T @ V, np.eye(m), atol=1e-9)                          # V orthonormal
    resid = np.linalg.norm(deficit - U @ V.T)
    ok &= abs(resid - math.sqrt(float(np.sum(SIG[m:] ** 2)))) < 1e-9          # residual closed form
    return bool(ok)


def pin_rank_r_exact_and_padding():
    lay, canon, target, delta, P, Q, deficit = _spectrum_case(seed=1)
    U, V, _ = po.form_patch_f64(canon, target, delta, lay, True, SIG.size)
    ok = np.allclose(U @ V.T, deficit, atol=1e-9)                            # rank(Delta) factors: exact
    U8, V8, _ = po.form_patch_f64(canon, target, delta, lay, True, 8)
    ok &= np.allclose(U8 @ V8.T, deficit, atol=1e-9)
    ok &= not U8[:, 6:].any() and not V8[:, 6:].any()                         # negligible columns are zero
    return bool(ok)


def pin_zero_deficit():
    # target = RoPE at the shifted positions exactly: nothing to patch
    lay, canon, target, delta, P, Q, deficit = _spectrum_case(seed=2)
    U, V, sig = po.form_patch_f64(canon, target - deficit, delta, lay, True, 4)
    return bool(np.max(np.abs(U @ V.T)) < 1e-9 * np.max(np.abs(canon)))


def pin_partial_span_interleaved():
    lay = _layout(H=1, D=128, o=64, R=64, style=ko.ROPE_INTERLEAVED, base=1e6)
    lay, canon, target, delta, P, Q, deficit = _spectrum_case(T=80, lay=lay, seed=3)
    U, V, _ = po.form_patch_f64(canon, target, delta, lay, True, SIG.size)
    return bool(np.allclose(U @ V.T, deficit, atol=1e-9))


def pin_unrotated_stream():
    # values (stream 1) are never rotated: Delta = target - canon
    rng = np.random.default_rng(4)
    lay = _layout()
    T, F = 64, lay.row_width
    P, _ = np.linalg.qr(rng.standard_normal((T, 3)))
    Q, _ = np.linalg.qr(rng.standard_normal((F, 3)))
    canon = rng.standard_normal((T, F))
    deficit = P @ np.diag([4.0, 2.0, 1.0]) @ Q.T
    U, V, _ = po.form_patch_f64(canon, canon + deficit, 999, lay, False, 3)
    return bool(np.allclose(U @ V.T, deficit, atol=1e-9))


def pin_sign_convention():
    lay, canon, target, delta, P, Q, deficit = _spectrum_case(seed=5)
    _, V, _ = po.form_patch_f64(canon, target, delta, lay, True, 5)
    return all(V[int(np.argmax(np.abs(V[:, i]))), i] > 0 for i in range(5))


def pin_closes_the_loop():
    # reuse(canon, delta, U, V) = target up to the Eckart-Young tail
    lay, canon, target, delta, P, Q, deficit = _spectrum_case(seed=6)
    m = 5
    U, V, _ = po.form_patch_f64(canon, target, delta, lay, True, m)
    y = ko.reuse_f64(canon, delta, U, V, lay, rotate=True)
    return abs(np.linalg.norm(y - target) - SIG[m]) < 1e-9


def pin_bits_round_once():
    lay, canon, target, delta, P, Q, deficit = _spectrum_case(seed=7)
    cb, tb = ko.f64_to_bf16_bits(canon), ko.f64_to_bf16_bits(target)
    ub, vb, U, V, _ = po.form_patch_bits(cb, tb, delta, lay, True, 4)
    ok = np.array_equal(ub, ko.f64_to_bf16_bits(U)) and np.array_equal(vb, ko.f64_to_bf16_bits(V))
    # the factors come from the widened bfloat16 rows, not from the float64 ones
    U2, V2, _ = po.form_patch_f64(ko.bf16_bits_to_f64(cb), ko.bf16_bits_to_f64(tb), delta, lay, True, 4)
    return bool(ok and np.array_equal(U, U2) and np.array_equal(V, V2))


def _orbit_case(T=48, seed=8):
    """A cached set of 3 chunks and every order of it.  A synthetic forward pass
    stands in for the model: chunk c placed at slot k after context A gets
    RoPE at positions base + k*T + t (the pin's own complex rotation) plus
    sum over c' in A of D[c][c'] (fixed rank-2 matrices).  Canonical rows are
    RoPE at positions t (p_c = 0)."""
    import itertools
    lay = _layout()
    F = lay.row_width
    rng = np.random.default_rng(seed)
    n, base = 3, 500
    keys = [rng.standard_normal((T, F)) for _ in range(n)]
    D = [[(rng.standard_normal((T, 2)) @ rng.standard_normal((2, F))) if c != d else None
          for d in range(n)] for c in range(n)]
    canon = [_rope(keys[c], np.arange(T), lay) for c in range(n)]
    views = {c: ([], []) for c in range(n)}   # chunk -> (targets, deltas)
    for order in itertools.permutations(range(n)):
        for k, c in enumerate(order):
            delta = base + k * T
            tgt = _rope(keys[c], delta + np.arange(T), lay)
            for d in order[:k]:
                tgt = tgt + D[c][d]
            views[c][0].append(tgt)
            views[c][1].append(delta)
    return lay, canon, views, D


def pin_orbit_brute_force_all_orders():
    # every other chunk precedes c in exactly half of the 3! orders, so the
    # orbit deficit is (1/2) sum_{d != c} D[c][d], and a patch of its rank
    # (2 + 2 = 4) reproduces it
    lay, canon, views, D = _orbit_case()
    ok = True
    for c in range(3):
        want = 0.5 * sum(D[c][d] for d in range(3) if d != c)
        got = po.orbit_deficit_f64(canon[c], views[c][0], views[c][1], lay, True)
        ok &= np.allclose(got, want, atol=1e-9)
        U, V, _ = po.form_orbit_patch_f64(canon[c], views[c][0], views[c][1], lay, True, 4)
        ok &= np.allclose(U @ V.T, want, atol=1e-9)
    return bool(ok)


def pin_orbit_single_view_is_plain_patch():
    lay, canon, target, delta, P, Q, deficit = _spectrum_case(seed=9)
    U1, V1, _ = po.form_orbit_patch_f64(canon, [target], [delta], lay, True, 4)
    U2, V2, _ = po.form_patch_f64(canon, target, delta, lay, True, 4)
    return bool(np.allclose(U1, U2, atol=1e-12) and np.allclose(V1, V2, atol=1e-12))


def pin_orbit_view_order_irrelevant():
    lay, canon, views, D = _orbit_case(seed=10)
    t, d = views[1]
    idx = [4, 1, 5, 0, 3, 2]
    a = po.orbit_deficit_f64(canon[1], t, d, lay, True)
    b = po.orbit_deficit_f64(canon[1], [t[i] for i in idx], [d[i] for i in idx], lay, True)
    return bool(np.allclose(a, b, atol=1e-12))


PINS = {
    "top_m": pin_top_m_of_known_spectrum,
    "rank_r": pin_rank_r_exact_and_padding,
    "zero": pin_zero_deficit,
    "partial_interleaved": pin_partial_span_interleaved,
    "unrotated": pin_unrotated_stream,
    "sign": pin_sign_convention,
    "loop": pin_closes_the_loop,
    "bits": pin_bits_round_once,
    "orbit_brute_force": pin_orbit_brute_force_all_orders,
    "orbit_single_view": pin_orbit_single_view_is_plain_patch,
    "orbit_view_order": pin_orbit_view_order_irrelevant,
}


@pytest.mark.parametrize("name", sorted(PINS))
def test_pin(name):
    assert PINS[name]()


# ---------------------------------------------------------------------------
# Planted mistakes
# ---------------------------------------------------------------------------

def _all():
    out = {}
    for k, f in PINS.items():
        try:
            out[k] = bool(f())
        except Exception:
            out[k] = False
    return out


def _mut_deficit_sign(canon, target, delta, layout, rotate):
    c = np.asarray(canon, np.float64)
    rel = ko.relocate_f64(c, delta, layout) if rotate else c
    return rel - np.asarray(target, np.float64)


def _mut_deficit_unshifted(canon, target, delta, layout, rotate):
    return np.asarray(target, np.float64) - np.asarray(canon, np.float64)


def _mut_deficit_reverse_shift(canon, target, delta, layout, rotate):
    c = np.asarray(canon, np.float64)
    rel = ko.relocate_f64(c, -delta, layout) if rotate else c
    return np.asarray(target, np.float64) - rel


def _mut_sigma_on_v(d, m):
    U, V, sig = _orig_factors(d, m)
    n = np.linalg.norm(U, axis=0)
    n[n == 0] = 1
    return U / n, V * n, sig


def _mut_bottom_m(d, m):
    uu, sig, vt = np.linalg.svd(np.asarray(d, np.float64), full_matrices=False)
    r = sig.size
    idx = list(range(r - 1, r - 1 - m, -1))
    U = np.zeros((d.shape[0], m))
    V = np.zeros((d.shape[1], m))
    for c, i in enumerate(idx):
        if i >= 0:
            U[:, c], V[:, c] = uu[:, i] * sig[i], vt[i]
    return U, V, sig


def _mut_no_sign_fix(d, m):
    uu, sig, vt = np.linalg.svd(np.asarray(d, np.float64), full_matrices=False)
    U = np.zeros((d.shape[0], m))
    V = np.zeros((d.shape[1], m))
    for i in range(min(m, sig.size)):
        if sig[i] > po.NEGLIGIBLE * sig[0]:
            U[:, i], V[:, i] = -uu[:, i] * sig[i], -vt[i]
    return U, V, sig


def _mut_keep_noise_columns(d, m):
    uu, sig, vt = np.linalg.svd(np.asarray(d, np.float64), full_matrices=False)
    U = np.zeros((d.shape[0], m))
    V = np.zeros((d.shape[1], m))
    for i in range(min(m, sig.size)):
        s = 1.0 if vt[i][int(np.argmax(np.abs(vt[i])))] >= 0 else -1.0
        U[:, i], V[:, i] = s * uu[:, i] * sig[i], s * vt[i]
    return U, V, sig


_orig_factors = po.truncated_svd_factors


def _mut_orbit_sum(canon, targets, deltas, layout, rotate):
    return sum(po.deficit_f64(canon, t, d, layout, rotate) for t, d in zip(targets, deltas))


def _mut_orbit_first_view(canon, targets, deltas, layout, rotate):
    return po.deficit_f64(canon, targets[0], deltas[0], layout, rotate)


def _mut_orbit_one_shift(canon, targets, deltas, layout, rotate):
    return sum(po.deficit_f64(canon, t, deltas[0], layout, rotate) for t in targets) / len(targets)


@pytest.mark.parametrize("name,attr,mutant", [
    ("deficit sign", "deficit_f64", _mut_deficit_sign),
    ("deficit without relocation", "deficit_f64", _mut_deficit_unshifted),
    ("deficit relocated by -delta", "deficit_f64", _mut_deficit_reverse_shift),
    ("singular values on V", "truncated_svd_factors", _mut_sigma_on_v),
    ("bottom-m factors", "truncated_svd_factors", _mut_bottom_m),
    ("sign convention dropped", "truncated_svd_factors", _mut_no_sign_fix),
    ("negligible columns kept", "truncated_svd_factors", _mut_keep_noise_columns),
    ("orbit: sum instead of mean", "orbit_deficit_f64", _mut_orbit_sum),
    ("orbit: first view only", "orbit_deficit_f64", _mut_orbit_first_view),
    ("orbit: one shift for every view", "orbit_deficit_f64", _mut_orbit_one_shift),
])
def test_planted_mistakes(monkeypatch, name, attr, mutant):
    assert all(_all().values())
    monkeypatch.setattr(po, attr, mutant)
    res = _all()
    assert not all(res.values()), f"no pin caught the planted mistake: {name}"
