"""Pins of the CPU oracle against facts the Kamera pages and mathematics fix.

Nothing here calls the HIP library.  Each pin checks the oracle against
something other than itself: hand-derived rounding cases, closed forms of the
RoPE frequencies, an independent formulation of standard RoPE, library
routines (cos/sin, matmul, SVD), brute force on tiny inputs, and the figures
the pages print.  ``test_planted_mistakes`` then breaks the oracle on purpose,
on the CPU, and checks that some pin fails for each plausible mistake.
"""

import math
import os

import numpy as np
import pytest
import torch

from oracle import kamera_oracle as ko
from oracle import scalar_oracle as so
from workloads import SENTINEL_BITS, TINY, bits, make_inputs, small_workload

RNG = np.random.default_rng(1234)


def gqa_layout(H=2, D=64, base=1e4, style=ko.ROPE_HALF, o=0, R=None, L=1, S=2):
    return ko.Layout(num_layers=L, num_heads=H, head_dim=D, rope_offset=o,
                     rope_dim=D if R is None else R, rope_base=base, num_streams=S,
                     rope_style=style)


# ---------------------------------------------------------------------------
# Independent formulations used by the pins
# ---------------------------------------------------------------------------

def rope_reference(x, pos, layout):
    """Standard RoPE of raw keys x[T, F] at positions pos[T], written as a
    complex rotation: each pair (a, b) is a + ib multiplied by exp(i pos theta_j).
    theta_j comes from its closed form base^(-2j/R) evaluated with math.pow.
    """
    x = np.asarray(x, np.float64)
    y = x.copy()
    o, R, D = layout.rope_offset, layout.rope_dim, layout.head_dim
    for h in range(layout.num_heads):
        for j in range(R // 2):
            if layout.rope_style == ko.ROPE_HALF:
                ia, ib = h * D + o + j, h * D + o + j + R // 2
            else:
                ia, ib = h * D + o + 2 * j, h * D + o + 2 * j + 1
            theta = math.pow(layout.rope_base, -2.0 * j / R)
            z = (x[:, ia] + 1j * x[:, ib]) * np.exp(1j * np.asarray(pos, np.float64) * theta)
            y[:, ia], y[:, ib] = z.real, z.imag
    return y


def rope_reference_rotate_half(x, pos, layout):
    """The rotate-half RoPE convention written with concatenations:
    y = x * cat(cos, cos) + cat(-x2, x1) * cat(sin, sin) on each head's span."""
    x = np.asarray(x, np.float64)
    y = x.copy()
    o, R, D = layout.rope_offset, layout.rope_dim, layout.head_dim
    inv = np.array([math.pow(layout.rope_base, -2.0 * j / R) for j in range(R // 2)])
    ang = np.outer(np.asarray(pos, np.float64), inv)
    cos2 = np.concatenate([np.cos(ang), np.cos(ang)], axis=1)
    sin2 = np.concatenate([np.sin(ang), np.sin(ang)], axis=1)
    for h in range(layout.num_heads):
        span = x[:, h * D + o: h * D + o + R]
        x1, x2 = span[:, : R // 2], span[:, R // 2:]
        y[:, h * D + o: h * D + o + R] = span * cos2 + np.concatenate([-x2, x1], axis=1) * sin2
    return y


def bf16_rand(shape, sigma=1.0):
    return bits(torch.from_numpy(RNG.normal(0, sigma, shape).astype(np.float32)).to(torch.bfloat16))


# ---------------------------------------------------------------------------
# Pin functions (return True when the oracle satisfies the pin)
# ---------------------------------------------------------------------------

def pin_rounding_golden(golden_dir):
    path = os.path.join(golden_dir, "bf16_rne_cases.txt")
    ok = True
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        hx, want = line.split()[:2]
        got = int(ko.f64_to_bf16_bits(np.float64(float.fromhex(hx))))
        ok &= got == int(want, 16)
    return ok


def pin_rounding_vs_torch():
    # binary32 values (so torch's binary32 -> bfloat16 RNE rounds only once),
    # many of them exact ties: a bfloat16 value plus half its spacing.
    base = RNG.normal(0, 3, 20000).astype(np.float32)
    b16 = torch.from_numpy(base).to(torch.bfloat16).float().numpy()
    spacing = np.abs(b16) * np.float32(2.0 ** -8)
    ties = (b16 + np.sign(b16) * spacing).astype(np.float32)
    vals = np.concatenate([base, ties, base * np.float32(1e-38), base * np.float32(1e30)])
    want = bits(torch.from_numpy(vals).to(torch.bfloat16))
    got = ko.f64_to_bf16_bits(vals.astype(np.float64))
    return np.array_equal(got, want)


def pin_theta_closed_forms():
    ok = np.array_equal(ko.rope_inv_freq(2, 1e4), [1.0])
    t4 = ko.rope_inv_freq(4, 1e4)
    ok &= abs(t4[0] - 1.0) < 1e-15 and abs(t4[1] - 0.01) < 1e-15
    for R, base in [(64, 1e4), (128, 1e6), (64, 5e5)]:
        t = ko.rope_inv_freq(R, base)
        ok &= len(t) == R // 2 and t[0] == 1.0
        ok &= abs(t[R // 4] - base ** -0.5) < 1e-14 * max(1.0, base ** -0.5)
        r = t[1:] / t[:-1]
        ok &= np.allclose(r, r[0], rtol=1e-12, atol=0) and r[0] < 1
    return bool(ok)


def pin_rope_equivalence(style):
    # canonical keys = RoPE at p + t; relocating by delta must equal RoPE at p + delta + t
    lay = gqa_layout(H=3, D=64, base=1e4, style=style)
    T = 17
    k = RNG.normal(0, 1, (T, lay.row_width))
    ok = True
    for p, d in [(0, 300), (1000, -713), (5, 32768), (40000, -32768), (0, 0)]:
        pos = p + np.arange(T)
        canon = rope_reference(k, pos, lay)
        moved = ko.relocate_f64(canon, d, lay)
        want = rope_reference(k, pos + d, lay)
        ok &= np.max(np.abs(moved - want)) <= 1e-9 * np.max(np.abs(want))
        if style == ko.ROPE_HALF:
            want2 = rope_reference_rotate_half(k, pos + d, lay)
            ok &= np.max(np.abs(moved - want2)) <= 1e-9 * np.max(np.abs(want2))
    return bool(ok)


def pin_unit_vectors():
    lay = gqa_layout(H=1, D=8, base=1e4)
    ok = True
    for d in [1, 7, -300, 32768]:
        for j in range(4):
            e = np.zeros((1, 8))
            e[0, j] = 1.0
            y = ko.relocate_f64(e, d, lay)
            ang = d * math.pow(1e4, -2.0 * j / 8)
            ok &= abs(y[0, j] - math.cos(ang)) < 1e-12 and abs(y[0, j + 4] - math.sin(ang)) < 1e-12
            ok &= np.count_nonzero(y) <= 2
    return bool(ok)


def pin_patch_alone():
    # zero canonical rows: output = bf16(U V^T); shapes make a transposed operand fail
    lay = gqa_layout(H=3, D=64)
    T, m = 37, 8
    u, v = bf16_rand((T, m), 1.0), bf16_rand((lay.row_width, m), 1.0)
    zero = np.zeros((T, lay.row_width), np.uint16)
    got = ko.reuse_block_bits(zero, 123, u, v, lay, rotate=True)
    want = ko.f64_to_bf16_bits(np.matmul(ko.bf16_bits_to_f64(u), ko.bf16_bits_to_f64(v).T))
    return np.array_equal(got, want)


def pin_lowrank_reconstruction():
    # Synthetic deficit of rank r: the top-r SVD factors reproduce KV(B|A) exactly
    # (in float64); fewer factors leave the Eckart-Young residual.
    lay = gqa_layout(H=2, D=64)
    T, F, r = 48, lay.row_width, 6
    canon = RNG.normal(0, 1, (T, F))
    P, Q = RNG.normal(0, 0.3, (T, r)), RNG.normal(0, 0.3, (F, r))
    target = ko.relocate_f64(canon, 700, lay) + P @ Q.T
    Uf, sv, Vt = np.linalg.svd(P @ Q.T, full_matrices=False)
    ok = True
    U_r, V_r = Uf[:, :r] * sv[:r], Vt[:r].T
    got = ko.reuse_f64(canon, 700, U_r, V_r, lay, rotate=True)
    ok &= np.max(np.abs(got - target)) < 1e-12 * np.max(np.abs(target))
    for mm in (1, 3, 5):
        got = ko.reuse_f64(canon, 700, Uf[:, :mm] * sv[:mm], Vt[:mm].T, lay, rotate=True)
        err = np.linalg.norm(got - target)
        ok &= abs(err - math.sqrt(np.sum(sv[mm:r] ** 2))) < 1e-9
    # and the rotation term itself is standard RoPE shifted by 700
    ok &= np.allclose(ko.relocate_f64(canon, 700, lay), rope_reference(canon, np.full(T, 700), lay),
                      rtol=0, atol=1e-12)
    return bool(ok)


def pin_scatter_bijection():
    # ID payload rows, delta 0, m 0: every pool slot must hold exactly its id.
    lay = gqa_layout(H=1, D=64, L=2, S=2)
    n, T, P = 3, 40, 16
    ppc = -(-T // P)
    num_pages = 12
    pt = RNG.permutation(num_pages)[: n * ppc].reshape(n, ppc)
    src = []
    for s in range(2):
        x = np.zeros((n, 2, T, 64), np.uint16)
        for c in range(n):
            for l in range(2):
                for t in range(T):
                    # small exact integers as bfloat16: c, l, t, s packed into the row
                    vals = np.array([c, l, t, s] * 16, np.float64)
                    x[c, l, t] = ko.f64_to_bf16_bits(vals)
        src.append(x)
    pools = [np.full((2, num_pages * P, 64), SENTINEL_BITS, np.uint16) for _ in range(2)]
    ko.reconstruct(lay, src, list(range(n)), [0] * n, pools, P, page_table=pt)
    ok = True
    written = np.zeros(num_pages * P, bool)
    for c in range(n):
        for t in range(T):
            slot = pt[c][t // P] * P + (t % P)      # brute force from the definition
            written[slot] = True
            for s in range(2):
                for l in range(2):
                    ok &= np.array_equal(ko.bf16_bits_to_f64(pools[s][l, slot][:4]), [c, l, t, s])
    for s in range(2):
        ok &= bool(np.all(pools[s][:, ~written] == SENTINEL_BITS))
    return bool(ok)


def pin_window_ops_positions():
    # reorder / recall: after the call, token t of output k sits at absolute
    # position base + k*T + t (reorder) or q_i + t (recall) — checked against
    # standard RoPE at those positions, from raw keys, by brute force.
    lay = gqa_layout(H=2, D=64)
    T, ns = 5, 4
    raw = RNG.normal(0, 1, (ns, T, lay.row_width))
    canon_pos = [0, 37, 1000, 5]
    canon = [rope_reference(raw[c], canon_pos[c] + np.arange(T), lay) for c in range(ns)]
    ok = True
    for perm in [(2, 0, 3, 1), (0, 1, 2, 3), (3, 2, 1, 0)]:
        base = 250
        ds = ko.deltas_reorder(perm, base, T, canon_pos)
        for k, c in enumerate(perm):
            got = ko.relocate_f64(canon[c], ds[k], lay)
            want = rope_reference(raw[c], base + k * T + np.arange(T), lay)
            ok &= np.max(np.abs(got - want)) < 1e-10
    ids, q = [3, 1], [90, -12]
    ds = ko.deltas_recall(ids, q, canon_pos)
    for i, c in enumerate(ids):
        got = ko.relocate_f64(canon[c], ds[i], lay)
        ok &= np.max(np.abs(got - rope_reference(raw[c], q[i] + np.arange(T), lay))) < 1e-10
    # identity placement gives delta 0
    ok &= ko.deltas_reorder([0, 1, 2], 0, T, [0, T, 2 * T]) == [0, 0, 0]
    ok &= ko.deltas_recall([2], [canon_pos[2]], canon_pos) == [0]
    return bool(ok)


def pin_scalar_agrees():
    w = TINY
    inp = make_inputs(w, "cpu")
    lay = ko.Layout(w.num_layers, w.num_heads, w.head_dim, w.rope_offset, w.rope_dim,
                    w.rope_base, w.num_streams, w.rope_style)
    d = int(inp["delta"][0])
    ok = True
    for s in range(w.num_streams):
        x = bits(inp["src"][s][0, 0])[:24]
        u = bits(inp["u"][s][0, 0])[:24]
        v = bits(inp["v"][s][0, 0])
        got = ko.reuse_block_bits(x, d, u, v, lay, rotate=(s == 0))
        want = so.reuse_block(x.tolist(), d, u.tolist(), v.tolist(), w.num_heads, w.head_dim,
                              w.rope_offset, w.rope_dim, w.rope_base, rotate=(s == 0))
        ok &= np.array_equal(got, np.array(want, np.uint16))
    return bool(ok)


# ---------------------------------------------------------------------------
# Tests
# ---------------------------------------------------------------------------

def test_rounding_golden(golden_dir):
    assert pin_rounding_golden(golden_dir)


def test_rounding_vs_torch():
    assert pin_rounding_vs_torch()


def test_scalar_rounding_golden(golden_dir):
    for line in open(os.path.join(golden_dir, "bf16_rne_cases.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            hx, want = line.split()[:2]
            assert so.round_to_bf16(float.fromhex(hx)) == int(want, 16), line


def test_theta_closed_forms():
    assert pin_theta_closed_forms()


def test_relocate_identity():
    lay = gqa_layout(H=2, D=64)
    x = RNG.normal(0, 1, (9, 128))
    assert np.array_equal(ko.relocate_f64(x, 0, lay), x)
    xb = bf16_rand((9, 128))
    for rot in (True, False):
        assert np.array_equal(ko.reuse_block_bits(xb, 0, None, None, lay, rot), xb)


@pytest.mark.parametrize("style", [ko.ROPE_HALF, ko.ROPE_INTERLEAVED])
def test_group_law(style):
    lay = gqa_layout(H=2, D=64, base=1e6, style=style)
    x = RNG.normal(0, 1, (11, 128))
    for d1, d2 in [(300, 4000), (-32768, 32768), (17, -9000)]:
        a = ko.relocate_f64(ko.relocate_f64(x, d1, lay), d2, lay)
        b = ko.relocate_f64(x, d1 + d2, lay)
        assert np.max(np.abs(a - b)) <= 1e-12 * np.max(np.abs(b))
    back = ko.relocate_f64(ko.relocate_f64(x, 12345, lay), -12345, lay)
    assert np.max(np.abs(back - x)) <= 1e-12


@pytest.mark.parametrize("style", [ko.ROPE_HALF, ko.ROPE_INTERLEAVED])
def test_rope_equivalence(style):
    assert pin_rope_equivalence(style)


def test_partial_span_and_mla_row():
    # MLA row: 512 c_KV elements untouched by R, 64 k_rope elements rotated.
    lay = ko.Layout(1, 1, 576, 512, 64, 1e4, 1)
    x = RNG.normal(0, 1, (6, 576))
    y = ko.relocate_f64(x, 4321, lay)
    assert np.array_equal(y[:, :512], x[:, :512])
    sub = ko.Layout(1, 1, 64, 0, 64, 1e4, 1)
    assert np.allclose(y[:, 512:], ko.relocate_f64(x[:, 512:], 4321, sub), rtol=0, atol=0)
    want = rope_reference(x, np.full(6, 4321), lay)
    assert np.max(np.abs(y - want)) < 1e-12
    xb = bf16_rand((6, 576))
    out = ko.reuse_block_bits(xb, 4321, None, None, lay, rotate=True)
    assert np.array_equal(out[:, :512], xb[:, :512])          # c_KV byte for byte at m = 0


def test_norm_preservation():
    lay = gqa_layout(H=4, D=128, base=1e6)
    x = RNG.normal(0, 1, (7, 512))
    y = ko.relocate_f64(x, -4097, lay)
    ia, ib, _ = ko.rope_pairs(lay)
    assert np.allclose(x[:, ia] ** 2 + x[:, ib] ** 2, y[:, ia] ** 2 + y[:, ib] ** 2, rtol=1e-12)


def test_unit_vectors():
    assert pin_unit_vectors()


def test_m0_is_pure_relocation():
    lay = gqa_layout(H=2, D=64)
    xb = bf16_rand((20, 128))
    a = ko.reuse_block_bits(xb, 555, None, None, lay, rotate=True)
    b = ko.f64_to_bf16_bits(ko.relocate_f64(ko.bf16_bits_to_f64(xb), 555, lay))
    assert np.array_equal(a, b)
    # the value stream is a byte copy
    assert np.array_equal(ko.reuse_block_bits(xb, 555, None, None, lay, rotate=False), xb)
    # an empty (m = 0) factor pair is the same as no patch
    e_u, e_v = np.zeros((20, 0), np.uint16), np.zeros((128, 0), np.uint16)
    assert np.array_equal(ko.reuse_block_bits(xb, 555, e_u, e_v, lay, rotate=True), a)


def test_patch_alone():
    assert pin_patch_alone()


def test_lowrank_reconstruction():
    assert pin_lowrank_reconstruction()


def test_scatter_bijection():
    assert pin_scatter_bijection()


def test_window_ops_positions():
    assert pin_window_ops_positions()


def test_patch_bytes_match_pages(golden_dir):
    for line in open(os.path.join(golden_dir, "patch_bytes_pages.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            m, frac, tol = line.split()
            assert abs(ko.patch_bytes_fraction(int(m), 512, 512) - float(frac)) <= float(tol)


def test_scalar_oracle_agrees_tiny_config():
    assert pin_scalar_agrees()


def test_scalar_oracle_agrees_interleaved_partial():
    lay = ko.Layout(1, 2, 96, 32, 64, 5e5, 2, ko.ROPE_INTERLEAVED)
    x, u, v = bf16_rand((9, 192)), bf16_rand((9, 16), 0.3), bf16_rand((192, 16), 0.3)
    for rot in (True, False):
        got = ko.reuse_block_bits(x, -777, u, v, lay, rot)
        want = so.reuse_block(x.tolist(), -777, u.tolist(), v.tolist(), 2, 96, 32, 64, 5e5,
                              rotate=rot, interleaved=True)
        assert np.array_equal(got, np.array(want, np.uint16))


def test_reconstruct_tiny_config_end_to_end():
    # The tiny MHA workload through the whole call: rows land where the
    # contiguous destination says and nowhere else.
    w = TINY
    inp = make_inputs(w, "cpu")
    lay = ko.Layout(w.num_layers, w.num_heads, w.head_dim, w.rope_offset, w.rope_dim,
                    w.rope_base, w.num_streams)
    src = [bits(t) for t in inp["src"]]
    pools = [bits(p).copy() for p in inp["pool"]]
    u = [bits(t) for t in inp["u"]]
    v = [bits(t) for t in inp["v"]]
    off = inp["dst_offset"].numpy()
    ko.reconstruct(lay, src, [0], ko.deltas_relocate(inp["delta"].tolist()), pools, 0,
                   dst_offset=off, u=u, v=v)
    for s in range(2):
        blk = ko.reuse_block_bits(src[s][0, 0], 300, u[s][0, 0], v[s][0, 0], lay, rotate=(s == 0))
        assert np.array_equal(pools[s][0, off[0]: off[0] + w.n_tokens], blk)
        mask = np.ones(pools[s].shape[1], bool)
        mask[off[0]: off[0] + w.n_tokens] = False
        assert np.all(pools[s][0, mask] == SENTINEL_BITS)


# ---------------------------------------------------------------------------
# Planted mistakes: each must make at least one pin fail
# ---------------------------------------------------------------------------

def _safe(fn, *a):
    try:
        return bool(fn(*a))
    except Exception:
        return False


def _all_pins(golden_dir):
    return {k: _safe(f, *a) for k, (f, a) in {
        "rounding_golden": (pin_rounding_golden, (golden_dir,)),
        "rounding_torch": (pin_rounding_vs_torch, ()),
        "theta": (pin_theta_closed_forms, ()),
        "rope_half": (pin_rope_equivalence, (ko.ROPE_HALF,)),
        "rope_inter": (pin_rope_equivalence, (ko.ROPE_INTERLEAVED,)),
        "unit": (pin_unit_vectors, ()),
        "patch": (pin_patch_alone, ()),
        "lowrank": (pin_lowrank_reconstruction, ()),
        "scatter": (pin_scatter_bijection, ()),
        "window": (pin_window_ops_positions, ()),
    }.items()}


def _mut_sign(x, delta, layout):
    y = np.array(x, dtype=np.float64, copy=True)
    ia, ib, j = ko.rope_pairs(layout)
    phi = delta * ko.rope_inv_freq(layout.rope_dim, layout.rope_base)[j]
    y[..., ia] = x[..., ia] * np.cos(phi) + x[..., ib] * np.sin(phi)
    y[..., ib] = x[..., ib] * np.cos(phi) - x[..., ia] * np.sin(phi)
    return y


def _mut_theta(rope_dim, base):
    j = np.arange(rope_dim // 2, dtype=np.float64)
    return np.power(np.float64(base), -1.0 * j / rope_dim)


def _mut_pairs(layout):
    ia, ib, jj = _orig_pairs(layout)
    return ia, ib, jj[::-1].copy()


def _mut_round_trunc(x):
    x = np.asarray(x, np.float64).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def _mut_round_via_f32(x):
    return bits(torch.from_numpy(np.asarray(x, np.float64).astype(np.float32)).to(torch.bfloat16))


def _mut_patch_rows_reversed(u, v):
    u, v = np.asarray(u, np.float64), np.asarray(v, np.float64)
    return u @ v[::-1].T


def _mut_patch_transposed(u, v):
    u, v = np.asarray(u, np.float64), np.asarray(v, np.float64)
    return (v @ u.T).T[:, ::-1] if v.shape[0] != u.shape[0] else (v @ u.T)


def _mut_patch_dropped(u, v):
    return np.zeros((np.asarray(u).shape[0], np.asarray(v).shape[0]))


def _mut_slots(i, n_tokens, page_size, page_table=None, dst_offset=None):
    t = np.arange(n_tokens, dtype=np.int64)
    if page_size > 0:
        pages = np.asarray(page_table, dtype=np.int64)[i]
        return pages[t // page_size] * page_size + (t + 1) % page_size
    return np.int64(dst_offset[i]) + t


def _mut_reorder(perm, base_pos, n_tokens, canon_pos=None):
    return [int(base_pos) + k * int(n_tokens) + (0 if canon_pos is None else int(canon_pos[int(c)]))
            for k, c in enumerate(perm)]


_orig_pairs = ko.rope_pairs


@pytest.mark.parametrize("name,attr,mutant", [
    ("rotation sign", "relocate_f64", _mut_sign),
    ("frequency exponent", "rope_inv_freq", _mut_theta),
    ("pair frequency index", "rope_pairs", _mut_pairs),
    ("truncating rounding", "f64_to_bf16_bits", _mut_round_trunc),
    ("double rounding via binary32", "f64_to_bf16_bits", _mut_round_via_f32),
    ("patch factor rows permuted", "patch_f64", _mut_patch_rows_reversed),
    ("patch operands transposed", "patch_f64", _mut_patch_transposed),
    ("patch dropped", "patch_f64", _mut_patch_dropped),
    ("page slot index", "dest_slots", _mut_slots),
    ("reorder delta sign of p_c", "deltas_reorder", _mut_reorder),
])
def test_planted_mistakes(monkeypatch, golden_dir, name, attr, mutant):
    assert all(_all_pins(golden_dir).values())
    monkeypatch.setattr(ko, attr, mutant)
    res = _all_pins(golden_dir)
    assert not all(res.values()), f"no pin caught the planted mistake: {name}"
