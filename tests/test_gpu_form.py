"""GPU parity of patch formation (kamera_form_patch) against the CPU oracle.

Inputs: canonical rows from the seeded generators; the forward-pass output
KV(B|A) is built here with the reuse oracle from factors of a chosen spectrum,
target = bf16(R(delta) canon + P diag(sigma) Q^T), so that the deficit the
oracle and the GPU both see (including the bfloat16 rounding of the target)
has a clear gap at m.  The oracle's factors are the exact truncated SVD of
that same deficit.

Bar: the product U V^T of the bfloat16 factors within
4e-3 (Frobenius, relative) of the oracle's float64 product, which is what
rounding both factors to bfloat16 costs; well-separated columns within 8e-3
(relative, per column) with the same sign; zero deficits give zero factors
bit for bit.
"""

import numpy as np
import pytest
import torch

import position_invariant_kv_amd as kam
from oracle import kamera_oracle as ko
from oracle import patch_oracle as po
from workloads import bits, make_inputs, small_workload

pytestmark = pytest.mark.gpu

PROD_TOL = 4e-3
COL_TOL = 8e-3


def _say(msg):
    print(f"[gpu-form] {msg}", flush=True)


def build_case(w, m, sig, seed):
    """Canonical rows (generator), the target built by the reuse oracle, and omega."""
    inp = make_inputs(w, "cuda", seed=seed)
    o_lay = ko.Layout(w.num_layers, w.num_heads, w.head_dim, w.rope_offset, w.rope_dim, w.rope_base,
                      w.num_streams, w.rope_style)
    g_lay = kam.Layout(w.num_layers, w.num_heads, w.head_dim, w.rope_offset, w.rope_dim, w.rope_base,
                       w.num_streams, w.rope_style)
    n, L, T, F, S = w.n_chunks, w.num_layers, w.n_tokens, w.row_width, w.num_streams
    rng = np.random.default_rng(seed)
    deltas = inp["delta"].cpu().tolist()
    canon_b = [bits(inp["src"][s][:n]) for s in range(S)]
    target_b = [np.empty_like(canon_b[s]) for s in range(S)]
    r = len(sig)
    for s in range(S):
        for i in range(n):
            for l in range(L):
                P, _ = np.linalg.qr(rng.standard_normal((T, r)))
                Q, _ = np.linalg.qr(rng.standard_normal((F, r)))
                y = ko.reuse_f64(ko.bf16_bits_to_f64(canon_b[s][i, l]), deltas[i], P * sig, Q, o_lay, rotate=(s == 0))
                target_b[s][i, l] = ko.f64_to_bf16_bits(y)
    canon = [torch.from_numpy(c.view(np.int16)).cuda().view(torch.bfloat16) for c in canon_b]
    target = [torch.from_numpy(t.view(np.int16)).cuda().view(torch.bfloat16) for t in target_b]
    return inp, o_lay, g_lay, canon, target, canon_b, target_b, deltas


def run_form(g_lay, canon, target, delta, n, L, T, F, S, m, p, q, seed):
    k = m + p
    gen = torch.Generator(device="cuda").manual_seed(seed)
    omega = torch.randn((k, F), generator=gen, device="cuda").to(torch.bfloat16)
    u = [torch.zeros((n, L, T, m), dtype=torch.bfloat16, device="cuda") for _ in range(S)]
    v = [torch.zeros((n, L, F, m), dtype=torch.bfloat16, device="cuda") for _ in range(S)]
    kam.form_patch(g_lay, canon, target, delta, u, v, omega, oversample=p, power_iters=q)
    torch.cuda.synchronize()
    return [bits(t) for t in u], [bits(t) for t in v]


def check_block(ub, vb, canon_b, target_b, delta, o_lay, rotate, m, where, col_check=4):
    _, _, U, V, sig = po.form_patch_bits(canon_b, target_b, delta, o_lay, rotate, m)
    return check_factors(ub, vb, U, V, sig, m, where, col_check)


def check_factors(ub, vb, U, V, sig, m, where, col_check=4):
    """The GPU's bfloat16 factors (ub, vb) against the oracle's (U, V, sigma)."""
    Ug, Vg = ko.bf16_bits_to_f64(ub), ko.bf16_bits_to_f64(vb)
    want = U @ V.T
    got = Ug @ Vg.T
    den = np.linalg.norm(want)
    rel = np.linalg.norm(got - want) / den if den > 0 else np.linalg.norm(got)
    assert rel <= PROD_TOL, f"{where}: product off by {rel:.2e} (relative Frobenius)"
    # well-separated leading columns: same vector, same sign
    for i in range(min(col_check, m, sig.size)):
        if sig[i] <= po.NEGLIGIBLE * sig[0]:
            continue
        gap = min(abs(sig[i] - sig[i - 1]) if i > 0 else np.inf, abs(sig[i] - sig[i + 1]) if i + 1 < sig.size else np.inf)
        if gap < 0.15 * sig[i]:
            continue
        for name, a, b in (("U", Ug[:, i], U[:, i]), ("V", Vg[:, i], V[:, i])):
            e = np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)
            assert e <= COL_TOL, f"{where}: column {i} of {name} off by {e:.2e}"
    return rel


SMALL = {
    # name: (workload keywords, m, p, q, spectrum)
    "gqa_m8": (dict(n_tokens=80, n_chunks=2), 8, 8, 1, 10.0 * 0.7 ** np.arange(8)),
    "gqa_d128_m16": (dict(num_heads=2, head_dim=128, rope_dim=128, rope_base=1e6, n_tokens=130, n_chunks=1,
                          delta_range=(-4096, 8192)), 16, 16, 2, 20.0 * 0.85 ** np.arange(16)),
    "gqa_m32_kp64": (dict(num_heads=2, head_dim=128, rope_dim=128, n_tokens=200, n_chunks=1), 32, 16, 2,
                     30.0 * 0.9 ** np.arange(32)),
    "interleaved_partial": (dict(rope_style=1, head_dim=128, rope_offset=64, rope_dim=64, n_tokens=70,
                                 n_chunks=2), 8, 8, 1, 10.0 * 0.7 ** np.arange(8)),
    "mla_row_m16": (dict(family="MLA", num_heads=1, head_dim=576, rope_offset=512, rope_dim=64, num_streams=1,
                         n_tokens=130, n_chunks=2, delta_range=(-32768, 32768)), 16, 16, 2,
                    20.0 * 0.85 ** np.arange(16)),
    "rank2_single_token_rows": (dict(n_tokens=1, n_chunks=3), 2, 0, 1, np.array([3.0])),
    "m4_long": (dict(n_tokens=1000, n_chunks=1, num_layers=1), 4, 12, 1, 10.0 * 0.6 ** np.arange(4)),
    # one 64-feature panel (F = 64): a feature tile's second panel does not exist
    "single_panel_f64": (dict(num_heads=1, n_tokens=90, n_chunks=2), 8, 8, 1, 10.0 * 0.7 ** np.arange(8)),
    # an odd sketch width (k = 33 of 64 columns): the small dense steps run on
    # 34, one of them a zero column
    "odd_k33": (dict(n_tokens=80, n_chunks=2), 8, 25, 1, 10.0 * 0.7 ** np.arange(8)),
}


@pytest.mark.parametrize("name", sorted(SMALL))
def test_form_patch_small(name):
    kw, m, p, q, sig = SMALL[name]
    w = small_workload(name=name, op="relocate_patch", rank=m, **kw)
    _say(f"{name}: {w} m={m} p={p} q={q}")
    seed = 1000 + len(name)
    inp, o_lay, g_lay, canon, target, canon_b, target_b, deltas = build_case(w, m, sig, seed)
    n, L, T, F, S = w.n_chunks, w.num_layers, w.n_tokens, w.row_width, w.num_streams
    ub, vb = run_form(g_lay, canon, target, inp["delta"][:n].contiguous(), n, L, T, F, S, m, p, q, seed)
    worst = 0.0
    for s in range(S):
        for i in range(n):
            for l in range(L):
                worst = max(worst, check_block(ub[s][i, l], vb[s][i, l], canon_b[s][i, l], target_b[s][i, l],
                                               deltas[i], o_lay, s == 0, m, f"{name} (i={i}, l={l}, s={s})"))
    _say(f"{name}: worst product error {worst:.2e}")


def test_form_patch_ignores_workspace_contents():
    # a workspace full of NaN bit patterns, the same workspace again with the
    # first call's leftovers, and a zeroed one give the same factors bit for
    # bit (at most two row tiles per product, so the Gram sums do not depend on
    # the order of their atomic adds), within the oracle's bar
    m, p, q = 16, 16, 2
    sig = 20.0 * 0.85 ** np.arange(m)
    w = small_workload(name="workspace_contents", op="relocate_patch", rank=m, n_tokens=200, n_chunks=2)
    inp, o_lay, g_lay, canon, target, canon_b, target_b, deltas = build_case(w, m, sig, 91)
    n, L, T, F, S = w.n_chunks, w.num_layers, w.n_tokens, w.row_width, w.num_streams
    delta = inp["delta"][:n].contiguous()
    gen = torch.Generator(device="cuda").manual_seed(91)
    omega = torch.randn((m + p, F), generator=gen, device="cuda").to(torch.bfloat16)
    need = kam.form_patch_workspace_bytes(g_lay, n, T, m, p)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    runs = []
    for wspace in (ws, ws, torch.zeros(need, dtype=torch.uint8, device="cuda")):
        u = [torch.zeros((n, L, T, m), dtype=torch.bfloat16, device="cuda") for _ in range(S)]
        v = [torch.zeros((n, L, F, m), dtype=torch.bfloat16, device="cuda") for _ in range(S)]
        kam.form_patch(g_lay, canon, target, delta, u, v, omega, oversample=p, power_iters=q, workspace=wspace)
        torch.cuda.synchronize()
        runs.append(([bits(t) for t in u], [bits(t) for t in v]))
    for r in runs[1:]:
        for s in range(S):
            assert np.array_equal(r[0][s], runs[0][0][s]) and np.array_equal(r[1][s], runs[0][1][s])
    for s in range(S):
        for i in range(n):
            for l in range(L):
                check_block(runs[0][0][s][i, l], runs[0][1][s][i, l], canon_b[s][i, l], target_b[s][i, l],
                            deltas[i], o_lay, s == 0, m, f"workspace_contents (i={i}, l={l}, s={s})")


def test_form_patch_exact_low_rank_without_power_iterations():
    # canonical rows 0 and a target that is an exact rank-4 product of small
    # integer matrices (every entry exact in bfloat16): Delta has rank 4 <= k,
    # so one sketch (q = 0) captures its range and the factors are the exact
    # truncated SVD up to fp32 rounding (then bfloat16 rounding of the factors)
    w = small_workload(op="relocate_patch", rank=4, n_tokens=96, n_chunks=2, num_layers=1)
    inp = make_inputs(w, "cuda", seed=9)
    o_lay = ko.Layout(w.num_layers, w.num_heads, w.head_dim, w.rope_offset, w.rope_dim, w.rope_base,
                      w.num_streams, w.rope_style)
    g_lay = kam.Layout(w.num_layers, w.num_heads, w.head_dim, w.rope_offset, w.rope_dim, w.rope_base,
                       w.num_streams, w.rope_style)
    n, L, T, F = w.n_chunks, w.num_layers, w.n_tokens, w.row_width
    rng = np.random.default_rng(9)
    canon_b = [np.zeros((n, L, T, F), np.uint16) for _ in range(2)]
    target_b = []
    for s in range(2):
        P = rng.integers(-3, 4, size=(n, L, T, 4)).astype(np.float64)
        Q = rng.integers(-3, 4, size=(n, L, F, 4)).astype(np.float64)
        target_b.append(ko.f64_to_bf16_bits(np.einsum("nltr,nlfr->nltf", P, Q)))
    to_dev = lambda b: torch.from_numpy(b.view(np.int16)).cuda().view(torch.bfloat16)
    canon = [to_dev(c) for c in canon_b]
    target = [to_dev(t) for t in target_b]
    ub, vb = run_form(g_lay, canon, target, inp["delta"][:n].contiguous(), n, L, T, F, 2, 4, 12, 0, 9)
    deltas = inp["delta"][:n].cpu().tolist()
    for s in range(2):
        for i in range(n):
            check_block(ub[s][i, 0], vb[s][i, 0], canon_b[s][i, 0], target_b[s][i, 0], deltas[i], o_lay, s == 0,
                        4, f"exact rank 4 (i={i}, s={s})")


def test_form_patch_zero_deficit_gives_zero_factors():
    # delta = 0 and target = canon: Delta is exactly zero, so are the factors
    w = small_workload(op="relocate_patch", rank=8, n_tokens=70, delta_fixed=0)
    inp = make_inputs(w, "cuda", seed=5)
    g_lay = kam.Layout(w.num_layers, w.num_heads, w.head_dim, w.rope_offset, w.rope_dim, w.rope_base,
                       w.num_streams, w.rope_style)
    n = w.n_chunks
    canon = [t[:n].contiguous() for t in inp["src"]]
    ub, vb = run_form(g_lay, canon, [c.clone() for c in canon], inp["delta"][:n].contiguous(), n, w.num_layers,
                      w.n_tokens, w.row_width, 2, 8, 8, 1, 5)
    for s in range(2):
        assert not ub[s].any() and not vb[s].any()


def test_form_then_reuse_restores_target():
    # the formed factors fed to kamera_relocate_patch reproduce KV(B|A) up to
    # the truncation: with rank(signal) = m, within the bfloat16 noise floor
    m, p, q = 16, 16, 2
    sig = 20.0 * 0.85 ** np.arange(m)
    w = small_workload(op="relocate_patch", rank=m, num_heads=2, head_dim=128, rope_dim=128, rope_base=1e6,
                       n_tokens=150, n_chunks=2, delta_range=(-4096, 8192))
    inp, o_lay, g_lay, canon, target, canon_b, target_b, deltas = build_case(w, m, sig, 77)
    n, L, T, F = w.n_chunks, w.num_layers, w.n_tokens, w.row_width
    u = [torch.zeros((n, L, T, m), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    v = [torch.zeros((n, L, F, m), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    gen = torch.Generator(device="cuda").manual_seed(77)
    omega = torch.randn((m + p, F), generator=gen, device="cuda").to(torch.bfloat16)
    delta = inp["delta"][:n].contiguous()
    kam.form_patch(g_lay, canon, target, delta, u, v, omega, oversample=p, power_iters=q)
    pool = [torch.zeros((L, n * T, F), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    off = torch.arange(n, dtype=torch.int64, device="cuda") * T
    kam.relocate_patch(g_lay, canon, delta, u, v, pool, dst_offset=off)
    torch.cuda.synchronize()
    for s in range(2):
        got = ko.bf16_bits_to_f64(bits(pool[s]))
        for i in range(n):
            for l in range(L):
                want = ko.bf16_bits_to_f64(target_b[s][i, l])
                err = np.abs(got[l, i * T:(i + 1) * T] - want)
                # target rounding (half an ulp) + factor rounding + output rounding
                assert float(err.max()) <= 0.05 * float(np.abs(want).max()), (s, i, l, float(err.max()))
                assert float(np.sqrt((err ** 2).mean())) <= 6e-3 * float(np.sqrt((want ** 2).mean()))


FULL = ["form_gqa_single_frame", "form_mla"]


@pytest.mark.parametrize("name", FULL)
def test_form_full_size_sampled(name):
    # the benchmark's formation workloads, whole call as bench.py launches it;
    # KV(B|A) built by the reuse oracle from the generator's signal factors;
    # six seeded whole blocks compared with the oracle's truncated SVD
    import random
    import time

    from workloads import form_by_name, make_form_inputs

    fw = form_by_name(name)
    b = fw.base
    n, L, T, F, S = b.n_chunks, b.num_layers, b.n_tokens, b.row_width, b.num_streams
    _say(f"full size {name}: {fw.blocks} blocks of {T} x {F}, m={fw.rank} p={fw.oversample} q={fw.power_iters}")
    inp = make_form_inputs(fw, "cuda")
    o_lay = ko.Layout(b.num_layers, b.num_heads, b.head_dim, b.rope_offset, b.rope_dim, b.rope_base, S,
                      b.rope_style)
    g_lay = kam.Layout(b.num_layers, b.num_heads, b.head_dim, b.rope_offset, b.rope_dim, b.rope_base, S,
                       b.rope_style)
    deltas = inp["delta"].cpu().tolist()
    t0 = time.time()
    target = []
    for s in range(S):
        tb = np.empty((n, L, T, F), np.uint16)
        for i in range(n):
            cb = bits(inp["src"][s][i])
            ub = bits(inp["u_sig"][s][i])
            vb = bits(inp["v_sig"][s][i])
            for l in range(L):
                y = ko.reuse_f64(ko.bf16_bits_to_f64(cb[l]), deltas[i], ko.bf16_bits_to_f64(ub[l]),
                                 ko.bf16_bits_to_f64(vb[l]), o_lay, rotate=(s == 0))
                tb[i, l] = ko.f64_to_bf16_bits(y)
            if i % 4 == 3:
                _say(f"{name}: oracle targets, stream {s}, chunk {i + 1}/{n} ({time.time() - t0:.0f} s)")
        target.append(torch.from_numpy(tb.view(np.int16)).cuda().view(torch.bfloat16))
        del tb
    del inp["u_sig"], inp["v_sig"]
    u = [torch.zeros((n, L, T, fw.rank), dtype=torch.bfloat16, device="cuda") for _ in range(S)]
    v = [torch.zeros((n, L, F, fw.rank), dtype=torch.bfloat16, device="cuda") for _ in range(S)]
    kam.form_patch(g_lay, inp["src"], target, inp["delta"], u, v, inp["omega"], oversample=fw.oversample,
                   power_iters=fw.power_iters)
    torch.cuda.synchronize()
    rng = random.Random(11)
    blocks = {(0, 0, 0), (n - 1, L - 1, S - 1)}
    while len(blocks) < 6:
        blocks.add((rng.randrange(n), rng.randrange(L), rng.randrange(S)))
    for (i, l, s) in sorted(blocks):
        rel = check_block(bits(u[s][i, l]), bits(v[s][i, l]), bits(inp["src"][s][i, l]), bits(target[s][i, l]),
                          deltas[i], o_lay, s == 0, fw.rank, f"{name} (i={i}, l={l}, s={s})")
        _say(f"{name}: block (i={i}, l={l}, s={s}) product error {rel:.2e}")
    del inp, target, u, v
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# orbit patches (kamera_form_orbit_patch): the mean deficit over orderings

def orbit_deltas(n, orders, T, base_pos):
    """[n, views] shifts: chunk i at slot orders[v].index(i) of ordering v, frames at 0."""
    d = np.empty((n, len(orders)), np.int64)
    for v, order in enumerate(orders):
        for slot, i in enumerate(order):
            d[i, v] = base_pos + slot * T
    return d


def build_orbit_case(w, orders, sig, unique, seed):
    """Canonical rows and, for every view v, KV_v(B|A_v) = bf16(R(delta_v) canon
    + P diag(sig) Q^T + unique * p_v q_v^T): a deficit shared by every ordering
    plus a rank-1 part of its own, so the mean has rank len(sig) + views."""
    inp = make_inputs(w, "cuda", seed=seed)
    o_lay = ko.Layout(w.num_layers, w.num_heads, w.head_dim, w.rope_offset, w.rope_dim, w.rope_base,
                      w.num_streams, w.rope_style)
    g_lay = kam.Layout(w.num_layers, w.num_heads, w.head_dim, w.rope_offset, w.rope_dim, w.rope_base,
                       w.num_streams, w.rope_style)
    n, L, T, F, S = w.n_chunks, w.num_layers, w.n_tokens, w.row_width, w.num_streams
    P = len(orders)
    deltas = orbit_deltas(n, orders, T, 96)
    rng = np.random.default_rng(seed)
    canon_b = [bits(inp["src"][s][:n]) for s in range(S)]
    target_b = [np.empty((n * P, L, T, F), np.uint16) for _ in range(S)]
    r = len(sig)
    for s in range(S):
        for i in range(n):
            for l in range(L):
                Pc, _ = np.linalg.qr(rng.standard_normal((T, r)))
                Qc, _ = np.linalg.qr(rng.standard_normal((F, r)))
                c = ko.bf16_bits_to_f64(canon_b[s][i, l])
                for v in range(P):
                    pv = rng.standard_normal((T, 1))
                    qv = rng.standard_normal((F, 1))
                    U = np.hstack([Pc * sig, unique * pv / np.linalg.norm(pv)])
                    V = np.hstack([Qc, qv / np.linalg.norm(qv)])
                    y = ko.reuse_f64(c, int(deltas[i, v]), U, V, o_lay, rotate=(s == 0))
                    target_b[s][i * P + v, l] = ko.f64_to_bf16_bits(y)
    to_dev = lambda b: torch.from_numpy(b.view(np.int16)).cuda().view(torch.bfloat16)
    return (o_lay, g_lay, [to_dev(c) for c in canon_b], [to_dev(t) for t in target_b], canon_b, target_b,
            deltas)


def run_orbit(g_lay, canon, targets, deltas, n, L, T, F, S, m, p, q, seed):
    gen = torch.Generator(device="cuda").manual_seed(seed)
    omega = torch.randn((m + p, F), generator=gen, device="cuda").to(torch.bfloat16)
    u = [torch.zeros((n, L, T, m), dtype=torch.bfloat16, device="cuda") for _ in range(S)]
    v = [torch.zeros((n, L, F, m), dtype=torch.bfloat16, device="cuda") for _ in range(S)]
    d = torch.from_numpy(np.ascontiguousarray(deltas)).cuda()
    kam.form_orbit_patch(g_lay, canon, targets, d, u, v, omega, oversample=p, power_iters=q)
    torch.cuda.synchronize()
    return [bits(t) for t in u], [bits(t) for t in v]


def check_orbit(ub, vb, canon_b, target_b, deltas, o_lay, S, m, name):
    n, L = canon_b[0].shape[:2]
    P = deltas.shape[1]
    worst = 0.0
    for s in range(S):
        for i in range(n):
            for l in range(L):
                tb = target_b[s][i * P:(i + 1) * P, l]
                _, _, U, V, sig = po.form_orbit_patch_bits(canon_b[s][i, l], tb, [int(x) for x in deltas[i]],
                                                           o_lay, s == 0, m)
                worst = max(worst, check_factors(ub[s][i, l], vb[s][i, l], U, V, sig, m,
                                                 f"{name} (i={i}, l={l}, s={s})"))
    _say(f"{name}: worst product error {worst:.2e}")


@pytest.mark.parametrize("case", ["gqa_m8", "gqa_m32_kp64", "mla_row_m16"])
def test_orbit_one_view_is_the_plain_patch(case):
    # one view, and two identical views, through kamera_form_orbit_patch:
    # bit for bit what kamera_form_patch gives for that view.  A single view
    # forms the deficit inside the first product; two views take the separate
    # deficit pass, so this also pins the two paths to each other (32 and 64
    # sketch columns, GQA and MLA rows)
    kw, m, p, q, sig = SMALL[case]
    w = small_workload(name=f"orbit_one_view_{case}", op="relocate_patch", rank=m, **kw)
    inp, o_lay, g_lay, canon, target, canon_b, target_b, deltas = build_case(w, m, sig, 31)
    n, L, T, F, S = w.n_chunks, w.num_layers, w.n_tokens, w.row_width, w.num_streams
    d1 = inp["delta"][:n].contiguous()
    ub, vb = run_form(g_lay, canon, target, d1, n, L, T, F, S, m, p, q, 31)
    d1_np = d1.cpu().numpy().reshape(n, 1)
    uo, vo = run_orbit(g_lay, canon, target, d1_np, n, L, T, F, S, m, p, q, 31)
    for s in range(S):
        assert np.array_equal(uo[s], ub[s]) and np.array_equal(vo[s], vb[s]), f"one view, stream {s}"
    twice = [t.repeat_interleave(2, dim=0).contiguous() for t in target]
    u2, v2 = run_orbit(g_lay, canon, twice, np.repeat(d1_np, 2, axis=1), n, L, T, F, S, m, p, q, 31)
    for s in range(S):
        assert np.array_equal(u2[s], ub[s]) and np.array_equal(v2[s], vb[s]), f"two equal views, stream {s}"


def test_orbit_patch_all_orders_of_three_chunks():
    # a cached set of three chunks, every one of its 3! orderings a view
    import itertools
    orders = list(itertools.permutations(range(3)))
    sig = 20.0 * 0.8 ** np.arange(8)
    m, p, q = 8 + len(orders), 18, 2
    w = small_workload(name="orbit_all_orders", op="relocate_patch", rank=m, n_tokens=72, n_chunks=3)
    _say(f"orbit over all {len(orders)} orders: {w} m={m}")
    o_lay, g_lay, canon, targets, canon_b, target_b, deltas = build_orbit_case(w, orders, sig, 6.0, 41)
    n, L, T, F, S = w.n_chunks, w.num_layers, w.n_tokens, w.row_width, w.num_streams
    ub, vb = run_orbit(g_lay, canon, targets, deltas, n, L, T, F, S, m, p, q, 41)
    check_orbit(ub, vb, canon_b, target_b, deltas, o_lay, S, m, "all orders of 3")


def test_orbit_patch_mla_four_sampled_orders():
    # MLA rows (c_KV copied, k_rope rotated), four chunks, four sampled orderings
    rng = np.random.default_rng(5)
    orders = [list(range(4))] + [list(rng.permutation(4)) for _ in range(3)]
    sig = 20.0 * 0.85 ** np.arange(8)
    m, p, q = 12, 20, 2
    w = small_workload(name="orbit_mla", op="relocate_patch", rank=m, family="MLA", num_heads=1, head_dim=576,
                       rope_offset=512, rope_dim=64, num_streams=1, n_tokens=130, n_chunks=4)
    _say(f"orbit MLA, 4 sampled orders: {w} m={m}")
    o_lay, g_lay, canon, targets, canon_b, target_b, deltas = build_orbit_case(w, orders, sig, 4.0, 43)
    n, L, T, F, S = w.n_chunks, w.num_layers, w.n_tokens, w.row_width, w.num_streams
    ub, vb = run_orbit(g_lay, canon, targets, deltas, n, L, T, F, S, m, p, q, 43)
    check_orbit(ub, vb, canon_b, target_b, deltas, o_lay, S, m, "MLA, 4 orders")


def test_form_orbit_full_size_sampled():
    # the orbit benchmark workload's shapes and call; blocks are independent,
    # so only the sampled blocks get targets built by the reuse oracle (every
    # view), the rest hold the canonical rows (copied with torch)
    import random

    from workloads import form_by_name, make_form_inputs

    fw = form_by_name("form_orbit_reorder")
    b = fw.base
    n, L, T, F, S, P = b.n_chunks, b.num_layers, b.n_tokens, b.row_width, b.num_streams, fw.views
    _say(f"full size orbit: {fw.blocks} blocks of {T} x {F}, {P} views, m={fw.rank}")
    inp = make_form_inputs(fw, "cuda")
    o_lay = ko.Layout(b.num_layers, b.num_heads, b.head_dim, b.rope_offset, b.rope_dim, b.rope_base, S,
                      b.rope_style)
    g_lay = kam.Layout(b.num_layers, b.num_heads, b.head_dim, b.rope_offset, b.rope_dim, b.rope_base, S,
                       b.rope_style)
    deltas = inp["delta"].cpu().numpy()
    rng = random.Random(17)
    blocks = {(0, 0, 0), (n - 1, L - 1, S - 1)}
    while len(blocks) < 4:
        blocks.add((rng.randrange(n), rng.randrange(L), rng.randrange(S)))
    targets = [inp["src"][s].repeat_interleave(P, dim=0).contiguous() for s in range(S)]
    want_t = {}
    for (i, l, s) in sorted(blocks):
        cb = bits(inp["src"][s][i, l])
        vb = ko.bf16_bits_to_f64(bits(inp["v_sig"][s][i, l]))
        tb = np.empty((P, T, F), np.uint16)
        for v in range(P):
            ub_ = ko.bf16_bits_to_f64(bits(inp["u_sig"][s][i * P + v, l]))
            tb[v] = ko.f64_to_bf16_bits(ko.reuse_f64(ko.bf16_bits_to_f64(cb), int(deltas[i, v]), ub_, vb, o_lay,
                                                     rotate=(s == 0)))
            targets[s][i * P + v, l] = torch.from_numpy(tb[v].view(np.int16)).cuda().view(torch.bfloat16)
        want_t[(i, l, s)] = (cb, tb)
    del inp["u_sig"], inp["v_sig"]
    u = [torch.zeros((n, L, T, fw.rank), dtype=torch.bfloat16, device="cuda") for _ in range(S)]
    v = [torch.zeros((n, L, F, fw.rank), dtype=torch.bfloat16, device="cuda") for _ in range(S)]
    kam.form_orbit_patch(g_lay, inp["src"], targets, inp["delta"], u, v, inp["omega"], oversample=fw.oversample,
                         power_iters=fw.power_iters)
    torch.cuda.synchronize()
    for (i, l, s), (cb, tb) in sorted(want_t.items()):
        _, _, U, V, sig = po.form_orbit_patch_bits(cb, tb, [int(x) for x in deltas[i]], o_lay, s == 0, fw.rank)
        rel = check_factors(bits(u[s][i, l]), bits(v[s][i, l]), U, V, sig, fw.rank,
                            f"orbit (i={i}, l={l}, s={s})")
        _say(f"orbit: block (i={i}, l={l}, s={s}) product error {rel:.2e}")
    del inp, targets, u, v
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
