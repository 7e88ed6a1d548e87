"""Pins of the decode-attention oracle (oracle/attention_oracle.py) on the CPU.

Every pin compares the oracle with something other than itself:
* a brute force in plain Python loops (complex-exponential RoPE via cmath,
  the patch as explicit sums, softmax via math.exp) on tiny contexts, for
  GQA with rotate-half pairs, a partial interleaved span, and MLA rows;
* closed forms: identical keys give the mean of the values and
  lse = log N + s; values constant per KV head give that constant, which
  fixes the query-head -> KV-head map; an empty context gives 0 and -inf;
* RoPE's relative-position property: moving the chunk by delta + x and the
  query by x leaves the output unchanged (this fixes the direction of the
  relocation against the rotation the query carries);
* the log-sum-exp merge of the per-chunk results equals the result over
  the concatenated context;
* pooled tokens (a sequence's own tokens in a paged pool): a brute force that
  walks the block table page by page in Python loops; pooled tokens equal a
  reused entry of the same rows at shift 0 with no patch; a context split
  between entries and pooled tokens equals the log-sum-exp merge of the two
  parts.
``test_planted_mistakes`` breaks the oracle on purpose and checks that a pin
catches each mistake.
"""

import cmath
import math

import numpy as np
import pytest

from oracle import attention_oracle as ao
from oracle import kamera_oracle as ko


def _bits(x):
    return ko.f64_to_bf16_bits(np.asarray(x, np.float64))


def _store(rng, S, n, L, T, F, scale=1.0):
    return [_bits(scale * rng.standard_normal((n, L, T, F))) for _ in range(S)]


def _brute(layout, layer, canon, patch, seq_entries, ids, deltas, q, Hq, scale):
    """Decode attention by explicit loops: RoPE as (a + ib) e^(i delta theta_j)."""
    D, H, R, o = layout.head_dim, layout.num_heads, layout.rope_dim, layout.rope_offset
    S = layout.num_streams
    F = H * D
    Dv = D if S == 2 else o
    f = ko.bf16_bits_to_f64
    B = len(seq_entries) - 1
    out = [[[0.0] * Dv for _ in range(Hq)] for _ in range(B)]
    lse = [[-math.inf] * Hq for _ in range(B)]
    for b in range(B):
        keys, vals = [], []
        for e in range(seq_entries[b], seq_entries[b + 1]):
            cid, dl = ids[e], deltas[e]
            T = canon[0].shape[2]
            for t in range(T):
                rows = []
                for s in range(S):
                    x = [float(v) for v in f(canon[s][cid, layer, t])]
                    y = list(x)
                    if s == 0:
                        for h in range(H):
                            for j in range(R // 2):
                                if layout.rope_style == ko.ROPE_HALF:
                                    ia, ib = h * D + o + j, h * D + o + j + R // 2
                                else:
                                    ia, ib = h * D + o + 2 * j, h * D + o + 2 * j + 1
                                z = complex(x[ia], x[ib]) * cmath.exp(1j * dl * math.pow(layout.rope_base, -2.0 * j / R))
                                y[ia], y[ib] = z.real, z.imag
                    if patch is not None:
                        u = f(patch[0][s][cid, layer, t])
                        v = f(patch[1][s][cid, layer])
                        for c in range(F):
                            y[c] += sum(float(u[k]) * float(v[c, k]) for k in range(u.size))
                    rows.append(y)
                keys.append(rows[0])
                vals.append(rows[1] if S == 2 else rows[0][:Dv])
        for h in range(Hq):
            g = h // (Hq // H) if S == 2 else 0
            c0 = g * D
            logits = [scale * sum(q[b][h][d] * k[c0 + d] for d in range(D)) for k in keys]
            if not logits:
                continue
            w = [math.exp(x) for x in logits]
            z = sum(w)
            vc0 = c0 if S == 2 else 0
            out[b][h] = [sum(w[t] * vals[t][vc0 + d] for t in range(len(w))) / z for d in range(Dv)]
            lse[b][h] = math.log(z)
    return np.array(out), np.array(lse)


def _tiny_case(layout, seed, Hq, m=2):
    rng = np.random.default_rng(seed)
    S, L, T, F = layout.num_streams, 2, 3, layout.row_width
    canon = _store(rng, S, 3, L, T, F)
    patch = ([_bits(0.3 * rng.standard_normal((3, L, T, m))) for _ in range(S)],
             [_bits(0.3 * rng.standard_normal((3, L, F, m))) for _ in range(S)]) if m else None
    seq_entries, ids, deltas = [0, 2, 3, 3], [1, 0, 2], [5, -3, 11]
    q = _bits(0.5 * rng.standard_normal((3, Hq, layout.head_dim)))
    return canon, patch, seq_entries, ids, deltas, ko.bf16_bits_to_f64(q)


def _close(a, b, tol=1e-12):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    fin = np.isfinite(b)
    return (np.array_equal(np.isfinite(a), fin) and np.array_equal(a[~fin], b[~fin])
            and np.allclose(a[fin], b[fin], rtol=tol, atol=tol))


def _check_brute(layout, Hq, seed, m=2):
    canon, patch, se, ids, ds, q = _tiny_case(layout, seed, Hq, m)
    o1, l1 = ao.decode_attention_f64(layout, 1, canon, patch, se, ids, ds, q, Hq, 0.3)
    o2, l2 = _brute(layout, 1, canon, patch, se, ids, ds, q.tolist(), Hq, 0.3)
    return _close(o1, o2) and _close(l1, l2)


def pin_brute_force_gqa():
    lay = ko.Layout(2, 2, 8, 0, 8, 100.0, 2, ko.ROPE_HALF)
    return _check_brute(lay, Hq=4, seed=1)


def pin_brute_force_partial_interleaved():
    lay = ko.Layout(2, 2, 8, 2, 4, 50.0, 2, ko.ROPE_INTERLEAVED)
    return _check_brute(lay, Hq=2, seed=2, m=3)


def pin_brute_force_mla():
    lay = ko.Layout(2, 1, 12, 8, 4, 100.0, 1, ko.ROPE_HALF)
    return _check_brute(lay, Hq=3, seed=3)


def pin_uniform_keys():
    # one chunk whose K rows are all equal: p is uniform, out is the mean of
    # the values, lse = log T + s (delta = 0, no patch: s = scale q . k)
    lay = ko.Layout(1, 2, 16, 0, 16, 1e4, 2, ko.ROPE_HALF)
    rng = np.random.default_rng(4)
    T, F = 50, lay.row_width
    k = rng.standard_normal(F)
    canon = [_bits(np.broadcast_to(k, (1, 1, T, F))), _bits(rng.standard_normal((1, 1, T, F)))]
    q = ko.bf16_bits_to_f64(_bits(rng.standard_normal((1, 4, 16))))
    kb, vb = ko.bf16_bits_to_f64(canon[0][0, 0]), ko.bf16_bits_to_f64(canon[1][0, 0])
    ok = True
    for d in (0, 777):
        out, lse = ao.decode_attention_f64(lay, 0, canon, None, [0, 1], [0], [d], q, 4, 0.25)
        for h in range(4):
            g = h // 2
            ok &= np.allclose(out[0, h], vb[:, g * 16:(g + 1) * 16].mean(axis=0), rtol=1e-12, atol=1e-12)
            if d == 0:
                ok &= abs(lse[0, h] - (math.log(T) + 0.25 * float(q[0, h] @ kb[0, g * 16:(g + 1) * 16]))) < 1e-12
    return bool(ok)


def pin_head_mapping():
    # values of KV head g are the constant g + 1: query head h must return h // G + 1
    lay = ko.Layout(1, 4, 8, 0, 8, 1e4, 2, ko.ROPE_HALF)
    rng = np.random.default_rng(5)
    T, F = 7, lay.row_width
    vals = np.repeat(np.arange(1, 5, dtype=np.float64), 8)
    canon = [_bits(rng.standard_normal((2, 1, T, F))), _bits(np.broadcast_to(vals, (2, 1, T, F)))]
    q = ko.bf16_bits_to_f64(_bits(rng.standard_normal((1, 12, 8))))
    out, _ = ao.decode_attention_f64(lay, 0, canon, None, [0, 2], [1, 0], [3, -9], q, 12, 0.5)
    return all(np.allclose(out[0, h], h // 3 + 1, rtol=0, atol=1e-12) for h in range(12))


def pin_empty_context():
    lay = ko.Layout(1, 1, 8, 0, 8, 1e4, 2, ko.ROPE_HALF)
    rng = np.random.default_rng(6)
    canon = _store(rng, 2, 1, 1, 4, 8)
    q = rng.standard_normal((2, 2, 8))
    out, lse = ao.decode_attention_f64(lay, 0, canon, None, [0, 0, 1], [0], [0], q, 2, 1.0)
    return bool(np.all(out[0] == 0) and np.all(np.isneginf(lse[0])) and np.all(np.isfinite(lse[1])))


def _rope_heads(x, pos, lay):
    """RoPE of per-head vectors x [..., D] at position pos (complex form)."""
    y = np.array(x, np.float64)
    o, R = lay.rope_offset, lay.rope_dim
    for j in range(R // 2):
        if lay.rope_style == ko.ROPE_HALF:
            ia, ib = o + j, o + j + R // 2
        else:
            ia, ib = o + 2 * j, o + 2 * j + 1
        z = (x[..., ia] + 1j * x[..., ib]) * np.exp(1j * pos * math.pow(lay.rope_base, -2.0 * j / R))
        y[..., ia], y[..., ib] = z.real, z.imag
    return y


def pin_relative_position():
    # canonical keys carry RoPE at p_c + t; the query carries RoPE at its own
    # position s.  Moving the chunk by delta + x and the query to s + x keeps
    # every relative offset, so out and lse are unchanged.
    lay = ko.Layout(1, 2, 16, 0, 16, 1e3, 2, ko.ROPE_HALF)
    rng = np.random.default_rng(7)
    T, F, Hq = 24, lay.row_width, 4
    raw = rng.standard_normal((T, 2, 16))
    pc = 100
    canon_k = np.concatenate([_rope_heads(raw[:, h], pc + np.arange(T), lay) for h in range(2)], axis=1)
    canon = [_bits(canon_k[None, None]), _bits(rng.standard_normal((1, 1, T, F)))]
    y = rng.standard_normal((Hq, 16))
    s0, delta, x = 5000, 1700, -1234
    q1 = _rope_heads(y, s0, lay)[None]
    q2 = _rope_heads(y, s0 + x, lay)[None]
    o1, l1 = ao.decode_attention_f64(lay, 0, canon, None, [0, 1], [0], [delta], q1, Hq, 0.3)
    o2, l2 = ao.decode_attention_f64(lay, 0, canon, None, [0, 1], [0], [delta + x], q2, Hq, 0.3)
    # and the query's offset matters at all: a different x for the query alone changes the result
    o3, _ = ao.decode_attention_f64(lay, 0, canon, None, [0, 1], [0], [delta], q2, Hq, 0.3)
    return _close(o1, o2, 1e-9) and _close(l1, l2, 1e-9) and not _close(o1, o3, 1e-6)


def pin_split_merge():
    # attention over [A, B, C] = log-sum-exp merge of attention over each
    lay = ko.Layout(2, 2, 8, 0, 8, 1e4, 2, ko.ROPE_HALF)
    rng = np.random.default_rng(8)
    canon = _store(rng, 2, 3, 2, 5, 16)
    patch = ([_bits(0.3 * rng.standard_normal((3, 2, 5, 2))) for _ in range(2)],
             [_bits(0.3 * rng.standard_normal((3, 2, 16, 2))) for _ in range(2)])
    q = rng.standard_normal((1, 4, 8))
    ids, ds = [2, 0, 1], [40, -7, 300]
    o, l = ao.decode_attention_f64(lay, 1, canon, patch, [0, 3], ids, ds, q, 4, 0.7)
    qs = np.repeat(q, 3, axis=0)
    oe, le = ao.decode_attention_f64(lay, 1, canon, patch, [0, 1, 2, 3], ids, ds, qs, 4, 0.7)
    L = np.logaddexp.reduce(le, axis=0)
    w = np.exp(le - L)
    om = (w[:, :, None] * oe).sum(axis=0)
    return _close(o[0], om, 1e-12) and _close(l[0], L, 1e-12)


def _pool_case(rng, lay, layer, n_seqs, max_pages, P, slots):
    """A pool [L][slots][F] per stream, a block table of distinct pages and token counts."""
    S, L, F = lay.num_streams, lay.num_layers, lay.row_width
    pool = [_bits(rng.standard_normal((L, slots, F))) for _ in range(S)]
    pages = rng.permutation(slots // P)[:n_seqs * max_pages].reshape(n_seqs, max_pages)
    counts = rng.integers(1, max_pages * P + 1, size=n_seqs)
    return pool, pages, counts


def _brute_pool(lay, layer, pool, P, table_row, n, q, Hq, scale):
    """Attention of one sequence over its pooled tokens, by explicit loops:
    the rows are gathered page by page, the softmax by math.exp."""
    D, H, S = lay.head_dim, lay.num_heads, lay.num_streams
    rows_k, rows_v = [], []
    left = int(n)
    for page in table_row:
        if left <= 0:
            break
        take = min(P, left)
        for r in range(take):
            slot = int(page) * P + r
            rows_k.append([float(x) for x in ko.bf16_bits_to_f64(pool[0][layer][slot])])
            if S == 2:
                rows_v.append([float(x) for x in ko.bf16_bits_to_f64(pool[1][layer][slot])])
        left -= take
    Dv = D if S == 2 else lay.rope_offset
    G = Hq // H
    outs, lses = [], []
    for h in range(Hq):
        g = h // G if S == 2 else 0
        ks = [r[g * D:(g + 1) * D] for r in rows_k] if S == 2 else rows_k
        vs = [r[g * D:(g + 1) * D] for r in rows_v] if S == 2 else [r[:Dv] for r in rows_k]
        sc = [scale * sum(float(q[h][d]) * k[d] for d in range(D)) for k in ks]
        mx = max(sc)
        w = [math.exp(x - mx) for x in sc]
        tot = sum(w)
        outs.append([sum(w[t] * vs[t][c] for t in range(len(w))) / tot for c in range(Dv)])
        lses.append(mx + math.log(tot))
    return np.array(outs), np.array(lses)


def _pool_brute(lay, Hq, seed):
    rng = np.random.default_rng(seed)
    P, max_pages = 4, 3
    pool, table, counts = _pool_case(rng, lay, 1, 2, max_pages, P, 40)
    q = rng.standard_normal((2, Hq, lay.head_dim))
    S = lay.num_streams
    canon = _store(rng, S, 1, lay.num_layers, 3, lay.row_width)
    o, l = ao.decode_attention_f64(lay, 1, canon, None, [0, 0, 0], [], [], q, Hq, 0.4,
                                   pool=(pool, P, table, counts))
    ok = True
    for b in range(2):
        bo, bl = _brute_pool(lay, 1, pool, P, table[b], counts[b], q[b], Hq, 0.4)
        ok = ok and _close(o[b], bo, 1e-11) and _close(l[b], bl, 1e-11)
    return ok


def pin_pool_brute_gqa():
    return _pool_brute(ko.Layout(2, 2, 8, 0, 8, 1e4, 2, ko.ROPE_HALF), 4, 21)


def pin_pool_brute_mla():
    return _pool_brute(ko.Layout(2, 1, 24, 16, 8, 1e4, 1, ko.ROPE_HALF), 3, 22)


def pin_pool_equals_zero_shift_entry():
    # pooled tokens are read as stored: the same rows as a reused entry at
    # shift 0 with no patch give the same attention
    lay = ko.Layout(2, 2, 8, 0, 8, 1e4, 2, ko.ROPE_HALF)
    rng = np.random.default_rng(23)
    P = 4
    pool, table, counts = _pool_case(rng, lay, 1, 1, 3, P, 32)
    n = int(counts[0])
    t = np.arange(n)
    slots = table[0][t // P] * P + t % P
    canon = [x[:, slots][None] for x in pool]          # [1, L, n, F]: the rows as a store chunk
    q = rng.standard_normal((1, 4, 8))
    o1, l1 = ao.decode_attention_f64(lay, 1, canon, None, [0, 0], [], [], q, 4, 0.9, pool=(pool, P, table, counts))
    o2, l2 = ao.decode_attention_f64(lay, 1, canon, None, [0, 1], [0], [0], q, 4, 0.9)
    return _close(o1, o2, 1e-13) and _close(l1, l2, 1e-13)


def pin_pool_union_merge():
    # entries + pooled tokens = the log-sum-exp merge of the two parts
    lay = ko.Layout(2, 2, 8, 0, 8, 1e4, 2, ko.ROPE_HALF)
    rng = np.random.default_rng(24)
    P = 4
    pool, table, counts = _pool_case(rng, lay, 1, 1, 2, P, 24)
    canon = _store(rng, 2, 2, 2, 5, 16)
    patch = ([_bits(0.3 * rng.standard_normal((2, 2, 5, 2))) for _ in range(2)],
             [_bits(0.3 * rng.standard_normal((2, 2, 16, 2))) for _ in range(2)])
    q = rng.standard_normal((1, 4, 8))
    ids, ds = [1, 0], [70, -5]
    o, l = ao.decode_attention_f64(lay, 1, canon, patch, [0, 2], ids, ds, q, 4, 0.7, pool=(pool, P, table, counts))
    oe, le = ao.decode_attention_f64(lay, 1, canon, patch, [0, 2], ids, ds, q, 4, 0.7)
    op, lp = ao.decode_attention_f64(lay, 1, canon, patch, [0, 0], [], [], q, 4, 0.7, pool=(pool, P, table, counts))
    L = np.logaddexp(le[0], lp[0])
    om = np.exp(le[0] - L)[:, None] * oe[0] + np.exp(lp[0] - L)[:, None] * op[0]
    return _close(o[0], om, 1e-12) and _close(l[0], L, 1e-12)


PINS = {
    "pool_brute_gqa": pin_pool_brute_gqa,
    "pool_brute_mla": pin_pool_brute_mla,
    "pool_zero_shift_entry": pin_pool_equals_zero_shift_entry,
    "pool_union_merge": pin_pool_union_merge,
    "brute_gqa": pin_brute_force_gqa,
    "brute_partial_interleaved": pin_brute_force_partial_interleaved,
    "brute_mla": pin_brute_force_mla,
    "uniform_keys": pin_uniform_keys,
    "head_mapping": pin_head_mapping,
    "empty": pin_empty_context,
    "relative_position": pin_relative_position,
    "split_merge": pin_split_merge,
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


_orig_rows = ao.context_rows_f64
_orig_attend = ao.attend_f64


def _mut_reverse_shift(layout, layer, canon, patch, ids, deltas):
    return _orig_rows(layout, layer, canon, patch, ids, [-d for d in deltas])


def _mut_no_patch(layout, layer, canon, patch, ids, deltas):
    return _orig_rows(layout, layer, canon, None, ids, deltas)


def _mut_no_value_patch(layout, layer, canon, patch, ids, deltas):
    K, _ = _orig_rows(layout, layer, canon, patch, ids, deltas)
    if patch is None or layout.num_streams == 1:
        return K, _orig_rows(layout, layer, canon, patch, ids, deltas)[1]
    _, V = _orig_rows(layout, layer, canon, ([patch[0][0], 0 * patch[0][1]], [patch[1][0], 0 * patch[1][1]]),
                      ids, deltas)
    return K, V


def _mut_first_entry_only(layout, layer, canon, patch, ids, deltas):
    return _orig_rows(layout, layer, canon, patch, ids[:1], deltas[:1])


def _mut_rotate_values_too(layout, layer, canon, patch, ids, deltas):
    K, V = _orig_rows(layout, layer, canon, patch, ids, deltas)
    if V is not None:
        T = canon[0].shape[2]
        V = np.concatenate([ko.relocate_f64(V[i * T:(i + 1) * T], int(d), layout) for i, d in enumerate(deltas)]
                           + [V[len(deltas) * T:]], axis=0)
    return K, V


_orig_pool = ao.pool_rows_f64


def _mut_pool_layer0(layout, layer, pool_bits, page_size, table_row, n_tokens):
    return _orig_pool(layout, 0, pool_bits, page_size, table_row, n_tokens)


def _mut_pool_no_in_page(layout, layer, pool_bits, page_size, table_row, n_tokens):
    t = np.arange(int(n_tokens), dtype=np.int64)
    slots = np.asarray(table_row, np.int64)[t // page_size] * page_size
    K = ko.bf16_bits_to_f64(pool_bits[0][layer][slots])
    V = ko.bf16_bits_to_f64(pool_bits[1][layer][slots]) if layout.num_streams == 2 else None
    return K, V


def _mut_pool_relocated(layout, layer, pool_bits, page_size, table_row, n_tokens):
    K, V = _orig_pool(layout, layer, pool_bits, page_size, table_row, n_tokens)
    return ko.relocate_f64(K, 50, layout), V


def _mut_no_scale(q, k, v, scale):
    return _orig_attend(q, k, v, 1.0)


def _mut_unnormalised(q, k, v, scale):
    o, l = _orig_attend(q, k, v, scale)
    return o * np.exp(l), l


def _mut_head_modulo(h, hq, hkv):
    return h % hkv


def _mut_mla_full_value(layout):
    return layout.head_dim


@pytest.mark.parametrize("name,attr,mutant", [
    ("relocation by -delta", "context_rows_f64", _mut_reverse_shift),
    ("patch dropped", "context_rows_f64", _mut_no_patch),
    ("value patch dropped", "context_rows_f64", _mut_no_value_patch),
    ("only the first entry of a context", "context_rows_f64", _mut_first_entry_only),
    ("values rotated too", "context_rows_f64", _mut_rotate_values_too),
    ("scale ignored", "attend_f64", _mut_no_scale),
    ("softmax not normalised", "attend_f64", _mut_unnormalised),
    ("query head h reads KV head h % Hkv", "kv_head_of", _mut_head_modulo),
    ("MLA value includes k_rope", "value_dim", _mut_mla_full_value),
    ("pooled rows read from layer 0", "pool_rows_f64", _mut_pool_layer0),
    ("pooled token's place in its page dropped", "pool_rows_f64", _mut_pool_no_in_page),
    ("pooled keys shifted", "pool_rows_f64", _mut_pool_relocated),
])
def test_planted_mistakes(monkeypatch, name, attr, mutant):
    assert all(_all().values())
    monkeypatch.setattr(ao, attr, mutant)
    res = _all()
    assert not all(res.values()), f"no pin caught the planted mistake: {name}"
