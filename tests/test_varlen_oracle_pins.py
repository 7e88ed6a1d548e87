"""Pins of the oracle's variable-length functions (CPU).

reconstruct_varlen reads store chunk c's layer-l rows at
[row_offset[c] + l*T_c, + T_c) of a packed store and scatters output chunk i's
T_c tokens to the first ceil(T_c/P) pages of its page-table row.  Its
arithmetic is the pinned fixed-length block function; what is new is the
indexing, and these tests fix that against the fixed-length oracle:

* equal lengths with row_offset[c] = c*L*T make the packed store the fixed
  store's own memory, so the result must equal ``reconstruct`` bit for bit;
* with different lengths, every output chunk must equal a one-chunk
  fixed-length call on that chunk's rows, cut out of the packed store by a
  reshape (not by the oracle's slicing), and no other slot may change;
* the reorder targets must tile [base, base + sum of lengths) in order, and
  reduce to base + k*T at equal lengths.
"""

import numpy as np
import pytest
import torch

from oracle import kamera_oracle as ko
from workloads import SENTINEL_BITS, VarlenWorkload, bits, make_inputs, make_varlen_inputs, small_workload


def _layout(w):
    return ko.Layout(w.num_layers, w.num_heads, w.head_dim, w.rope_offset, w.rope_dim, w.rope_base,
                     w.num_streams, w.rope_style)


def _np(t):
    return None if t is None else t.cpu().numpy()


@pytest.mark.parametrize("page_size,rank", [(16, 8), (0, 8), (16, 0)])
def test_equal_lengths_reduce_to_fixed_store(page_size, rank):
    w = small_workload(op="recall", n_tokens=48, n_chunks=3, n_store=4, rank=rank, page_size=page_size,
                       canon_pos_range=(0, 500))
    inp = make_inputs(w, seed=11)
    lay = _layout(w)
    L, T, F, S = w.num_layers, w.n_tokens, w.row_width, w.num_streams
    ns = w.store_chunks
    ids = inp["chunk_ids"].numpy()
    cp = inp["canon_pos"].numpy()
    deltas = ko.deltas_recall(ids, inp["target_pos"].numpy(), cp)
    src = [bits(x) for x in inp["src"]]
    u = None if inp["u"] is None else [bits(x) for x in inp["u"]]
    v = None if inp["v"] is None else [bits(x) for x in inp["v"]]
    pools_a = [bits(p).copy() for p in inp["pool"]]
    pools_b = [bits(p).copy() for p in inp["pool"]]
    ko.reconstruct(lay, src, ids, deltas, pools_a, page_size, _np(inp["page_table"]), _np(inp["dst_offset"]),
                   u, v)
    packed = [x.reshape(ns * L * T, F) for x in src]
    upk = None if u is None else [x.reshape(ns * L * T, rank) for x in u]
    row_offset = np.arange(ns, dtype=np.int64) * L * T
    n_tok = np.full(ns, T, dtype=np.int32)
    ko.reconstruct_varlen(lay, packed, row_offset, n_tok, ids, deltas, pools_b, page_size,
                          _np(inp["page_table"]), _np(inp["dst_offset"]), upk, v)
    for s in range(S):
        assert np.array_equal(pools_a[s], pools_b[s])


@pytest.mark.parametrize("page_size", [16, 0])
def test_each_chunk_equals_a_one_chunk_fixed_call(page_size):
    base = small_workload(op="recall", n_chunks=4, n_store=5, rank=8, page_size=page_size,
                          canon_pos_range=(0, 900))
    vw = VarlenWorkload("pin", base, len_range=(1, 70), len_multiple=1)
    inp = make_varlen_inputs(vw, seed=5)
    lay = _layout(base)
    L, F, S, m = base.num_layers, base.row_width, base.num_streams, base.rank
    lengths = inp["lengths"]
    ro = inp["row_offset"].numpy()
    ids = inp["chunk_ids"].numpy()
    cp = inp["canon_pos"].numpy()
    deltas = ko.deltas_recall(ids, inp["target_pos"].numpy(), cp)
    src = [bits(x) for x in inp["src"]]
    u = [bits(x) for x in inp["u"]]
    v = [bits(x) for x in inp["v"]]
    pt = _np(inp["page_table"])
    offs = _np(inp["dst_offset"])
    pools = [bits(p).copy() for p in inp["pool"]]
    ko.reconstruct_varlen(lay, src, ro, inp["n_tokens"].numpy(), ids, deltas, pools, page_size, pt, offs, u, v)

    expect = [np.full_like(p, SENTINEL_BITS) for p in pools]
    for i, c in enumerate(ids):
        T = lengths[c]
        one_src = [x[ro[c]:ro[c] + L * T].reshape(1, L, T, F) for x in src]
        one_u = [x[ro[c]:ro[c] + L * T].reshape(1, L, T, m) for x in u]
        one_v = [x[c:c + 1] for x in v]
        if page_size:
            one_pt = pt[i:i + 1, :-(-T // page_size)]
            ko.reconstruct(lay, one_src, [0], [deltas[i]], expect, page_size, page_table=one_pt,
                           u=one_u, v=one_v)
            assert (pt[i, -(-T // page_size):] == -1).all()   # entries past the chunk's pages are unused
        else:
            ko.reconstruct(lay, one_src, [0], [deltas[i]], expect, 0, dst_offset=offs[i:i + 1], u=one_u, v=one_v)
    for s in range(S):
        assert np.array_equal(pools[s], expect[s])
    # every output token landed somewhere: the written slots number sum(T_i) per (layer, stream)
    written = (pools[0][0] != SENTINEL_BITS).any(axis=-1).sum()
    assert written == sum(lengths[c] for c in ids)


def test_zero_length_chunk_writes_nothing():
    base = small_workload(op="relocate_patch", n_chunks=2, n_store=2, rank=8, page_size=16)
    lay = _layout(base)
    L, F, m = base.num_layers, base.row_width, base.rank
    rng = np.random.default_rng(3)
    src = [bits(torch.from_numpy(rng.standard_normal((L * 20, F)).astype(np.float32)).to(torch.bfloat16))
           for _ in range(2)]
    u = [np.zeros((L * 20, m), dtype=np.uint16) for _ in range(2)]
    v = [np.zeros((2, L, F, m), dtype=np.uint16) for _ in range(2)]
    pools = [np.full((L, 64, F), SENTINEL_BITS, dtype=np.uint16) for _ in range(2)]
    pt = np.array([[0, 1], [2, 3]], dtype=np.int64)
    ko.reconstruct_varlen(lay, src, np.array([0, 0]), np.array([0, 20]), [0, 1], [0, 0], pools, 16, pt, None, u, v)
    assert (pools[0][:, :32] == SENTINEL_BITS).all()          # chunk 0 is empty
    # chunk 1 (20 tokens, delta 0, zero factors) is its rows copied: pages 2 and 3
    for l in range(L):
        assert np.array_equal(pools[1][l, 32:52], src[1][l * 20:(l + 1) * 20])


def test_reorder_targets_tile_the_window():
    rng = np.random.default_rng(7)
    lengths = rng.integers(1, 300, size=12)
    order = rng.permutation(12)
    base = 1000
    tg = ko.targets_reorder_varlen(order, lengths, base)
    spans = sorted((tg[k], tg[k] + int(lengths[c])) for k, c in enumerate(order))
    assert spans[0][0] == base
    assert all(spans[j][1] == spans[j + 1][0] for j in range(len(spans) - 1))
    assert spans[-1][1] == base + int(lengths.sum())
    # equal lengths: the fixed-length reorder's base + k*T
    eq = ko.targets_reorder_varlen(order, np.full(12, 64), base)
    assert eq == ko.deltas_reorder(order, base, 64)
