"""CPU oracle of decode attention over a reused context.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The product path never imports, calls or
links it, and it imports nothing from the product package.

Source: "Kamera: Unified Position-Invariant Multimodal KV Cache for
Training-Free Reuse", technical summaries on gist.science (paper 2606.23581).
Section 2 gives the reuse equation KV^(B|A) = R(delta) KV(B|empty) + U_m V_m^T;
section 3 ("Production deployment") has the engine's attention read the
reconstructed cache; section 4 notes that the cost moves to memory bandwidth,
the bound of the decode phase.  What a decode step computes from that cache is
ordinary scaled dot-product attention, written out here in float64:

* the context of one sequence is a list of entries e, each a stored chunk
  (chunk_ids[e]) placed with shift deltas[e]; its keys and values at layer l
  are the reuse equation applied to the stored rows (the reuse oracle's
  ``reuse_f64``: R(delta) on the key stream only, then U V^T), exactly, with
  no bfloat16 rounding in between;
* GQA/MHA: query head h reads KV head g = h // G with G = Hq / Hkv (groups of
  consecutive query heads share a KV head); its keys and values are the D
  columns of head g;
* MLA (one stream): every query head reads the one joint row as its key (all
  head_dim columns) and the row's first rope_offset columns (c_KV) as its
  value; the caller's queries are the absorbed ones, head_dim wide;
* s_t = scale * q . k_t,  p = softmax(s) over the whole context,
  out = sum_t p_t v_t,  lse = log sum_t exp(s_t)  (natural logarithm);
* a sequence with an empty context gets out = 0 and lse = -inf.

Nothing is blocked, split or reordered: the keys and values are built in full
and the softmax is taken over them in one piece.
"""

from __future__ import annotations

import numpy as np

from . import kamera_oracle as ko


def value_dim(layout: "ko.Layout") -> int:
    """Width of one head's value: head_dim (two streams), rope_offset (MLA)."""
    return layout.head_dim if layout.num_streams == 2 else layout.rope_offset


def kv_head_of(h: int, num_q_heads: int, num_kv_heads: int) -> int:
    """KV head read by query head h: h // G, G = Hq / Hkv (consecutive query heads share one)."""
    return h // (num_q_heads // num_kv_heads)


def context_rows_f64(layout: "ko.Layout", layer: int, canon_bits, patch, chunk_ids, deltas):
    """Keys and values of a context at one layer, float64: (K [N, F], V [N, F] or None for MLA).

    canon_bits[s]: bfloat16 bits [n_store, L, T, F] of stream s.  patch: None
    or (u_bits, v_bits) with u_bits[s] [n_store, L, T, m], v_bits[s]
    [n_store, L, F, m].  Entry e contributes its T rows in order.
    """
    S = layout.num_streams
    ks, vs = [], []
    for cid, d in zip(chunk_ids, deltas):
        rows = []
        for s in range(S):
            x = ko.bf16_bits_to_f64(canon_bits[s][cid, layer])
            u = v = None
            if patch is not None:
                u = ko.bf16_bits_to_f64(patch[0][s][cid, layer])
                v = ko.bf16_bits_to_f64(patch[1][s][cid, layer])
            rows.append(ko.reuse_f64(x, int(d), u, v, layout, rotate=(s == 0)))
        ks.append(rows[0])
        if S == 2:
            vs.append(rows[1])
    F = layout.row_width
    K = np.concatenate(ks, axis=0) if ks else np.zeros((0, F))
    V = (np.concatenate(vs, axis=0) if vs else np.zeros((0, F))) if S == 2 else None
    return K, V


def attend_f64(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float):
    """softmax(scale * k q) v and its log-sum-exp for one query vector.

    q [D], k [N, D], v [N, Dv]; N = 0 gives (zeros, -inf).
    """
    if k.shape[0] == 0:
        return np.zeros(v.shape[1]), -np.inf
    s = scale * (k @ q)
    mx = s.max()
    p = np.exp(s - mx)
    l = p.sum()
    return (p @ v) / l, mx + np.log(l)


def pool_rows_f64(layout: "ko.Layout", layer: int, pool_bits, page_size: int, table_row, n_tokens: int):
    """Keys and values of a sequence's first n_tokens tokens in a paged pool.

    The engine's own cache (Kamera summary, section 3, "Production
    deployment": its attention reads the cache in its pool): token t sits in
    slot table_row[t // P] * P + t % P of the pool [L][slots][F] of each
    stream, stored in its own frame, so it is read as it is -- widened, no
    shift, no patch.  Returns (K [n, F], V [n, F] or None for MLA).
    """
    t = np.arange(int(n_tokens), dtype=np.int64)
    slots = np.asarray(table_row, np.int64)[t // page_size] * page_size + t % page_size
    K = ko.bf16_bits_to_f64(pool_bits[0][layer][slots])
    V = ko.bf16_bits_to_f64(pool_bits[1][layer][slots]) if layout.num_streams == 2 else None
    return K, V


def decode_attention_f64(layout: "ko.Layout", layer: int, canon_bits, patch, seq_entries, chunk_ids, deltas,
                         q, num_q_heads: int, scale: float, pool=None):
    """Decode attention of every sequence over its reused context.

    seq_entries [B + 1]: sequence b owns entries seq_entries[b] .. seq_entries[b+1]-1
    of chunk_ids / deltas.  q: float64 [B, Hq, head_dim] (the query as given,
    already rotated to its own position).  pool: None, or (pool_bits,
    page_size, block_table [B][max_pages], seq_tokens [B]): sequence b also
    attends its first seq_tokens[b] pooled tokens (pool_rows_f64); the
    softmax runs over the union.  Returns (out [B, Hq, Dv], lse [B, Hq]).
    """
    q = np.asarray(q, np.float64)
    B = len(seq_entries) - 1
    D = layout.head_dim
    Dv = value_dim(layout)
    mla = layout.num_streams == 1
    out = np.zeros((B, num_q_heads, Dv))
    lse = np.full((B, num_q_heads), -np.inf)
    for b in range(B):
        e0, e1 = int(seq_entries[b]), int(seq_entries[b + 1])
        K, V = context_rows_f64(layout, layer, canon_bits, patch, chunk_ids[e0:e1], deltas[e0:e1])
        if pool is not None:
            pool_bits, P, table, counts = pool
            Kp, Vp = pool_rows_f64(layout, layer, pool_bits, P, table[b], counts[b])
            K = np.concatenate([K, Kp])
            V = None if V is None else np.concatenate([V, Vp])
        for h in range(num_q_heads):
            if mla:
                k, v = K, K[:, :Dv]
            else:
                g = kv_head_of(h, num_q_heads, layout.num_heads)
                k, v = K[:, g * D:(g + 1) * D], V[:, g * D:(g + 1) * D]
            out[b, h], lse[b, h] = attend_f64(q[b, h], k, v, scale)
    return out, lse
