"""CPU oracle of the Kamera reuse operator.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The product path (the HIP library and its
Python binding) never imports, calls or links it, and this module imports
nothing from the product package.  The two share no code: the seeded input
generators live in ``workloads/`` and hold none of the operator's arithmetic.

Source of the method: "Kamera: Unified Position-Invariant Multimodal KV Cache
for Training-Free Reuse", technical summaries on gist.science (paper
2606.23581; Italian and Chinese pages, which are parallel translations).
Citations below name the section of those pages.

What is computed (Kamera summary, section 2 "Methodology: the Kamera
operator", reuse equation):

    KV^(B|A) = R(delta) . KV(B|empty) + U_m V_m^T

* R(delta) re-rotates the cached keys by the RoPE phase shift of the chunk's
  new position; the pages call it an exact algebraic operation, not a forward
  pass (section 2, "Relocation" bullet).
* U_m V_m^T is the rank-m conditioning patch, added after the relocation
  (section 2, "Patch application" bullet).
* GQA/MHA relocate the full K and patch K and V; MLA relocates only the
  decoupled 64-dim k_rope, reuses c_KV byte for byte, and patches both channels
  (section 2, "Unified architecture support").

The result has a plain closed form, so this oracle is that definition written
out: every element in float64, rounded ONCE to bfloat16 with round-to-nearest-
even.  Elements that neither the rotation nor the patch touch are copied bit
for bit.  Nothing is blocked, fused or reordered beyond the definition.

Readings of points the pages leave open (each is stated where it is used):

* Frame: canonical keys already carry RoPE at chunk positions p_c + t, and
  R(delta) is one uniform phase shift delta for the whole chunk.
* Pairing: rotate-half (element j pairs with j + R/2 inside the rotated span
  of a head) by default, interleaved (2j, 2j+1) as an option.  Positive delta
  moves the chunk later: (a, b) -> (a cos - b sin, b cos + a sin).
* Frequencies: theta_j = base^(-2j/R), no frequency scaling.
* One patch per (chunk, layer, stream) over the flattened H*D feature axis;
  U is T x m, V is F x m; the patch is added in the destination frame.
* Destination: per layer and stream a token-major pool [slots][F]; token t of
  output chunk i goes to slot page_table[i][t // P] * P + t % P (paged) or
  dst_offset[i] + t (contiguous).
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

ROPE_HALF = 0          # rotate-half pairing (j, j + R/2)
ROPE_INTERLEAVED = 1   # interleaved pairing (2j, 2j + 1)


@dataclass(frozen=True)
class Layout:
    """Shape of one row of the KV store.

    A row holds num_heads heads of head_dim elements (F = num_heads*head_dim).
    In every head of stream 0 the elements [rope_offset, rope_offset+rope_dim)
    carry RoPE; stream 1 (GQA/MHA values) never does.  MLA is one stream whose
    row is c_KV followed by k_rope (Kamera summary, section 2, "Unified
    architecture support").
    """

    num_layers: int
    num_heads: int
    head_dim: int
    rope_offset: int
    rope_dim: int
    rope_base: float
    num_streams: int
    rope_style: int = ROPE_HALF

    @property
    def row_width(self) -> int:
        return self.num_heads * self.head_dim


# ---------------------------------------------------------------------------
# bfloat16 <-> float64
# ---------------------------------------------------------------------------

def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact widening: a bfloat16 is the top 16 bits of a binary32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x) -> np.ndarray:
    """Round float64 values ONCE to bfloat16, round-to-nearest, ties-to-even.

    bfloat16 keeps 8 significant bits.  For |x| in [2^(e-1), 2^e) the spacing
    of representable values is 2^(e-8); below the smallest normal (2^-126) the
    spacing stays at the subnormal quantum 2^-133.  The value is scaled so the
    quantum becomes 1, rounded with numpy's rint (ties to even), scaled back,
    and the now exactly representable value is read off as the top half of a
    binary32.  Rounding through float32 first would round twice, which is not
    what the definition asks for.
    """
    x = np.asarray(x, dtype=np.float64)
    neg = np.signbit(x)
    a = np.abs(x)
    _, e = np.frexp(a)                       # a = f * 2^e with f in [0.5, 1)
    q = np.maximum(e - 8, -133)              # log2 of the spacing at a
    with np.errstate(over="ignore", invalid="ignore"):
        y = np.ldexp(np.rint(np.ldexp(a, -q)), q)
        y32 = y.astype(np.float32)           # exact (or inf past the top)
    bits = (y32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    return bits | (neg.astype(np.uint16) << np.uint16(15))


# ---------------------------------------------------------------------------
# RoPE relocation R(delta)
# ---------------------------------------------------------------------------

def rope_inv_freq(rope_dim: int, base: float) -> np.ndarray:
    """theta_j = base^(-2j/R), j = 0 .. R/2-1 (standard RoPE frequencies)."""
    j = np.arange(rope_dim // 2, dtype=np.float64)
    return np.power(np.float64(base), -2.0 * j / rope_dim)


def rope_pairs(layout: Layout):
    """Element index pairs (a, b) of one row and their frequency index j.

    Rotate-half pairs element o+j with o+j+R/2; interleaved pairs o+2j with
    o+2j+1; o is rope_offset inside each head.
    """
    o, r, d = layout.rope_offset, layout.rope_dim, layout.head_dim
    j = np.arange(r // 2)
    ia, ib, jj = [], [], []
    for h in range(layout.num_heads):
        base = h * d + o
        if layout.rope_style == ROPE_HALF:
            ia.append(base + j)
            ib.append(base + j + r // 2)
        else:
            ia.append(base + 2 * j)
            ib.append(base + 2 * j + 1)
        jj.append(j)
    return np.concatenate(ia), np.concatenate(ib), np.concatenate(jj)


def relocate_f64(x: np.ndarray, delta: int, layout: Layout) -> np.ndarray:
    """R(delta) on rows x[..., F] (float64): rotate every RoPE pair by delta*theta_j.

    Kamera summary, section 2, "Relocation": the keys are turned again by the
    RoPE phase shift of the new position.  Elements outside the RoPE span are
    returned unchanged.
    """
    y = np.array(x, dtype=np.float64, copy=True)
    ia, ib, j = rope_pairs(layout)
    phi = np.float64(delta) * rope_inv_freq(layout.rope_dim, layout.rope_base)[j]
    c, s = np.cos(phi), np.sin(phi)
    a, b = x[..., ia], x[..., ib]
    y[..., ia] = a * c - b * s
    y[..., ib] = b * c + a * s
    return y


def rope_touched_mask(layout: Layout) -> np.ndarray:
    """Boolean [F]: True on elements the rotation acts on."""
    m = np.zeros(layout.row_width, dtype=bool)
    ia, ib, _ = rope_pairs(layout)
    m[ia] = True
    m[ib] = True
    return m


# ---------------------------------------------------------------------------
# Rank-m patch U_m V_m^T and the reuse operator
# ---------------------------------------------------------------------------

def patch_f64(u: np.ndarray, v: np.ndarray) -> np.ndarray:
    """U V^T with U [T, m] and V [F, m]: the rank-m conditioning patch [T, F].

    Kamera summary, section 2, "Patch application".
    """
    return np.asarray(u, np.float64) @ np.asarray(v, np.float64).T


def reuse_f64(x: np.ndarray, delta: int, u, v, layout: Layout, rotate: bool) -> np.ndarray:
    """R(delta) x + U V^T for one (chunk, layer, stream) block, all float64.

    Kamera summary, section 2, reuse equation.  ``rotate`` is True for the
    stream that carries RoPE (GQA/MHA keys, the MLA joint row).  ``u``/``v``
    may be None for m = 0.
    """
    y = relocate_f64(x, delta, layout) if rotate else np.array(x, dtype=np.float64)
    if u is not None and np.asarray(u).shape[-1] > 0:
        y = y + patch_f64(u, v)
    return y


def reuse_block_bits(x_bits, delta: int, u_bits, v_bits, layout: Layout, rotate: bool) -> np.ndarray:
    """The operator on bfloat16 storage for one block [T, F] -> bfloat16 bits.

    Inputs are widened exactly, the result is formed in float64 and rounded
    once.  Elements that neither the rotation nor the patch touches are copied
    bit for bit: with m = 0 the value stream and the MLA c_KV channel are byte
    copies (Kamera summary, section 2, "Unified architecture support", MLA).
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    m = 0 if u_bits is None else np.asarray(u_bits).shape[-1]
    u = None if m == 0 else bf16_bits_to_f64(u_bits)
    v = None if m == 0 else bf16_bits_to_f64(v_bits)
    y = reuse_f64(bf16_bits_to_f64(x_bits), delta, u, v, layout, rotate)
    out = f64_to_bf16_bits(y)
    if m == 0:
        keep = ~rope_touched_mask(layout) if rotate else np.ones(layout.row_width, bool)
        out[..., keep] = x_bits[..., keep]
    return out


# ---------------------------------------------------------------------------
# Per-chunk shift delta for the three window operations
# ---------------------------------------------------------------------------

def deltas_relocate(delta) -> list[int]:
    """Sliding-window survival and plain relocation: delta_i is given.

    Kamera summary, section 3, "Sliding-Window Survival": survivors only need
    the exact re-rotation.
    """
    return [int(d) for d in delta]


def deltas_reorder(perm, base_pos: int, n_tokens: int, canon_pos=None) -> list[int]:
    """Reorder: output slot k holds store chunk c = perm[k] at base + k*T.

    Kamera summary, section 3, "Reorder": one orbit patch per chunk serves
    every ordering, so only the shift changes with the order.  The chunk's
    cached frame starts at canon_pos[c] (0 when absent), hence
    delta_k = base + k*T - p_c.
    """
    out = []
    for k, c in enumerate(perm):
        p = 0 if canon_pos is None else int(canon_pos[int(c)])
        out.append(int(base_pos) + k * int(n_tokens) - p)
    return out


def deltas_recall(chunk_ids, target_pos, canon_pos=None) -> list[int]:
    """Recall: evicted store chunk ids[i] is rehydrated at target position q_i.

    Kamera summary, section 3, "Recall (reversible eviction)": the chunk comes
    back from the canonical store with a fresh patch; delta_i = q_i - p_c.
    """
    out = []
    for c, q in zip(chunk_ids, target_pos):
        p = 0 if canon_pos is None else int(canon_pos[int(c)])
        out.append(int(q) - p)
    return out


# ---------------------------------------------------------------------------
# Destination slots and the whole call
# ---------------------------------------------------------------------------

def dest_slots(i: int, n_tokens: int, page_size: int, page_table=None, dst_offset=None) -> np.ndarray:
    """Pool slot of every token of output chunk i.

    Paged (page_size P > 0): slot = page_table[i][t // P] * P + t % P.
    Contiguous (P = 0): slot = dst_offset[i] + t.
    """
    t = np.arange(n_tokens, dtype=np.int64)
    if page_size > 0:
        pages = np.asarray(page_table, dtype=np.int64)[i]
        return pages[t // page_size] * page_size + t % page_size
    return np.int64(dst_offset[i]) + t


def reconstruct(layout: Layout, src, src_ids, deltas, pools, page_size: int,
                page_table=None, dst_offset=None, u=None, v=None) -> None:
    """Apply the operator for a list of output chunks and scatter into the pool.

    src[s]   : uint16 [n_store, L, T, F]   canonical rows of stream s
    src_ids  : store chunk id of every output chunk i
    deltas   : shift of every output chunk i
    pools[s] : uint16 [L, slots, F]        written in place; other slots untouched
    u[s], v[s]: uint16 [n_store, L, T, m] and [n_store, L, F, m], or None (m = 0)
    Stream 0 carries RoPE; stream 1 (if any) never does.
    """
    n_tokens = src[0].shape[2]
    for i, (c, d) in enumerate(zip(src_ids, deltas)):
        slots = dest_slots(i, n_tokens, page_size, page_table, dst_offset)
        for s in range(layout.num_streams):
            for l in range(layout.num_layers):
                ub = None if u is None or u[s] is None else u[s][c, l]
                vb = None if v is None or v[s] is None else v[s][c, l]
                blk = reuse_block_bits(src[s][c, l], d, ub, vb, layout, rotate=(s == 0))
                pools[s][l, slots] = blk


def targets_reorder_varlen(order, lengths, base_pos: int) -> list[int]:
    """Target positions of a reorder of variable-length chunks.

    Kamera summary, section 3, "Reorder" places the cached chunks of a set in
    a new order; the pages fix no chunk length.  Reading: the chunks follow
    one another without gaps from base_pos on, so the chunk in slot k starts
    after the lengths of the chunks in slots 0..k-1.  (Equal lengths T give
    base_pos + k*T, the fixed-length reorder.)
    """
    out, pos = [], int(base_pos)
    for c in order:
        out.append(pos)
        pos += int(lengths[int(c)])
    return out


def reconstruct_varlen(layout: Layout, src, row_offset, n_tokens, src_ids, deltas, pools, page_size: int,
                       page_table=None, dst_offset=None, u=None, v=None) -> None:
    """The operator over a store of variable-length chunks, scattered into the pool.

    src[s]    : uint16 [total_rows, F]; store chunk c has T_c = n_tokens[c]
                tokens per layer, its layer-l rows at
                src[s][row_offset[c] + l*T_c : row_offset[c] + (l+1)*T_c]
    u[s]      : uint16 [total_rows, m], rows in the same order; v[s]: uint16
                [n_store, L, F, m]; or None (m = 0)
    src_ids   : store chunk id of every output chunk i; deltas: its shift
    pools[s]  : uint16 [L, slots, F], written in place: output chunk i's
                T_c tokens go to dest_slots(i, T_c, ...), i.e. the first
                ceil(T_c/P) entries of its page-table row (paged) or
                dst_offset[i] + t (contiguous)
    Every (chunk, layer, stream) block is the same closed form as for a
    fixed-length store (reuse_block_bits); only where the rows come from and
    how many there are differ.
    """
    for i, (c, d) in enumerate(zip(src_ids, deltas)):
        c = int(c)
        T = int(n_tokens[c])
        if T == 0:
            continue
        r0 = int(row_offset[c])
        slots = dest_slots(i, T, page_size, page_table, dst_offset)
        for s in range(layout.num_streams):
            for l in range(layout.num_layers):
                rows = slice(r0 + l * T, r0 + (l + 1) * T)
                ub = None if u is None or u[s] is None else u[s][rows]
                vb = None if v is None or v[s] is None else v[s][c, l]
                pools[s][l, slots] = reuse_block_bits(src[s][rows], d, ub, vb, layout, rotate=(s == 0))


def patch_bytes_fraction(rank: int, n_tokens: int, row_width: int) -> float:
    """Bytes of one rank-m patch (U: T x m, V: F x m) over the block's KV bytes (T x F).

    Kamera summary, section 4, "Efficiency / Memory" prints this ratio for
    rank 64 and rank 16 segments.
    """
    return rank * (n_tokens + row_width) / (n_tokens * row_width)
