"""Seeded synthetic inputs for the Kamera reuse operator.

This module produces INPUTS only — canonical rows, patch factors, shifts,
permutations, page tables and sentinel-filled pools — and holds none of the
operator's arithmetic (no rotation, no patch product, no output rounding).  It
serves both the CPU oracle and the HIP path; neither of those imports the
other.

The five workloads mirror the shapes the Kamera pages report on (Kamera summary
on gist.science, paper 2606.23581: section 2 "Unified architecture support" for
the GQA/MLA families, section 3 "Three cheap window operations" for sliding
window survival, reorder and recall, section 4 for the Qwen2.5-VL / DeepSeek
backbones).  The pages' datasets (MM-NIAH, MileBench, long video) and model
weights are not used: seeded Gaussian rows of the same shapes stand in for
them.

Recipe (every tensor is seeded; sigma is a standard deviation):
* canonical rows ~ N(0, 1) drawn in float32 and rounded to bfloat16 by torch;
  "outlier" workloads then scale a seeded 5% of feature columns per
  (layer, stream) by 8 (exact in bfloat16);
* patch factors ~ N(0, sigma), same rounding;
* shifts: integers uniform over the inclusive range, one draw per chunk;
* page tables: a seeded permutation of ceil(1.25 x needed) pool pages, the
  first `needed` used row by row; pools are pre-filled with the sentinel
  bfloat16 bit pattern 0x7FA5 (a NaN payload the operator never produces).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, replace

import numpy as np
import torch

SENTINEL_BITS = 0x7FA5
ROPE_HALF = 0
ROPE_INTERLEAVED = 1


@dataclass(frozen=True)
class Workload:
    name: str
    family: str                 # "MHA" | "GQA" | "MLA"
    op: str                     # "relocate" | "relocate_patch" | "reorder" | "recall"
    num_layers: int
    num_heads: int
    head_dim: int
    rope_offset: int
    rope_dim: int
    rope_base: float
    num_streams: int
    n_tokens: int               # T, tokens per chunk
    n_chunks: int               # output chunks of one call
    rank: int = 0               # m
    sigma: float = 0.0          # factor standard deviation
    page_size: int = 0          # 0 = contiguous destination
    delta_fixed: int | None = None
    delta_range: tuple | None = None    # inclusive (lo, hi)
    delta_negate: bool = False          # sliding window: delta = -(evicted length)
    outlier_frac: float = 0.0
    n_store: int | None = None          # chunks in the canonical store (default n_chunks)
    rope_style: int = ROPE_HALF
    canon_pos_range: tuple | None = None  # frame start p_c of each store chunk
    base_pos: int = 0                     # reorder: position of output slot 0
    contiguous_slack: int = 64            # spare slots around a contiguous chunk

    @property
    def row_width(self) -> int:
        return self.num_heads * self.head_dim

    @property
    def store_chunks(self) -> int:
        return self.n_store if self.n_store is not None else self.n_chunks

    @property
    def pages_per_chunk(self) -> int:
        return -(-self.n_tokens // self.page_size) if self.page_size else 0

    def kv_bytes(self) -> int:
        """Canonical rows read + rows written (bfloat16) by one call."""
        return 2 * 2 * self.num_streams * self.num_layers * self.n_chunks * self.n_tokens * self.row_width

    def factor_bytes(self) -> int:
        """U (T x m) and V (F x m) read once per (output chunk, layer, stream)."""
        return (2 * self.rank * (self.n_tokens + self.row_width)
                * self.num_streams * self.num_layers * self.n_chunks)

    def index_bytes(self) -> int:
        per = 4 * self.pages_per_chunk if self.page_size else 8
        return self.n_chunks * (per + 8)

    def algorithmic_bytes(self) -> int:
        return self.kv_bytes() + self.factor_bytes() + self.index_bytes()


CONFIGS = [
    Workload("tiny_mha_relocate_patch", "MHA", "relocate_patch", num_layers=1, num_heads=2,
             head_dim=64, rope_offset=0, rope_dim=64, rope_base=1e4, num_streams=2,
             n_tokens=256, n_chunks=1, rank=8, sigma=0.05, delta_fixed=300),
    Workload("gqa_single_frame_reuse", "GQA", "relocate_patch", num_layers=28, num_heads=4,
             head_dim=128, rope_offset=0, rope_dim=128, rope_base=1e6, num_streams=2,
             n_tokens=1024, n_chunks=1, rank=16, sigma=0.02, delta_range=(-4096, 8192),
             outlier_frac=0.05),
    Workload("sliding_window_survival", "GQA", "relocate", num_layers=36, num_heads=8,
             head_dim=128, rope_offset=0, rope_dim=128, rope_base=1e6, num_streams=2,
             n_tokens=1024, n_chunks=64, rank=0, page_size=16, delta_range=(1024, 16384),
             delta_negate=True),
    Workload("reorder_recall_rank32", "GQA", "reorder", num_layers=36, num_heads=8,
             head_dim=128, rope_offset=0, rope_dim=128, rope_base=1e6, num_streams=2,
             n_tokens=2048, n_chunks=32, rank=32, sigma=0.02, page_size=16),
    Workload("mla_reuse", "MLA", "relocate_patch", num_layers=27, num_heads=1,
             head_dim=576, rope_offset=512, rope_dim=64, rope_base=1e4, num_streams=1,
             n_tokens=4096, n_chunks=16, rank=32, sigma=0.02, page_size=64,
             delta_range=(-32768, 32768)),
]

# the workloads above by name
_BY_NAME = {w.name: w for w in CONFIGS}
TINY, SINGLE_FRAME, SURVIVAL, REORDER, MLA = (_BY_NAME[n] for n in (
    "tiny_mha_relocate_patch", "gqa_single_frame_reuse", "sliding_window_survival", "reorder_recall_rank32",
    "mla_reuse"))

# Recall at the reorder workload's shapes: 16 of the 32 stored chunks come back.
RECALL_CONFIG = replace(REORDER, name="recall_rank32", op="recall", n_chunks=16, n_store=32)


def by_name(name: str) -> Workload:
    for w in CONFIGS + [RECALL_CONFIG]:
        if w.name == name:
            return w
    raise KeyError(name)


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _gauss_bf16(shape, sigma, g, device) -> torch.Tensor:
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if sigma != 1.0:
        x.mul_(sigma)
    return x.to(torch.bfloat16)


def make_inputs(w: Workload, device="cpu", seed: int = 20261202) -> dict:
    """All inputs of one call of workload ``w`` as torch tensors on ``device``.

    Large tensors are drawn with a generator on ``device``; small index data
    (shifts, permutations, page tables, outlier columns) with a CPU generator,
    so they do not depend on the device.
    """
    gd = _gen(device, seed)
    gc = _gen("cpu", seed + 1)
    L, T, F, S = w.num_layers, w.n_tokens, w.row_width, w.num_streams
    ns, n = w.store_chunks, w.n_chunks

    src = []
    for s in range(S):
        x = torch.empty((ns, L, T, F), dtype=torch.bfloat16, device=device)
        for c in range(ns):
            x[c] = _gauss_bf16((L, T, F), 1.0, gd, device)
        if w.outlier_frac > 0:
            k = int(round(w.outlier_frac * F))
            for l in range(L):
                cols = torch.randperm(F, generator=gc)[:k].to(device)
                x[:, l, :, cols] *= 8
        src.append(x)

    u = v = None
    if w.rank > 0:
        u, v = [], []
        for s in range(S):
            u.append(_gauss_bf16((ns, L, T, w.rank), w.sigma, gd, device))
            v.append(_gauss_bf16((ns, L, F, w.rank), w.sigma, gd, device))

    out = dict(workload=w, src=src, u=u, v=v, page_size=w.page_size)

    canon_pos = None
    if w.canon_pos_range is not None:
        lo, hi = w.canon_pos_range
        canon_pos = torch.randint(lo, hi + 1, (ns,), generator=gc, dtype=torch.int64)
    out["canon_pos"] = canon_pos

    if w.op in ("relocate", "relocate_patch"):
        if w.delta_fixed is not None:
            delta = torch.full((n,), w.delta_fixed, dtype=torch.int64)
        else:
            lo, hi = w.delta_range
            delta = torch.randint(lo, hi + 1, (n,), generator=gc, dtype=torch.int64)
            if w.delta_negate:
                delta = -delta
        out["delta"] = delta
    elif w.op == "reorder":
        out["perm"] = torch.randperm(ns, generator=gc)[:n].to(torch.int32)
        out["base_pos"] = int(w.base_pos)
    elif w.op == "recall":
        out["chunk_ids"] = torch.randperm(ns, generator=gc)[:n].to(torch.int32)
        # each recalled chunk lands in a seeded window slot k*T
        slots = torch.randperm(max(n, ns), generator=gc)[:n].to(torch.int64)
        out["target_pos"] = slots * T + int(w.base_pos)
    else:
        raise ValueError(w.op)

    if w.page_size:
        needed = n * w.pages_per_chunk
        num_pages = int(math.ceil(1.25 * needed))
        pt = torch.randperm(num_pages, generator=gc)[:needed].reshape(n, w.pages_per_chunk)
        out["page_table"] = pt.to(torch.int32)
        out["num_pages"] = num_pages
        num_slots = num_pages * w.page_size
        out["dst_offset"] = None
    else:
        slack = w.contiguous_slack
        num_slots = n * T + 2 * slack
        perm = torch.randperm(n, generator=gc)
        offs = torch.randint(0, slack + 1, (1,), generator=gc, dtype=torch.int64)
        out["dst_offset"] = perm.to(torch.int64) * T + offs
        out["page_table"] = None
        out["num_pages"] = 0
    out["num_slots"] = num_slots

    for key in ("delta", "perm", "chunk_ids", "target_pos", "canon_pos", "page_table", "dst_offset"):
        if out.get(key) is not None:
            out[key] = out[key].to(device)

    pools = []
    for s in range(S):
        p = torch.empty((L, num_slots, F), dtype=torch.int16, device=device)
        p.fill_(SENTINEL_BITS)
        pools.append(p.view(torch.bfloat16))
    out["pool"] = pools
    return out


def bits(t: torch.Tensor) -> np.ndarray:
    """bfloat16 tensor (any device) -> numpy uint16 bit patterns on the host."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def small_workload(**kw) -> Workload:
    """A Workload with defaults suitable for quick tests; keywords override."""
    base = dict(name="small", family="GQA", op="relocate_patch", num_layers=2, num_heads=2,
                head_dim=64, rope_offset=0, rope_dim=64, rope_base=1e4, num_streams=2,
                n_tokens=80, n_chunks=2, rank=8, sigma=0.05, delta_range=(-500, 900))
    base.update(kw)
    return Workload(**base)


# ---------------------------------------------------------------------------
# Patch formation workloads (Kamera summary, section 2, "Patch application")
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class FormWorkload:
    """Inputs of one patch-formation call at a reuse workload's shapes.

    The forward-pass output KV(B|A) is not generated here (building it is the
    reuse equation): this module draws the canonical rows and shifts of
    ``base``, a deficit "signal" as bfloat16 factors with a decaying spectrum
    (columns of u_sig scaled by sigma0 * decay^i / sqrt(T), v_sig / sqrt(F),
    Gaussian, so that their product has singular values close to the
    spectrum), and the sketch test matrix omega [m + p, F] ~ N(0, 1).  The
    deficit the pages describe is concentrated in ~32 feature directions
    (section 3, "Deficit diagnosis"); signal_rank sets that count.

    views > 1 makes it an orbit-patch call (section 3, Reorder): the n chunks
    form one cached set, and view v places them in a seeded ordering (view 0
    in stored order) at consecutive slots of T tokens from position base_pos,
    so chunk i of view v is shifted by base_pos + slot * T from its canonical
    frame at 0.  Each view has its own token-side signal factors u_sig
    (n * views chunks, view v of chunk i at i * views + v) over the chunk's
    shared feature directions v_sig.
    """

    name: str
    base: Workload
    rank: int            # m
    oversample: int      # p
    power_iters: int     # q
    signal_rank: int
    sigma0: float
    decay: float
    views: int = 1       # orderings averaged by an orbit patch

    @property
    def blocks(self) -> int:
        b = self.base
        return b.n_chunks * b.num_layers * b.num_streams

    def row_bytes(self) -> int:
        """Canonical + target rows (bfloat16) one call consumes: every canonical
        row once and every view's target row once."""
        b = self.base
        return 2 * (1 + self.views) * self.blocks * b.n_tokens * b.row_width

    def factor_bytes(self) -> int:
        """The rank-m factors written (bfloat16): U (T x m) and V (F x m) per block."""
        b = self.base
        return 2 * self.rank * (b.n_tokens + b.row_width) * self.blocks

    def method_bytes(self) -> int:
        """The method's own data: every canonical row and every view's KV(B|A)
        row read once, the factors written once."""
        return self.row_bytes() + self.factor_bytes()

    def implementation_bytes(self) -> int:
        """What this implementation of randomized subspace iteration moves: the
        rows once to form the deficit, the deficit written once as bfloat16
        high and low parts (4 bytes per element), the passes reading it (2q + 1
        for one view, whose first product forms the deficit itself; 2q + 2 for
        several), plus the factors."""
        b = self.base
        elems = self.blocks * b.n_tokens * b.row_width
        reads = 2 * self.power_iters + (1 if self.views == 1 else 2)
        return self.row_bytes() + 4 * elems * (1 + reads) + self.factor_bytes()

    def sketch_flops(self) -> int:
        """Flops of the products with the deficit that randomized subspace
        iteration needs: 2q + 2 products of a T x F block with k = m + p
        columns (the range sketch, q power-iteration pairs and the final
        projection), 2 T F k flops each."""
        b = self.base
        k = self.rank + self.oversample
        return (2 * self.power_iters + 2) * 2 * b.n_tokens * b.row_width * k * self.blocks


FORM_CONFIGS = [
    FormWorkload("form_gqa_single_frame", replace(SINGLE_FRAME, name="form_gqa_single_frame", outlier_frac=0.0),
                 rank=16, oversample=16, power_iters=2, signal_rank=16, sigma0=20.0, decay=0.85),
    FormWorkload("form_mla", replace(MLA, name="form_mla", page_size=0), rank=32, oversample=16,
                 power_iters=2, signal_rank=32, sigma0=40.0, decay=0.9),
    # orbit patches of a cached set of 4 chunks at the reorder workload's
    # shapes, averaged over 4 sampled orderings
    FormWorkload("form_orbit_reorder", replace(REORDER, name="form_orbit_reorder", op="relocate_patch",
                                               n_chunks=4, page_size=0, delta_range=(0, 0)),
                 rank=32, oversample=16, power_iters=2, signal_rank=32, sigma0=40.0, decay=0.9, views=4),
]


def form_by_name(name: str) -> FormWorkload:
    for w in FORM_CONFIGS:
        if w.name == name:
            return w
    raise KeyError(name)


def make_form_inputs(fw: FormWorkload, device="cpu", seed: int = 20261203) -> dict:
    """Canonical rows, shifts, signal factors and omega of one formation call."""
    b = fw.base
    inp = make_inputs(replace(b, rank=0), device, seed)
    L, T, F, S, n = b.num_layers, b.n_tokens, b.row_width, b.num_streams, b.n_chunks
    gd = _gen(device, seed + 7)
    scale = torch.tensor([fw.sigma0 * fw.decay ** i for i in range(fw.signal_rank)], device=device)
    u_sig, v_sig = [], []
    for s in range(S):
        u = torch.randn((n, L, T, fw.signal_rank), generator=gd, device=device) * (scale / math.sqrt(T))
        v = torch.randn((n, L, F, fw.signal_rank), generator=gd, device=device) / math.sqrt(F)
        u_sig.append(u.to(torch.bfloat16))
        v_sig.append(v.to(torch.bfloat16))
    omega = _gauss_bf16((fw.rank + fw.oversample, F), 1.0, gd, device)
    delta = inp["delta"]
    if fw.views > 1:
        # orbit: per-view token-side factors over the chunk's feature directions
        u_sig = []
        for s in range(S):
            u = torch.randn((n * fw.views, L, T, fw.signal_rank), generator=gd, device=device)
            u_sig.append((u * (scale / math.sqrt(T))).to(torch.bfloat16))
        gc = _gen("cpu", seed + 8)
        delta = torch.empty((n, fw.views), dtype=torch.int64)
        for v in range(fw.views):
            perm = torch.arange(n) if v == 0 else torch.randperm(n, generator=gc)
            for slot, i in enumerate(perm.tolist()):
                delta[i, v] = b.base_pos + slot * T
        delta = delta.to(device)
    return dict(workload=fw, src=inp["src"], delta=delta, u_sig=u_sig, v_sig=v_sig, omega=omega)


# ---------------------------------------------------------------------------
# Decode attention over a reused context (relocated and patched on read)
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class DecodeWorkload:
    """One decode step of attention over a reused context at a reuse workload's shapes.

    ``base`` gives the canonical store (n_store = n_chunks chunks of T tokens,
    every layer) and the patch rank and spread.  Each of num_seqs sequences
    attends all stored chunks, placed in a seeded order at consecutive slots
    of T tokens from position 0 (the reorder placement: chunk at slot k is
    shifted by k * T from its canonical frame at 0).  Queries are N(0, 1),
    one per (layer, sequence, query head), as bfloat16.  num_q_heads follows
    the backbone: 32 query heads over 8 KV heads of 128 (G = 4) for the GQA
    shapes; 16 absorbed query heads, 576 wide, over the one MLA row.

    pool_tokens > 0: each sequence also attends that many of its own tokens
    in a paged pool (pages of pool_page tokens, a seeded permutation of
    ceil(1.25 x needed) pages, rows N(0, 1) as bfloat16): the engine's cache
    next to the reused chunks.
    """

    name: str
    base: Workload
    num_q_heads: int
    num_seqs: int = 1
    qk_dim: int = 0      # dimension the softmax scale is taken over (0: head_dim)
    pool_tokens: int = 0
    pool_page: int = 16

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.qk_dim or self.base.head_dim)

    @property
    def value_dim(self) -> int:
        b = self.base
        return b.head_dim if b.num_streams == 2 else b.rope_offset

    def context_tokens(self) -> int:
        return self.base.n_chunks * self.base.n_tokens + self.pool_tokens

    @property
    def pool_pages(self) -> int:
        return -(-self.pool_tokens // self.pool_page)

    def layer_bytes(self) -> int:
        """Bytes one layer's attention must read: every sequence's K and V rows
        once (reused and pooled), the patch factors of its chunks once, its
        block-table row, the queries; and the output written (fp32)."""
        b = self.base
        S = b.num_streams
        rows = 2 * S * self.context_tokens() * b.row_width * self.num_seqs
        factors = 2 * S * b.rank * (b.n_tokens + b.row_width) * b.n_chunks * self.num_seqs
        table = 4 * self.pool_pages * self.num_seqs
        qo = self.num_seqs * self.num_q_heads * (2 * b.head_dim + 4 * self.value_dim)
        return rows + factors + table + qo

    def step_bytes(self) -> int:
        return self.layer_bytes() * self.base.num_layers


DECODE_CONFIGS = [
    DecodeWorkload("decode_reorder_rank32", replace(REORDER, name="decode_reorder_rank32", op="relocate_patch",
                                                   page_size=0, delta_range=(0, 0)), num_q_heads=32),
    # MLA backbone: 16 query heads over the one joint row; softmax scale over
    # the 128 + 64 dimensions of a query-key head before absorption
    DecodeWorkload("decode_mla_rank32", replace(MLA, name="decode_mla_rank32", page_size=0,
                                               delta_range=(0, 0)), num_q_heads=16, qk_dim=192),
    # the same 65,536-token contexts, half reused chunks relocated on read and
    # half the sequence's own tokens in the engine's paged pool
    DecodeWorkload("decode_paged_reorder_rank32", replace(REORDER, name="decode_paged_reorder_rank32",
                                                         op="relocate_patch", n_chunks=16, page_size=0,
                                                         delta_range=(0, 0)),
                   num_q_heads=32, pool_tokens=32768, pool_page=16),
    DecodeWorkload("decode_paged_mla_rank32", replace(MLA, name="decode_paged_mla_rank32", n_chunks=8,
                                                     page_size=0, delta_range=(0, 0)),
                   num_q_heads=16, qk_dim=192, pool_tokens=32768, pool_page=64),
]


def decode_by_name(name: str) -> DecodeWorkload:
    for w in DECODE_CONFIGS:
        if w.name == name:
            return w
    raise KeyError(name)


def make_decode_inputs(dw: DecodeWorkload, device="cpu", seed: int = 20261204) -> dict:
    """Store rows, patch factors, contexts and queries of one decode step."""
    b = dw.base
    inp = make_inputs(b, device, seed)
    gc = _gen("cpu", seed + 9)
    gd = _gen(device, seed + 10)
    n, T = b.n_chunks, b.n_tokens
    ids, deltas, se = [], [], [0]
    for _ in range(dw.num_seqs):
        perm = torch.randperm(n, generator=gc)
        for slot, c in enumerate(perm.tolist()):
            ids.append(c)
            deltas.append(slot * T)
        se.append(len(ids))
    q = _gauss_bf16((b.num_layers, dw.num_seqs, dw.num_q_heads, b.head_dim), 1.0, gd, device)
    out = dict(workload=dw, src=inp["src"], u=inp["u"], v=inp["v"], q=q,
               seq_entries=torch.tensor(se, dtype=torch.int32, device=device),
               chunk_ids=torch.tensor(ids, dtype=torch.int32, device=device),
               delta=torch.tensor(deltas, dtype=torch.int64, device=device),
               pool=None, block_table=None, pool_tokens=None)
    if dw.pool_tokens:
        P, need = dw.pool_page, dw.pool_pages * dw.num_seqs
        num_pages = int(math.ceil(1.25 * need))
        table = torch.randperm(num_pages, generator=gc)[:need].reshape(dw.num_seqs, dw.pool_pages)
        pool = []
        for s in range(b.num_streams):
            x = torch.empty((b.num_layers, num_pages * P, b.row_width), dtype=torch.bfloat16, device=device)
            for l in range(b.num_layers):
                x[l] = _gauss_bf16((num_pages * P, b.row_width), 1.0, gd, device)
            pool.append(x)
        out.update(pool=pool, block_table=table.to(torch.int32).to(device),
                   pool_tokens=torch.full((dw.num_seqs,), dw.pool_tokens, dtype=torch.int32, device=device))
    return out


__all__ = ["Workload", "CONFIGS", "TINY", "SINGLE_FRAME", "SURVIVAL", "REORDER", "MLA", "RECALL_CONFIG", "SENTINEL_BITS", "by_name", "make_inputs",
           "bits", "small_workload", "ROPE_HALF", "ROPE_INTERLEAVED", "FormWorkload", "FORM_CONFIGS",
           "form_by_name", "make_form_inputs", "DecodeWorkload", "DECODE_CONFIGS", "decode_by_name",
           "make_decode_inputs"]


# ---------------------------------------------------------------------------
# Variable-length chunks: one packed store whose chunks differ in length
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class VarlenWorkload:
    """Chunks of seeded lengths in a packed store.

    ``base`` fixes the row shape, the op ("relocate", "relocate_patch" or
    "recall"), rank, factor scale, page size, shift range and counts
    (n_store, n_chunks); its n_tokens is ignored.  Chunk lengths are uniform
    over the multiples of ``len_multiple`` in ``len_range`` (inclusive).  For
    "recall" the output is every chosen chunk in a seeded order, each placed
    right after the previous one from base_pos on (a reorder of variable-length
    chunks).  Store chunk c's rows sit at rows [row_offset[c], + L*T_c), layer
    by layer, in store order; U rows follow the same order.
    """
    name: str
    base: Workload
    len_range: tuple
    len_multiple: int = 16

    @property
    def max_tokens(self) -> int:
        return self.len_range[1]

    @property
    def family(self) -> str:
        return self.base.family


VARLEN_CONFIGS = [
    # the reorder/recall row shapes (GQA, 36 layers, 8 KV heads x 128, rank 32,
    # 16-token pages) with 32 chunks of 256..3840 tokens (mean 2048, about the
    # 65,536-token context of the fixed-length workload), all 32 recalled in a
    # seeded order
    VarlenWorkload("varlen_recall_rank32", replace(REORDER, name="varlen_recall_rank32", op="recall",
                                                   n_chunks=32, n_store=32), len_range=(256, 3840)),
    # sliding-window survival (m = 0) over 64 chunks of 256..1792 tokens (mean
    # 1024, the fixed-length workload's 65,536-token window)
    VarlenWorkload("varlen_survival", replace(SURVIVAL, name="varlen_survival"), len_range=(256, 1792)),
    # recall from a pinned host store: 8 of 16 stored chunks of 256..3840 tokens
    VarlenWorkload("varlen_recall_host_rank32", replace(REORDER, name="varlen_recall_host_rank32", op="recall",
                                                        n_chunks=8, n_store=16), len_range=(256, 3840)),
]


def varlen_by_name(name: str) -> VarlenWorkload:
    for w in VARLEN_CONFIGS:
        if w.name == name:
            return w
    raise KeyError(name)


def varlen_bytes(vw: VarlenWorkload, lengths) -> int:
    """Algorithmic bytes of one call whose output chunks have ``lengths``
    tokens: rows read + written, factors read once
    per (output chunk, layer, stream), page-table rows / offsets and the
    per-chunk length, offset and shift inputs."""
    w = vw.base
    tok = int(sum(int(t) for t in lengths))
    S, L, F, m = w.num_streams, w.num_layers, w.row_width, w.rank
    kv = 2 * 2 * S * L * tok * F
    fac = 2 * m * (tok + len(lengths) * F) * S * L
    ppc = -(-vw.max_tokens // w.page_size) if w.page_size else 0
    idx = len(lengths) * ((4 * ppc if w.page_size else 8) + 8 + 8 + 4)
    return kv + fac + idx


def make_varlen_inputs(vw: VarlenWorkload, device="cpu", seed: int = 20261205, index_only: bool = False) -> dict:
    """All inputs of one variable-length call as torch tensors on ``device``.

    index_only: skip the rows, factors and pools (the index data -- lengths,
    offsets, shifts, targets, page table -- come out the same).

    Keys: src (per stream [total_rows, F]), row_offset (int64 [n_store]),
    n_tokens (int32 [n_store]), max_tokens, u (per stream [total_rows, m]) and
    v (per stream [n_store, L, F, m]) or None, canon_pos, then per op: delta
    (relocate*) or chunk_ids + target_pos (recall); out_ids (the store chunk of
    every output chunk); page_table ([n, ceil(max_tokens/P)] int32, entries a
    chunk does not use are -1) or dst_offset; pool (sentinel-filled), num_slots.
    """
    w = vw.base
    gd = _gen(device, seed)
    gc = _gen("cpu", seed + 1)
    L, F, S = w.num_layers, w.row_width, w.num_streams
    ns, n = w.store_chunks, w.n_chunks
    lo, hi = vw.len_range
    q = vw.len_multiple
    lengths = (torch.randint(lo // q, hi // q + 1, (ns,), generator=gc, dtype=torch.int64) * q).tolist()
    row_offset, r = [], 0
    for t in lengths:
        row_offset.append(r)
        r += L * t
    total_rows = r

    src = []
    for s in range(0 if index_only else S):
        x = torch.empty((total_rows, F), dtype=torch.bfloat16, device=device)
        step = 1 << 16
        for a in range(0, total_rows, step):
            b = min(total_rows, a + step)
            x[a:b] = _gauss_bf16((b - a, F), 1.0, gd, device)
        src.append(x)
    u = v = None
    if w.rank > 0 and not index_only:
        u = [_gauss_bf16((total_rows, w.rank), w.sigma, gd, device) for _ in range(S)]
        v = [_gauss_bf16((ns, L, F, w.rank), w.sigma, gd, device) for _ in range(S)]

    out = dict(workload=vw, src=src, u=u, v=v, page_size=w.page_size, lengths=lengths,
               max_tokens=vw.max_tokens, total_rows=total_rows,
               row_offset=torch.tensor(row_offset, dtype=torch.int64),
               n_tokens=torch.tensor(lengths, dtype=torch.int32))
    canon_pos = None
    if w.canon_pos_range is not None:
        clo, chi = w.canon_pos_range
        canon_pos = torch.randint(clo, chi + 1, (ns,), generator=gc, dtype=torch.int64)
    out["canon_pos"] = canon_pos

    if w.op in ("relocate", "relocate_patch"):
        out_ids = list(range(n))
        dlo, dhi = w.delta_range if w.delta_range is not None else (w.delta_fixed, w.delta_fixed)
        delta = torch.randint(dlo, dhi + 1, (n,), generator=gc, dtype=torch.int64)
        out["delta"] = -delta if w.delta_negate else delta
    elif w.op == "recall":
        out_ids = torch.randperm(ns, generator=gc)[:n].tolist()
        targets, pos = [], int(w.base_pos)
        for c in out_ids:
            targets.append(pos)
            pos += lengths[c]
        out["chunk_ids"] = torch.tensor(out_ids, dtype=torch.int32)
        out["target_pos"] = torch.tensor(targets, dtype=torch.int64)
    else:
        raise ValueError(w.op)
    out["out_ids"] = out_ids
    out_len = [lengths[c] for c in out_ids]
    out["out_lengths"] = out_len

    if w.page_size:
        P = w.page_size
        ppc = -(-vw.max_tokens // P)
        need = [-(-t // P) for t in out_len]
        num_pages = max(1, int(math.ceil(1.25 * sum(need))))
        pages = torch.randperm(num_pages, generator=gc)[:sum(need)].tolist()
        pt = torch.full((n, ppc), -1, dtype=torch.int32)
        k = 0
        for i, c in enumerate(need):
            pt[i, :c] = torch.tensor(pages[k:k + c], dtype=torch.int32)
            k += c
        out["page_table"] = pt
        out["dst_offset"] = None
        num_slots = num_pages * P
    else:
        slack = w.contiguous_slack
        order = torch.randperm(n, generator=gc).tolist()
        offs = [0] * n
        pos = int(torch.randint(0, slack + 1, (1,), generator=gc))
        for i in order:
            offs[i] = pos
            pos += out_len[i]
        out["dst_offset"] = torch.tensor(offs, dtype=torch.int64)
        out["page_table"] = None
        num_slots = pos + slack
    out["num_slots"] = num_slots

    for key in ("row_offset", "n_tokens", "delta", "chunk_ids", "target_pos", "canon_pos", "page_table",
                "dst_offset"):
        if out.get(key) is not None:
            out[key] = out[key].to(device)
    pools = []
    for s in range(0 if index_only else S):
        p = torch.empty((L, num_slots, F), dtype=torch.int16, device=device)
        p.fill_(SENTINEL_BITS)
        pools.append(p.view(torch.bfloat16))
    out["pool"] = pools
    out["algorithmic_bytes"] = varlen_bytes(vw, out_len)
    return out
