"""Parity harness: runs a workload through the HIP library and through the CPU
oracle on the same seeded inputs, and compares them.

Used by the GPU tests and by ``__graft_entry__.smoke()``.  The comparison bar:
  * bit-exact for the scatter map, the sentinel of untouched slots, and
    elements neither the rotation nor the patch touches (values and c_KV at
    m = 0);
  * otherwise the stated bar -- per element, at most 1 bfloat16 ulp from the
    oracle's single rounding OR |gpu - y| <= 4e-3 * max|y| over the (chunk,
    layer, stream) block, y being the oracle's float64 value -- tightened to
    what the kernels' arithmetic can guarantee, so that a small systematic
    error cannot hide under the absolute clause (see compare_block).
"""

from __future__ import annotations

import numpy as np
import torch

import position_invariant_kv_amd as kam
from oracle import kamera_oracle as ko
from workloads import SENTINEL_BITS, Workload, bits

REL_TOL = 4e-3              # the stated bar's absolute clause (x max|y| of the block)

# How far the GPU's float32 value can be from y.  Rotation: cos/sin carry
# <= 6e-8 absolute error (plus <= 1.5e-8 rad of phase at |delta| <= 1e7), and
# each product and the fused add round once (2^-24 relative), so
# |gpu32 - y| <= ~1.3e-7 * (|a| + |b|) <= 2.6e-7 * max|x|.  The rank-m patch
# adds m exact bf16 products in float32: far smaller at sigma <= 1.  Rounding
# the float32 value to bfloat16 then lands within 1 ulp of RNE(y) whenever that
# error is below one ulp of y, which is > 2^-8 |y|: i.e. for every |y| above
# ~2^-14 max|x|.  Hence, with a 16x margin (max|y| standing in for max|x|):
STRICT_FLOOR = 2.0 ** -10     # |y| >= STRICT_FLOOR * max|y|: within 1 ulp, no exception
NEAR_ZERO_TOL = 2.0 ** -16    # below it: 1 ulp, or |gpu - y| <= NEAR_ZERO_TOL * max|y|
# (the float32 error plus half a bf16 ulp of a value under the floor is
# < 2^-18 max|y|; 2^-16 leaves a 4x margin and is 260x tighter than 4e-3)
MAX_WIDE = 1e-3               # at most this fraction of a block (plus 8) may be > 1 ulp off
# An element can round to the other side of RNE(y) only when y lies within
# the float32 error of a rounding midpoint.  For N(0,1)-like rows that is a
# fraction ~2e-5 of a block (measured with a float32 emulation of the kernels
# on the single-frame block, and ~6e-5 on the GPU's smoke case); a systematic
# error (an angle formed as a float32 product at |delta| >= 4096, a dropped
# patch) moves far more elements.
MAX_DIFF = 2e-3               # at most this fraction of a block (plus 8) may differ at all


def layouts(w: Workload):
    o = ko.Layout(w.num_layers, w.num_heads, w.head_dim, w.rope_offset, w.rope_dim,
                  w.rope_base, w.num_streams, w.rope_style)
    g = kam.Layout(w.num_layers, w.num_heads, w.head_dim, w.rope_offset, w.rope_dim,
                   w.rope_base, w.num_streams, w.rope_style)
    return o, g


def prepare_gpu(w: Workload, inp: dict, error_word=None, stream=None, page_order="auto") -> "kam.Call":
    """A prepared call of the workload's entry point through the C ABI.
    page_order: "auto" lets a paged call write the pool in page-address order,
    None keeps the page-table order."""
    _, lay = layouts(w)
    kw = dict(page_size=w.page_size, page_table=inp["page_table"], dst_offset=inp["dst_offset"],
              canon_pos=inp["canon_pos"], error_word=error_word, page_order=page_order, stream=stream)
    if w.op == "relocate":
        return kam.prepare_relocate(lay, inp["src"], inp["delta"], inp["pool"], **kw)
    if w.op == "relocate_patch":
        return kam.prepare_relocate_patch(lay, inp["src"], inp["delta"], inp["u"], inp["v"], inp["pool"], **kw)
    if w.op == "reorder":
        return kam.prepare_reorder(lay, inp["src"], inp["perm"], inp["base_pos"], inp["pool"], u=inp["u"],
                                   v=inp["v"], **kw)
    if w.op == "recall":
        return kam.prepare_recall(lay, inp["src"], inp["chunk_ids"], inp["target_pos"], inp["pool"],
                                  u=inp["u"], v=inp["v"], **kw)
    raise ValueError(w.op)


def run_gpu(w: Workload, inp: dict, error_word=None, stream=None, page_order="auto"):
    """One call of the workload's entry point through the C ABI."""
    prepare_gpu(w, inp, error_word=error_word, stream=stream, page_order=page_order)()


def chunk_plan(w: Workload, inp: dict):
    """(store chunk id, shift) of every output chunk, from the oracle's rules."""
    canon = None if inp["canon_pos"] is None else inp["canon_pos"].cpu().tolist()
    if w.op in ("relocate", "relocate_patch"):
        ids = list(range(w.n_chunks))
        ds = ko.deltas_relocate(inp["delta"].cpu().tolist())
    elif w.op == "reorder":
        ids = inp["perm"].cpu().tolist()
        ds = ko.deltas_reorder(ids, inp["base_pos"], w.n_tokens, canon)
    else:
        ids = inp["chunk_ids"].cpu().tolist()
        ds = ko.deltas_recall(ids, inp["target_pos"].cpu().tolist(), canon)
    return ids, ds


def slots_of(w: Workload, inp: dict, i: int) -> np.ndarray:
    pt = None if inp["page_table"] is None else inp["page_table"].cpu().numpy()
    off = None if inp["dst_offset"] is None else inp["dst_offset"].cpu().numpy()
    return ko.dest_slots(i, w.n_tokens, w.page_size, pt, off)


def ordinal(b: np.ndarray) -> np.ndarray:
    """bfloat16 bits -> integers that are monotone in the value (+0 == -0)."""
    b = b.astype(np.int32)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def expected_block(w: Workload, inp: dict, i: int, l: int, s: int, plan=None):
    """Oracle bits and float64 values of output chunk i, layer l, stream s."""
    o_lay, _ = layouts(w)
    ids, ds = plan if plan is not None else chunk_plan(w, inp)
    c, d = ids[i], ds[i]
    x = bits(inp["src"][s][c, l])
    u = v = None
    if w.rank > 0:
        u, v = bits(inp["u"][s][c, l]), bits(inp["v"][s][c, l])
    want = ko.reuse_block_bits(x, d, u, v, o_lay, rotate=(s == 0))
    y = ko.reuse_f64(ko.bf16_bits_to_f64(x), d,
                     None if u is None else ko.bf16_bits_to_f64(u),
                     None if v is None else ko.bf16_bits_to_f64(v), o_lay, rotate=(s == 0))
    touched = np.ones(w.row_width, bool) if w.rank > 0 else (
        ko.rope_touched_mask(o_lay) if s == 0 else np.zeros(w.row_width, bool))
    return want, y, touched, x


def block_errors(got: np.ndarray, want: np.ndarray, y: np.ndarray, touched: np.ndarray) -> list[str]:
    """Every way the block misses the bar (an empty list: it passes).

    * copied columns (touched False): bit for bit;
    * |y| >= STRICT_FLOOR * max|y|: within 1 ulp of the oracle's rounding;
    * below that: within 1 ulp, or |gpu - y| <= NEAR_ZERO_TOL * max|y|
      (near-cancellation values, whose ulp is finer than the float32 error);
    * at most MAX_WIDE * size + 8 elements more than 1 ulp off, and at most
      MAX_DIFF * size + 8 not bit-identical;
    * and every element within the stated bar (1 ulp or 4e-3 * max|y|), which
      the rules above imply.
    """
    errs = []
    if got.shape != want.shape:
        return [f"shape {got.shape} != {want.shape}"]
    if (~touched).any():
        bad = got[:, ~touched] != want[:, ~touched]
        if bad.any():
            errs.append(f"{int(bad.sum())} copied elements differ")
    ulp = np.abs(ordinal(got) - ordinal(want))
    g = ko.bf16_bits_to_f64(got)
    ay = np.abs(y)
    scale = float(np.max(ay)) if y.size else 0.0
    err = np.abs(g - y)
    strict = ay >= STRICT_FLOOR * scale
    bad_strict = strict & (ulp > 1)
    bad_small = ~strict & (ulp > 1) & ~(err <= NEAR_ZERO_TOL * scale)
    bad_bar = ~((ulp <= 1) | (err <= REL_TOL * scale))
    wide = int((ulp > 1).sum())
    diff = int((ulp > 0).sum())

    def detail(mask):
        idx = np.argwhere(mask)[:5]
        return [(tuple(int(k) for k in t), int(got[tuple(t)]), int(want[tuple(t)]), float(y[tuple(t)]))
                for t in idx]

    if bad_strict.any():
        errs.append(f"{int(bad_strict.sum())} elements with |y| >= 2^-10 max|y| are > 1 ulp off, "
                    f"e.g. {detail(bad_strict)}")
    if bad_small.any():
        errs.append(f"{int(bad_small.sum())} near-zero elements are > 1 ulp and > 2^-16 max|y| off, "
                    f"e.g. {detail(bad_small)}")
    if bad_bar.any():
        errs.append(f"{int(bad_bar.sum())} elements outside 1 ulp / 4e-3 max|y|, e.g. {detail(bad_bar)}")
    if wide > MAX_WIDE * ulp.size + 8:
        errs.append(f"{wide} of {ulp.size} elements are > 1 ulp off (cap {MAX_WIDE * ulp.size + 8:.0f})")
    if diff > MAX_DIFF * ulp.size + 8:
        errs.append(f"{diff} of {ulp.size} elements differ from the oracle's rounding "
                    f"(cap {MAX_DIFF * ulp.size + 8:.0f})")
    return errs


def compare_block(got: np.ndarray, want: np.ndarray, y: np.ndarray, touched: np.ndarray, where=""):
    """Assert the bar above (block_errors); return (max ulp, fraction bit-identical)."""
    errs = block_errors(got, want, y, touched)
    if errs:
        raise AssertionError(f"{where}: " + "; ".join(errs))
    ulp = np.abs(ordinal(got) - ordinal(want))
    return int(ulp.max()) if ulp.size else 0, float((ulp == 0).mean()) if ulp.size else 1.0


def check_blocks(w: Workload, inp: dict, blocks, where=""):
    """Compare the listed (i, l, s) output blocks with the oracle."""
    plan = chunk_plan(w, inp)
    stats = []
    for (i, l, s) in blocks:
        slots = torch.from_numpy(slots_of(w, inp, i)).to(inp["pool"][s].device)
        got = bits(inp["pool"][s][l].index_select(0, slots))
        want, y, touched, _ = expected_block(w, inp, i, l, s, plan)
        stats.append(compare_block(got, want, y, touched, f"{where} block (i={i}, l={l}, s={s})"))
    return stats


def written_mask(w: Workload, inp: dict, num_slots: int, device) -> torch.Tensor:
    mask = torch.zeros(num_slots, dtype=torch.bool, device=device)
    for i in range(w.n_chunks):
        mask[torch.from_numpy(slots_of(w, inp, i)).to(device)] = True
    return mask


def check_untouched_slots(w: Workload, inp: dict):
    """Every slot no output token maps to still holds the sentinel (all layers/streams)."""
    pool = inp["pool"][0]
    mask = written_mask(w, inp, pool.shape[1], pool.device)
    for s in range(w.num_streams):
        p = inp["pool"][s].view(torch.int16)
        rest = p[:, ~mask]
        assert bool((rest == SENTINEL_BITS).all()), f"stream {s}: an untouched slot was written"
        got = p[:, mask]
        assert not bool((got == SENTINEL_BITS).all(dim=-1).any()), f"stream {s}: a target slot was not written"


def check_copy_stream(w: Workload, inp: dict, s: int, cols=None):
    """At m = 0, elements the rotation does not touch are byte copies: check the
    whole stream on the device (any size)."""
    ids, _ = chunk_plan(w, inp)
    src, pool = inp["src"][s].view(torch.int16), inp["pool"][s].view(torch.int16)
    for i, c in enumerate(ids):
        slots = torch.from_numpy(slots_of(w, inp, i)).to(pool.device)
        got = pool.index_select(1, slots)                    # [L, T, F]
        want = src[c]
        if cols is not None:
            got, want = got[..., cols], want[..., cols]
        assert torch.equal(got, want), f"stream {s} chunk {i}: copy is not bit-exact"
