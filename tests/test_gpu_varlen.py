"""GPU parity of the variable-length entry points (kamera_relocate_patch_varlen,
kamera_recall_varlen) against the oracle's reconstruct_varlen.

The bar is the one of the fixed-length parity tests (tests/harness.py):
bit-exact scatter map, sentinel and copied elements; otherwise within 1 bf16
ulp of the oracle's single rounding or 4e-3 of the block's max|y|.  Chunk
lengths are seeded and ragged (any length, including tails shorter than a
page or a 32-token tile), so every case spans several tiles and tails.
"""

import random
from dataclasses import replace

import numpy as np
import pytest
import torch

import position_invariant_kv_amd as kam
from oracle import kamera_oracle as ko
from tests import harness as H
from workloads import (SENTINEL_BITS, VarlenWorkload, bits, make_inputs, make_varlen_inputs, small_workload,
                       varlen_by_name)

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-varlen] {msg}", flush=True)


def run_varlen(vw, inp, error_word=None):
    w = vw.base
    _, lay = H.layouts(w)
    kw = dict(u=inp["u"], v=inp["v"], page_size=w.page_size, page_table=inp["page_table"],
              dst_offset=inp["dst_offset"], canon_pos=inp["canon_pos"], error_word=error_word)
    if w.op == "recall":
        kam.recall_varlen(lay, inp["src"], inp["row_offset"], inp["n_tokens"], inp["max_tokens"], inp["chunk_ids"],
                          inp["target_pos"], inp["pool"], **kw)
    else:
        kam.relocate_patch_varlen(lay, inp["src"], inp["row_offset"], inp["n_tokens"], inp["max_tokens"],
                                  inp["delta"], inp["pool"], **kw)


def plan(vw, inp):
    w = vw.base
    ids = list(inp["out_ids"])
    if w.op == "recall":
        canon = None if inp["canon_pos"] is None else inp["canon_pos"].cpu().tolist()
        return ids, ko.deltas_recall(ids, inp["target_pos"].cpu().tolist(), canon)
    return ids, ko.deltas_relocate(inp["delta"].cpu().tolist())


def slots_of(vw, inp, i, T):
    pt = None if inp["page_table"] is None else inp["page_table"].cpu().numpy()
    off = None if inp["dst_offset"] is None else inp["dst_offset"].cpu().numpy()
    return ko.dest_slots(i, T, vw.base.page_size, pt, off)


def check_blocks(vw, inp, blocks, where):
    w = vw.base
    o_lay, _ = H.layouts(w)
    ids, ds = plan(vw, inp)
    lengths = inp["lengths"]
    ro = inp["row_offset"].cpu().tolist()
    for (i, l, s) in blocks:
        c, d = ids[i], ds[i]
        T = lengths[c]
        if T == 0:
            continue
        rows = slice(ro[c] + l * T, ro[c] + (l + 1) * T)
        x = bits(inp["src"][s][rows])
        u = v = None
        if w.rank > 0:
            u, v = bits(inp["u"][s][rows]), bits(inp["v"][s][c, l])
        want = ko.reuse_block_bits(x, d, u, v, o_lay, rotate=(s == 0))
        y = ko.reuse_f64(ko.bf16_bits_to_f64(x), d, None if u is None else ko.bf16_bits_to_f64(u),
                         None if v is None else ko.bf16_bits_to_f64(v), o_lay, rotate=(s == 0))
        touched = np.ones(w.row_width, bool) if w.rank > 0 else (
            ko.rope_touched_mask(o_lay) if s == 0 else np.zeros(w.row_width, bool))
        sl = torch.from_numpy(slots_of(vw, inp, i, T)).to(inp["pool"][s].device)
        got = bits(inp["pool"][s][l].index_select(0, sl))
        H.compare_block(got, want, y, touched, f"{where} block (i={i}, l={l}, s={s})")


def check_untouched(vw, inp, skip=()):
    """Slots of no (kept) output token hold the sentinel; every target slot was written."""
    pool = inp["pool"][0]
    lengths = inp["lengths"]
    mask = torch.zeros(pool.shape[1], dtype=torch.bool, device=pool.device)
    for i, c in enumerate(inp["out_ids"]):
        if i in skip:
            continue
        mask[torch.from_numpy(slots_of(vw, inp, i, lengths[c])).to(pool.device)] = True
    for s in range(vw.base.num_streams):
        p = inp["pool"][s].view(torch.int16)
        assert bool((p[:, ~mask] == SENTINEL_BITS).all()), f"stream {s}: a slot outside the chunks was written"
        assert not bool((p[:, mask] == SENTINEL_BITS).all(dim=-1).any()), f"stream {s}: a target slot was not written"


def all_blocks(vw):
    w = vw.base
    return [(i, l, s) for i in range(w.n_chunks) for l in range(w.num_layers) for s in range(w.num_streams)]


CASES = {
    # name: (base workload keywords, length range, length multiple)
    "gqa_recall_paged_m16": (dict(op="recall", n_store=6, n_chunks=5, rank=16, page_size=16,
                                  canon_pos_range=(0, 3000)), (1, 100), 1),
    "gqa_relocate_patch_contiguous_m8": (dict(op="relocate_patch", n_store=4, n_chunks=4, rank=8), (0, 130), 1),
    "gqa_survival_m0_paged": (dict(op="relocate", n_store=5, n_chunks=5, rank=0, page_size=16,
                                   delta_range=(64, 4000), delta_negate=True), (16, 160), 16),
    "gqa_m0_interleaved_contiguous": (dict(op="relocate", n_store=3, n_chunks=3, rank=0,
                                           rope_style=1), (3, 90), 1),
    "gqa_recall_m32_wide_rows": (dict(op="recall", num_heads=4, head_dim=128, rope_dim=128, rope_base=1e6,
                                      n_store=4, n_chunks=3, rank=32, sigma=0.02, page_size=32), (20, 150), 1),
    "mla_relocate_patch_paged64": (dict(op="relocate_patch", family="MLA", num_heads=1, head_dim=576,
                                        rope_offset=512, rope_dim=64, num_streams=1, n_store=3, n_chunks=3,
                                        rank=8, page_size=64, delta_range=(-30000, 30000)), (1, 200), 1),
    "mla_m0_paged64": (dict(op="relocate", family="MLA", num_heads=1, head_dim=576, rope_offset=512,
                            rope_dim=64, num_streams=1, n_store=3, n_chunks=3, rank=0, page_size=64,
                            delta_range=(-30000, 30000)), (64, 256), 64),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_varlen_full_parity(name):
    kw, lr, q = CASES[name]
    vw = VarlenWorkload(name, small_workload(name=name, **kw), len_range=lr, len_multiple=q)
    inp = make_varlen_inputs(vw, "cuda", seed=400 + len(name))
    _say(f"{name}: lengths {inp['lengths']} out {inp['out_ids']}")
    ew = torch.zeros(1, dtype=torch.int32, device="cuda")
    run_varlen(vw, inp, error_word=ew)
    torch.cuda.synchronize()
    assert int(ew.item()) == 0
    check_blocks(vw, inp, all_blocks(vw), name)
    check_untouched(vw, inp)


def test_zero_length_chunks_write_nothing():
    base = small_workload(op="relocate_patch", n_store=4, n_chunks=4, rank=8, page_size=16)
    vw = VarlenWorkload("zero", base, len_range=(1, 60), len_multiple=1)
    inp = make_varlen_inputs(vw, "cuda", seed=9)
    # chunks 1 and 3 become empty (their rows stay where they are, unused)
    nt = inp["n_tokens"].clone()
    nt[1] = 0
    nt[3] = 0
    inp["n_tokens"] = nt
    inp["lengths"] = nt.cpu().tolist()
    ew = torch.zeros(1, dtype=torch.int32, device="cuda")
    run_varlen(vw, inp, error_word=ew)
    torch.cuda.synchronize()
    assert int(ew.item()) == 0
    check_blocks(vw, inp, all_blocks(vw), "zero-length")
    check_untouched(vw, inp, skip=(1, 3))


@pytest.mark.parametrize("op,rank,page_size", [("recall", 16, 16), ("relocate", 0, 16), ("relocate_patch", 8, 0)])
def test_equal_lengths_match_the_fixed_length_call(op, rank, page_size):
    # the packed store of equal-length chunks is the fixed store's own memory
    w = small_workload(op=op, n_tokens=72, n_chunks=3, n_store=4 if op == "recall" else 3, rank=rank,
                       page_size=page_size, canon_pos_range=(0, 800))
    inp = make_inputs(w, "cuda", seed=21)
    pool0 = [p.clone() for p in inp["pool"]]
    H.run_gpu(w, inp, page_order=None)
    ns, L, T, F = inp["src"][0].shape
    _, lay = H.layouts(w)
    packed = [x.reshape(ns * L * T, F) for x in inp["src"]]
    u = None if inp["u"] is None else [x.reshape(ns * L * T, rank) for x in inp["u"]]
    ro = torch.arange(ns, dtype=torch.int64, device="cuda") * (L * T)
    nt = torch.full((ns,), T, dtype=torch.int32, device="cuda")
    kw = dict(u=u, v=inp["v"], page_size=page_size, page_table=inp["page_table"], dst_offset=inp["dst_offset"],
              canon_pos=inp["canon_pos"])
    if op == "recall":
        kam.recall_varlen(lay, packed, ro, nt, T, inp["chunk_ids"], inp["target_pos"], pool0, **kw)
    else:
        kam.relocate_patch_varlen(lay, packed, ro, nt, T, inp["delta"], pool0, **kw)
    torch.cuda.synchronize()
    for s in range(w.num_streams):
        assert torch.equal(pool0[s].view(torch.int16), inp["pool"][s].view(torch.int16)), f"stream {s}"


@pytest.mark.parametrize("rank", [0, 8])
def test_bad_lengths_offsets_and_slots_are_skipped(rank):
    base = small_workload(op="relocate_patch", n_store=4, n_chunks=4, rank=rank, page_size=0)
    vw = VarlenWorkload("bad", base, len_range=(10, 60), len_multiple=1)
    inp = make_varlen_inputs(vw, "cuda", seed=13)
    nt = inp["n_tokens"].clone()
    nt[0] = vw.max_tokens + 1                      # longer than the call's bound
    inp["n_tokens"] = nt
    ro = inp["row_offset"].clone()
    ro[2] = inp["total_rows"] - 1                  # rows past the end of the store
    inp["row_offset"] = ro
    off = inp["dst_offset"].clone()
    off[3] = inp["num_slots"] - 1                  # does not fit the pool
    inp["dst_offset"] = off
    ew = torch.zeros(1, dtype=torch.int32, device="cuda")
    run_varlen(vw, inp, error_word=ew)
    torch.cuda.synchronize()
    assert int(ew.item()) == kam.EW_CHUNK | kam.EW_OFFSET
    check_blocks(vw, inp, [(1, l, s) for l in range(base.num_layers) for s in range(base.num_streams)], "bad")
    # chunk 1 alone was written; every other slot keeps the sentinel
    check_untouched(vw, inp, skip=(0, 2, 3))


def _full_size(name, blocks_wanted, seed):
    vw = varlen_by_name(name)
    _say(f"full size: {vw}")
    inp = make_varlen_inputs(vw, "cuda")
    _say(f"{len(inp['out_ids'])} chunks, {sum(inp['out_lengths'])} tokens, max {vw.max_tokens}")
    ew = torch.zeros(1, dtype=torch.int32, device="cuda")
    run_varlen(vw, inp, error_word=ew)
    torch.cuda.synchronize()
    assert int(ew.item()) == 0
    w = vw.base
    rng = random.Random(seed)
    blocks = {(0, 0, 0), (w.n_chunks - 1, w.num_layers - 1, w.num_streams - 1)}
    while len(blocks) < blocks_wanted:
        blocks.add((rng.randrange(w.n_chunks), rng.randrange(w.num_layers), rng.randrange(w.num_streams)))
    check_blocks(vw, inp, sorted(blocks), f"{name} full size")
    check_untouched(vw, inp)
    del inp
    torch.cuda.empty_cache()


def test_varlen_recall_full_size_sampled():
    # the benchmark's variable-length workload in bench's launch configuration
    _full_size("varlen_recall_rank32", 6, 3)


def test_varlen_survival_full_size_sampled():
    # 9.7 GB of m = 0 rows: the one-vector-per-thread rows kernel
    _full_size("varlen_survival", 6, 4)
